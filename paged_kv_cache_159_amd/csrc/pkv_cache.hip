// Cache write and block copy for gfx950: pure data movement in 16-byte
// vectors, bit-exact.
//
// reshape_and_cache [P2 "Copy-on-Write共享解码的显存优化原理": the new token's
// K/V goes into its block; P3 §3.1.3 address formula]: with the pool laid out
// [block][offset][head][dim], slot = block*block_size + offset starts at
// element slot*kv_dim, so a token's whole K row (kv_dim elements) is one
// contiguous run and the write is a row copy. One workgroup per token.
//
// copy_blocks [P2 "Python 演示" copy_on_write; P3 §3.1.5 "CoW机制的实现"]: each
// (src, dst) pair copies block_size*kv_dim elements of K and of V. A block of
// the LLaMA-7B shape is 128 KiB per pool, so it is split over workgroups of
// 16 KiB each; every thread issues its four 16-byte loads before its stores.

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kCacheThreads = 256;
constexpr int kCopyVecsPerThread = 4;
static_assert(kCopyVecsPerGroup == kCacheThreads * kCopyVecsPerThread, "copy group size");

__global__ void __launch_bounds__(kCacheThreads)
reshape_and_cache_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                         uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
                         const int64_t* __restrict__ slot_mapping, int row_vecs) {
  const int t = blockIdx.x;
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;  // padding token
  const uint4* ks = key + (size_t)t * row_vecs;
  const uint4* vs = value + (size_t)t * row_vecs;
  uint4* kd = key_cache + (size_t)slot * row_vecs;
  uint4* vd = value_cache + (size_t)slot * row_vecs;
  for (int i = threadIdx.x; i < row_vecs; i += kCacheThreads) {
    const uint4 k = ks[i];
    const uint4 v = vs[i];
    kd[i] = k;
    vd[i] = v;
  }
}

__global__ void __launch_bounds__(kCacheThreads)
copy_blocks_kernel(uint4* __restrict__ key_cache, uint4* __restrict__ value_cache,
                   const int32_t* __restrict__ block_mapping, int64_t block_vecs,
                   int groups_per_block) {
  const int g = blockIdx.x % groups_per_block;
  const int pool = (blockIdx.x / groups_per_block) & 1;
  const int pair = blockIdx.x / (2 * groups_per_block);
  const int64_t src = block_mapping[2 * pair];
  const int64_t dst = block_mapping[2 * pair + 1];
  uint4* base = pool ? value_cache : key_cache;
  const uint4* sp = base + src * block_vecs;
  uint4* dp = base + dst * block_vecs;
  const int64_t first = (int64_t)g * kCopyVecsPerGroup + threadIdx.x;
  uint4 v[kCopyVecsPerThread];
#pragma unroll
  for (int i = 0; i < kCopyVecsPerThread; ++i) {
    const int64_t e = first + (int64_t)i * kCacheThreads;
    if (e < block_vecs) v[i] = sp[e];
  }
#pragma unroll
  for (int i = 0; i < kCopyVecsPerThread; ++i) {
    const int64_t e = first + (int64_t)i * kCacheThreads;
    if (e < block_vecs) dp[e] = v[i];
  }
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int64_t* slot_mapping, int num_tokens,
                                    int row_elems, hipStream_t stream) {
  const int row_vecs = row_elems / 8;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(kCacheThreads), 0, stream,
                     static_cast<const uint4*>(key), static_cast<const uint4*>(value),
                     static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache),
                     slot_mapping, row_vecs);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* key_cache, void* value_cache, const int32_t* block_mapping,
                              int num_pairs, int64_t block_elems, hipStream_t stream) {
  const int64_t block_vecs = block_elems / 8;
  const int groups = (int)((block_vecs + kCopyVecsPerGroup - 1) / kCopyVecsPerGroup);
  const unsigned grid = (unsigned)num_pairs * 2u * (unsigned)groups;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(grid), dim3(kCacheThreads), 0, stream,
                     static_cast<uint4*>(key_cache), static_cast<uint4*>(value_cache),
                     block_mapping, block_vecs, groups);
  return hipGetLastError();
}

}  // namespace pkv
