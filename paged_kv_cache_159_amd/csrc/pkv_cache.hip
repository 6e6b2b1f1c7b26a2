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
//
// swap_blocks [P1 §3.3.3 "显存不足时的处理策略", CPU Swap: a swapped-out
// sequence's blocks are copied page by page to pre-allocated host buffers and
// its device blocks freed; swapping in copies them back into newly allocated
// device blocks; P2 "vLLM高性能推理架构的工程落地考量": swap is bound by the
// host link]: the same block copy between two pools, one of which is pinned
// host memory that the kernel reads or writes directly over the host link.
// One launch moves every listed block (no per-block DMA command). The kernel
// ends with a system-scope release so that its writes to host memory are
// visible to the host once the stream has been synchronised.

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
  // Non-temporal stores: the rows stream to HBM instead of sitting dirty in
  // the caches, where their write-back slowed the decode that follows (by
  // ~18 us after a 567 MB write in the shared-prefix step on MI355X).
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  for (int i = threadIdx.x; i < row_vecs; i += kCacheThreads) {
    const uint4 k = ks[i];
    const uint4 v = vs[i];
    __builtin_nontemporal_store(__builtin_bit_cast(u4v, k), reinterpret_cast<u4v*>(kd + i));
    __builtin_nontemporal_store(__builtin_bit_cast(u4v, v), reinterpret_cast<u4v*>(vd + i));
  }
}

// One workgroup's 16 KiB piece g of a block copy from sp to dp (block_vecs
// 16-byte vectors per block).
__device__ __forceinline__ void copy_block_piece(const uint4* __restrict__ sp, uint4* __restrict__ dp,
                                                 int64_t block_vecs, int g) {
  const int64_t first = (int64_t)g * kCopyVecsPerGroup + threadIdx.x;
  // Loads are unconditional (indices past the block re-read its last vector)
  // and all four are issued before the stores, so they are in flight at once.
  static_assert(kCopyVecsPerThread == 4, "four named vectors below");
  const int64_t e0 = first, e1 = first + kCacheThreads, e2 = first + 2 * kCacheThreads,
                e3 = first + 3 * kCacheThreads;
  const int64_t last = block_vecs - 1;
  const uint4 v0 = sp[e0 < block_vecs ? e0 : last];
  const uint4 v1 = sp[e1 < block_vecs ? e1 : last];
  const uint4 v2 = sp[e2 < block_vecs ? e2 : last];
  const uint4 v3 = sp[e3 < block_vecs ? e3 : last];
  __builtin_amdgcn_sched_barrier(0);
  if (e0 < block_vecs) dp[e0] = v0;
  if (e1 < block_vecs) dp[e1] = v1;
  if (e2 < block_vecs) dp[e2] = v2;
  if (e3 < block_vecs) dp[e3] = v3;
}

template <bool SYSTEM_RELEASE>
__global__ void __launch_bounds__(kCacheThreads)
copy_blocks_kernel(const uint4* __restrict__ src_key, const uint4* __restrict__ src_value,
                   uint4* __restrict__ dst_key, uint4* __restrict__ dst_value,
                   const int32_t* __restrict__ block_mapping, int64_t block_vecs,
                   int groups_per_block) {
  const int g = blockIdx.x % groups_per_block;
  const int pool = (blockIdx.x / groups_per_block) & 1;
  const int pair = blockIdx.x / (2 * groups_per_block);
  const int64_t src = block_mapping[2 * pair];
  const int64_t dst = block_mapping[2 * pair + 1];
  copy_block_piece((pool ? src_value : src_key) + src * block_vecs,
                   (pool ? dst_value : dst_key) + dst * block_vecs, block_vecs, g);
  if constexpr (SYSTEM_RELEASE) __threadfence_system();
}

// Scatter of consecutive staging slots to listed destination blocks: pair i
// copies slot slot0 + i to block ids.dst[i]. The ids travel in the kernel's
// arguments, which the launch copies, so no host buffer has to outlive the
// enqueue (and a captured launch replays with the same ids).
template <bool SYSTEM_RELEASE>
__global__ void __launch_bounds__(kCacheThreads)
scatter_blocks_kernel(const uint4* __restrict__ src_key, const uint4* __restrict__ src_value,
                      uint4* __restrict__ dst_key, uint4* __restrict__ dst_value, ScatterIds ids,
                      int slot0, int64_t block_vecs, int groups_per_block) {
  const int g = blockIdx.x % groups_per_block;
  const int pool = (blockIdx.x / groups_per_block) & 1;
  const int pair = blockIdx.x / (2 * groups_per_block);
  const int64_t src = slot0 + pair;
  const int64_t dst = ids.dst[pair];
  copy_block_piece((pool ? src_value : src_key) + src * block_vecs,
                   (pool ? dst_value : dst_key) + dst * block_vecs, block_vecs, g);
  if constexpr (SYSTEM_RELEASE) __threadfence_system();
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

hipError_t launch_copy_blocks(const void* src_key, const void* src_value, void* dst_key,
                              void* dst_value, const int32_t* block_mapping, int num_pairs,
                              int64_t block_elems, bool system_release, hipStream_t stream) {
  const int64_t block_vecs = block_elems / 8;
  const int groups = (int)((block_vecs + kCopyVecsPerGroup - 1) / kCopyVecsPerGroup);
  const unsigned grid = (unsigned)num_pairs * 2u * (unsigned)groups;
  auto* sk = static_cast<const uint4*>(src_key);
  auto* sv = static_cast<const uint4*>(src_value);
  auto* dk = static_cast<uint4*>(dst_key);
  auto* dv = static_cast<uint4*>(dst_value);
  if (system_release)
    hipLaunchKernelGGL(copy_blocks_kernel<true>, dim3(grid), dim3(kCacheThreads), 0, stream, sk,
                       sv, dk, dv, block_mapping, block_vecs, groups);
  else
    hipLaunchKernelGGL(copy_blocks_kernel<false>, dim3(grid), dim3(kCacheThreads), 0, stream, sk,
                       sv, dk, dv, block_mapping, block_vecs, groups);
  return hipGetLastError();
}

hipError_t launch_scatter_blocks(const void* src_key, const void* src_value, void* dst_key,
                                 void* dst_value, const ScatterIds& ids, int num_pairs, int slot0,
                                 int64_t block_elems, bool system_release, hipStream_t stream) {
  const int64_t block_vecs = block_elems / 8;
  const int groups = (int)((block_vecs + kCopyVecsPerGroup - 1) / kCopyVecsPerGroup);
  const unsigned grid = (unsigned)num_pairs * 2u * (unsigned)groups;
  auto* sk = static_cast<const uint4*>(src_key);
  auto* sv = static_cast<const uint4*>(src_value);
  auto* dk = static_cast<uint4*>(dst_key);
  auto* dv = static_cast<uint4*>(dst_value);
  if (system_release)
    hipLaunchKernelGGL(scatter_blocks_kernel<true>, dim3(grid), dim3(kCacheThreads), 0, stream, sk,
                       sv, dk, dv, ids, slot0, block_vecs, groups);
  else
    hipLaunchKernelGGL(scatter_blocks_kernel<false>, dim3(grid), dim3(kCacheThreads), 0, stream,
                       sk, sv, dk, dv, ids, slot0, block_vecs, groups);
  return hipGetLastError();
}

}  // namespace pkv
