// Device checks of the data-dependent preconditions that the C ABI leaves to
// the caller (block-table entries, context lengths, group and chunk layouts,
// slots, copy pairs). They run only when the environment variable
// PAGED_KV_DEBUG is "1", on the call's stream before its main launches; the
// call then waits for them and returns PKV_ERR_DATA instead of launching when
// one fails. Every check reads only inside the arrays' stated sizes, so it is
// safe on the bad inputs it is meant to catch.

#include <stdlib.h>
#include <string.h>

#include "pkv_debug.h"

namespace pkv {

// Bits of DebugFlag, OR-ed by the check kernels of the current call.
__device__ unsigned g_debug_status;

namespace {

constexpr int kDebugThreads = 256;

__device__ __forceinline__ void flag(unsigned bit) { atomicOr(&g_debug_status, bit); }

__global__ void debug_reset_kernel() {
  if (threadIdx.x == 0) g_debug_status = 0u;
}

// One thread per table entry (s, j): context length of s in
// [min_ctx, max_blocks * block_size]; entries j < ceil(ctx / block_size) in
// [0, num_blocks).
__global__ void check_tables_kernel(const int32_t* block_tables, const int32_t* context_lens,
                                    int num_seqs, int max_blocks, int block_size, int num_blocks,
                                    int min_ctx) {
  const int64_t n = (int64_t)num_seqs * max_blocks;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int s = (int)(i / max_blocks);
    const int j = (int)(i % max_blocks);
    const int ctx = context_lens[s];
    if (j == 0 && (ctx < min_ctx || (int64_t)ctx > (int64_t)max_blocks * block_size))
      flag(kDebugContext);
    const int64_t used = ctx > 0 ? ((int64_t)ctx + block_size - 1) / block_size : 0;
    if (j < used) {
      const int32_t id = block_tables[i];
      if (id < 0 || id >= num_blocks) flag(kDebugTable);
    }
  }
}

// Groups of the grouped decode. Thread 0 checks group_start itself (0 first,
// nondecreasing, num_seqs last); the thread of sequence s finds its group g
// (group_start[g] <= s < group_start[g + 1]) and checks that the group's
// shared blocks are full blocks of s's context and that s's first
// shared_blocks[g] table entries equal the group's first member's.
__global__ void check_groups_kernel(const int32_t* group_start, const int32_t* shared_blocks,
                                    int num_groups, int num_seqs, const int32_t* block_tables,
                                    const int32_t* context_lens, int max_blocks, int block_size) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t == 0) {
    if (group_start[0] != 0 || group_start[num_groups] != num_seqs) flag(kDebugGroup);
    for (int g = 0; g < num_groups; ++g)
      if (group_start[g] > group_start[g + 1]) flag(kDebugGroup);
  }
  for (int s = t; s < num_seqs; s += gridDim.x * blockDim.x) {
    int g = -1;
    for (int k = 0; k < num_groups; ++k)
      if (group_start[k] <= s && s < group_start[k + 1]) g = k;
    if (g < 0) {
      flag(kDebugGroup);
      continue;
    }
    const int sb = shared_blocks[g];
    const int s0 = group_start[g];            // 0 <= s0 <= s once g was found
    if (sb < 0 || sb > max_blocks || (int64_t)sb * block_size > context_lens[s] || s0 < 0) {
      flag(kDebugGroup);
      continue;
    }
    const int32_t* row = block_tables + (int64_t)s * max_blocks;
    const int32_t* first = block_tables + (int64_t)s0 * max_blocks;
    for (int j = 0; j < sb; ++j)
      if (row[j] != first[j]) {
        flag(kDebugGroup);
        break;
      }
  }
}

// Chunks of the prefill call: query_start[0] = 0 and, per sequence,
// 0 <= q_len <= min(max_query_len, context_lens[s]).
__global__ void check_prefill_kernel(const int32_t* query_start, const int32_t* context_lens,
                                     int num_seqs, int max_query_len) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t == 0 && query_start[0] != 0) flag(kDebugQuery);
  for (int s = t; s < num_seqs; s += gridDim.x * blockDim.x) {
    const int q_len = query_start[s + 1] - query_start[s];
    if (q_len < 0 || q_len > max_query_len || q_len > context_lens[s]) flag(kDebugQuery);
  }
}

// Slots of the cache write: < num_slots (negative ones are padding), and no
// slot written twice (each thread compares its slot with the later ones).
__global__ void check_slots_kernel(const int64_t* slot_mapping, int num_tokens,
                                   int64_t num_slots) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < num_tokens;
       i += gridDim.x * blockDim.x) {
    const int64_t v = slot_mapping[i];
    if (v < 0) continue;
    if (v >= num_slots) flag(kDebugSlot);
    for (int k = i + 1; k < num_tokens; ++k)
      if (slot_mapping[k] == v) {
        flag(kDebugSlotDup);
        break;
      }
  }
}

// Block pairs (src, dst): src < src_blocks, dst < dst_blocks, no destination
// twice and, within one pool, no destination that is also a source.
__global__ void check_pairs_kernel(const int32_t* pairs, int num_pairs, int src_blocks,
                                   int dst_blocks, int same_pool) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < num_pairs;
       i += gridDim.x * blockDim.x) {
    const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) flag(kDebugPair);
    for (int k = 0; k < num_pairs; ++k) {
      if (k > i && pairs[2 * k + 1] == dst) flag(kDebugPairDup);
      if (same_pool && pairs[2 * k] == dst) flag(kDebugPairDup);
    }
  }
}

unsigned grid_for(int64_t n) {
  const int64_t g = (n + kDebugThreads - 1) / kDebugThreads;
  return (unsigned)(g < 1 ? 1 : (g > 4096 ? 4096 : g));
}

}  // namespace

bool debug_enabled() {
  const char* v = getenv("PAGED_KV_DEBUG");
  return v != nullptr && strcmp(v, "1") == 0;
}

hipError_t debug_reset(hipStream_t st) {
  hipLaunchKernelGGL(debug_reset_kernel, dim3(1), dim3(64), 0, st);
  return hipGetLastError();
}

hipError_t debug_check_tables(const int32_t* block_tables, const int32_t* context_lens,
                              int num_seqs, int max_blocks, int block_size, int num_blocks,
                              int min_ctx, hipStream_t st) {
  hipLaunchKernelGGL(check_tables_kernel, dim3(grid_for((int64_t)num_seqs * max_blocks)),
                     dim3(kDebugThreads), 0, st, block_tables, context_lens, num_seqs, max_blocks,
                     block_size, num_blocks, min_ctx);
  return hipGetLastError();
}

hipError_t debug_check_groups(const int32_t* group_start, const int32_t* shared_blocks,
                              int num_groups, int num_seqs, const int32_t* block_tables,
                              const int32_t* context_lens, int max_blocks, int block_size,
                              hipStream_t st) {
  hipLaunchKernelGGL(check_groups_kernel, dim3(grid_for(num_seqs)), dim3(kDebugThreads), 0, st,
                     group_start, shared_blocks, num_groups, num_seqs, block_tables, context_lens,
                     max_blocks, block_size);
  return hipGetLastError();
}

hipError_t debug_check_prefill(const int32_t* query_start, const int32_t* context_lens,
                               int num_seqs, int max_query_len, hipStream_t st) {
  hipLaunchKernelGGL(check_prefill_kernel, dim3(grid_for(num_seqs)), dim3(kDebugThreads), 0, st,
                     query_start, context_lens, num_seqs, max_query_len);
  return hipGetLastError();
}

hipError_t debug_check_slots(const int64_t* slot_mapping, int num_tokens, int64_t num_slots,
                             hipStream_t st) {
  hipLaunchKernelGGL(check_slots_kernel, dim3(grid_for(num_tokens)), dim3(kDebugThreads), 0, st,
                     slot_mapping, num_tokens, num_slots);
  return hipGetLastError();
}

hipError_t debug_check_pairs(const int32_t* pairs, int num_pairs, int src_blocks, int dst_blocks,
                             bool same_pool, hipStream_t st) {
  hipLaunchKernelGGL(check_pairs_kernel, dim3(grid_for(num_pairs)), dim3(kDebugThreads), 0, st,
                     pairs, num_pairs, src_blocks, dst_blocks, same_pool ? 1 : 0);
  return hipGetLastError();
}

hipError_t debug_status(hipStream_t st, unsigned* status) {
  *status = 0u;
  hipError_t e = hipMemcpyFromSymbolAsync(status, HIP_SYMBOL(g_debug_status), sizeof(unsigned), 0,
                                          hipMemcpyDeviceToHost, st);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(st);
}

}  // namespace pkv
