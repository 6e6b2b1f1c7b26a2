// Optional device checks of the callers' data-dependent preconditions
// (PAGED_KV_DEBUG=1); see pkv_debug.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Bits of the status the checks report.
enum DebugFlag : unsigned {
  kDebugContext = 1u,    // a context length outside its allowed range
  kDebugTable = 2u,      // a block-table entry that is read lies outside [0, num_blocks)
  kDebugGroup = 4u,      // group_start / shared_blocks break the grouped call's constraints
  kDebugQuery = 8u,      // query_start / chunk lengths break the prefill call's constraints
  kDebugSlot = 16u,      // a slot at or past num_blocks * block_size
  kDebugSlotDup = 32u,   // a slot written twice in one call
  kDebugPair = 64u,      // a block id of a copy pair out of range
  kDebugPairDup = 128u,  // a destination twice, or a destination that is also a source
};

// True when the environment variable PAGED_KV_DEBUG is "1" (read at each call).
bool debug_enabled();

// Clears the status; the checks below OR their findings into it.
hipError_t debug_reset(hipStream_t st);
hipError_t debug_check_tables(const int32_t* block_tables, const int32_t* context_lens,
                              int num_seqs, int max_blocks, int block_size, int num_blocks,
                              int min_ctx, hipStream_t st);
hipError_t debug_check_groups(const int32_t* group_start, const int32_t* shared_blocks,
                              int num_groups, int num_seqs, const int32_t* block_tables,
                              const int32_t* context_lens, int max_blocks, int block_size,
                              hipStream_t st);
hipError_t debug_check_prefill(const int32_t* query_start, const int32_t* context_lens,
                               int num_seqs, int max_query_len, hipStream_t st);
hipError_t debug_check_slots(const int64_t* slot_mapping, int num_tokens, int64_t num_slots,
                             hipStream_t st);
hipError_t debug_check_pairs(const int32_t* pairs, int num_pairs, int src_blocks, int dst_blocks,
                             bool same_pool, hipStream_t st);
// Waits for the stream and returns the status bits of the checks since the
// last debug_reset.
hipError_t debug_status(hipStream_t st, unsigned* status);

}  // namespace pkv
