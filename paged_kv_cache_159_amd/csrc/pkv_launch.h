// Host-side launchers of the gfx950 kernels. Arguments are already validated by
// the C ABI layer (pkv_api.hip); these only pick a kernel instance and launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// copy_blocks: 16-byte vectors one workgroup copies (256 threads x 4 = 16 KiB).
constexpr int kCopyVecsPerGroup = 1024;

// Grouped decode: 16-token tiles of the shared prefix per shared-prefix unit
// (128 tokens, streamed through LDS one tile at a time).
constexpr int kSharedChunkTiles = 8;

struct DecodeArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int num_seqs;
  int num_heads;
  int head_dim;
  int max_blocks_per_seq;
  int block_size;       // tokens per block: 8, 16 or 32
  int part_tokens;      // tokens per context partition (decode_partition_tokens)
  int num_parts;        // partial slots per (sequence, head) in the workspace layout
  int tail_parts;       // partitions per sequence the partition launch covers
  int slot_base;        // first slot of those partitions (grouped call: after the shared chunks)
  const int32_t* group_start;    // grouped call only (else nullptr): [num_groups + 1]
  const int32_t* shared_blocks;  // grouped call only: [num_groups]
  int num_groups;
  float scale;
  int dtype;            // 0 fp16, 1 bf16
  float* ws_ml;         // [num_seqs][num_heads][num_parts][2] (running max, exp sum), log2 domain
  float* ws_o;          // [num_seqs][num_heads][num_parts][head_dim] normalised partial outputs
  int32_t* ws_seq;      // grouped call: [num_seqs] shared-prefix tokens of each sequence,
                        // written by the main launch, read by the merge
  uint32_t* flags;      // plain call with a planned item order: claim flags of the
                        // backed-up items, [backup_items][head groups]
  int backup_items;
};

// Tokens per context partition for these sizes (256 or 512): 512 for tables
// of more than 4096 tokens or grids of kLargeGridSlots or more 256-token
// (sequence, partition, head group) slots.
constexpr int64_t kLargeGridSlots = 8192;
int decode_partition_tokens(int num_seqs, int num_heads, int head_dim, int max_blocks_per_seq,
                            int block_size);

// Workspace layout shared by the two decode launches.
size_t decode_workspace_bytes(int num_seqs, int num_heads, int head_dim, int num_parts);
void decode_workspace_split(void* ws, int num_seqs, int num_heads, int num_parts, float** ml,
                            float** o);

hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);
// Grouped call, main launch: shared-prefix units and tail partitions in one
// grid (the merge follows with launch_decode_merge).
hipError_t launch_decode_grouped(const DecodeArgs& a, hipStream_t stream);

// Prefill / chunked-prefill attention (MFMA): one launch.
struct PrefillArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;   // [num_seqs + 1] packed query rows per sequence
  int num_seqs;
  int num_heads;
  int head_dim;
  int max_blocks_per_seq;
  int block_size;
  int max_query_len;            // bound on query_start[s+1] - query_start[s]
  float scale;
  int dtype;
};
// Chunk rows one prefill workgroup covers (the grid has ceil(max_query_len /
// rows) tiles per sequence and head).
int prefill_rows_per_tile();
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* key_cache,
                                    void* value_cache, const int64_t* slot_mapping, int num_tokens,
                                    int row_elems, hipStream_t stream);

// Block copy from (src_key, src_value) to (dst_key, dst_value): the same pools
// for copy_blocks, a device pool and a pinned host pool for swap_blocks
// (system_release: end with a system-scope release for the host side).
hipError_t launch_copy_blocks(const void* src_key, const void* src_value, void* dst_key,
                              void* dst_value, const int32_t* block_mapping, int num_pairs,
                              int64_t block_elems, bool system_release, hipStream_t stream);

// Destination block ids of one scatter launch (swap_blocks_staged), passed
// by value in the kernel arguments: 896 ids keep the arguments under 4 KiB.
constexpr int kScatterIds = 896;
struct ScatterIds {
  int32_t dst[kScatterIds];
};

// Copies staging slots slot0 .. slot0 + num_pairs - 1 of (src_key, src_value)
// to blocks ids.dst[0 .. num_pairs) of (dst_key, dst_value); num_pairs <=
// kScatterIds.
hipError_t launch_scatter_blocks(const void* src_key, const void* src_value, void* dst_key,
                                 void* dst_value, const ScatterIds& ids, int num_pairs, int slot0,
                                 int64_t block_elems, bool system_release, hipStream_t stream);

}  // namespace pkv
