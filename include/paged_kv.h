/*
 * paged_kv.h — C ABI of libpaged_kv.so: paged KV-cache decode attention, the
 * slot-mapped cache write and the copy-on-write block copy, for AMD Instinct
 * MI355X (gfx950).
 *
 * Pages cited:
 *   [P1] "3.3 页面级显存管理" (page-level GPU memory management), aiknowledge.cn/article/68056
 *   [P2] "vLLM三大核心技术分页内存与共享解码", aiqz.cc/article/vllm-core-techniques.html
 *   [P3] "3.1 PagedAttention的核心原理", aiknowledge.cn/article/68054
 *   [P4] reading notes on "vLLM: Easy, Fast, and Cheap LLM Serving with PagedAttention",
 *        zmoe.com/3008.html
 *
 * Common conventions
 * ------------------
 * Element types: PKV_F16 (IEEE binary16) or PKV_BF16 (bfloat16). Every 16-bit
 * tensor of one call has the same type.
 *
 * Layouts (all row-major and dense; every pointer 16-byte aligned):
 *   key_cache, value_cache  [num_blocks][block_size][num_heads][head_dim]
 *       One physical block ("page") holds block_size consecutive tokens; one
 *       token holds num_heads*head_dim elements (kv_dim). The element of token
 *       t of a sequence is at physical*block_size*kv_dim + (t % block_size)*kv_dim
 *       with physical = block_table[t / block_size] [P3 §3.1.3 "逻辑地址到物理地址
 *       的转换"; P3 §3.1.2 "页面结构设计" gives separate Key and Value caches].
 *   query, out              [num_seqs][num_heads][head_dim]
 *   block_tables            int32 [num_seqs][max_blocks_per_seq], one flattened
 *       table per sequence [P3 §3.1.3: a flat block_table array]; entries at
 *       and past ceil(context_len / block_size) are never read.
 *   context_lens            int32 [num_seqs]
 *   slot_mapping            int64 [num_tokens]; slot = physical*block_size + offset
 *   block_mapping           int32 [num_pairs][2] = (src, dst)
 *
 * Supported: block_size 8, 16 or 32 (16 is the pages' default; larger blocks
 * mean fewer table entries and lookups, smaller ones less waste in a
 * sequence's last block: P2 "KV Cache逻辑块物理块映射机制" and "vLLM高性能推理
 * 架构的工程落地考量"; P4 "PagedAttention: 页式管理内存"; P1 §3.3.5
 * "自动调优策略"), head_dim 64 or 128, any num_heads >= 1. Any other block
 * size or head_dim returns PKV_ERR_UNSUPPORTED.
 *
 * Ownership: the caller owns every buffer (pools, query, out, tables,
 * workspace). The library allocates and frees nothing and keeps no state
 * between calls. All pointers except `stream` are device pointers.
 *
 * Execution: every call validates its scalar arguments and pointers on the
 * host, then enqueues kernels on `stream` (a hipStream_t; NULL is the default
 * stream) and returns without synchronising. A launch failure reported by
 * hipGetLastError becomes PKV_ERR_LAUNCH. Nothing is thrown across the ABI.
 *
 * Data-dependent preconditions are the caller's (checking them would need a
 * device synchronisation): block-table entries that are read lie in
 * [0, num_blocks); 1 <= context_lens[s] <= max_blocks_per_seq*block_size;
 * slots are < num_blocks*block_size and unique within a call; copy pairs have
 * unique destinations that are not sources in the same call; for the grouped
 * call, the group constraints stated at paged_attention_decode_grouped.
 *
 * Debug checks: with the environment variable PAGED_KV_DEBUG set to "1" (read
 * at every call), the decode, grouped decode, prefill, cache-write,
 * block-copy and swap_blocks calls first check those preconditions with
 * device kernels on `stream`, wait for them (so the call synchronises), and
 * return PKV_ERR_DATA without launching anything else if one fails. The
 * checks read only within the arrays' stated sizes. paged_attention_decode_merge
 * is not checked; swap_blocks_dma and swap_blocks_staged check their host
 * mappings always.
 */
#ifndef PAGED_KV_H
#define PAGED_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F16 = 0, PKV_BF16 = 1 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = -2,       /* a count is out of range or sizes overflow */
  PKV_ERR_UNSUPPORTED = -3, /* dtype, block_size or head_dim not supported */
  PKV_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required */
  PKV_ERR_LAUNCH = -5,      /* the HIP runtime rejected a kernel launch */
  PKV_ERR_ALIGN = -6,       /* a pointer is not 16-byte aligned */
  PKV_ERR_MEMORY = -7,      /* swap_blocks: a buffer is not device memory of the current
                               device or pinned host memory, or is smaller than its sizes */
  PKV_ERR_DATA = -8,        /* PAGED_KV_DEBUG=1 only: a data-dependent precondition does not
                               hold; nothing was launched */
  PKV_ERR_SCRATCH = -9      /* paged_attention_decode_noalloc: the call needs more than
                               PKV_NOALLOC_SCRATCH_BYTES of scratch */
} pkv_status;

/* Bytes of the fixed per-device scratch array of paged_attention_decode_noalloc. */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Library version, major*10000 + minor*100 + patch. */
int pkv_version(void);

/* Static text for a status code (never NULL). */
const char* pkv_status_string(int status);

/*
 * Workspace bytes paged_attention_decode needs for these sizes: fp32 partial
 * results (running max, exponent sum and a head_dim vector) of every context
 * partition of every (sequence, head). A partition is 512 tokens when
 * max_blocks_per_seq*block_size > 4096, or when num_seqs * ceil(num_heads /
 * G) * ceil(max_blocks_per_seq*block_size / 256) >= 8192 (G = 4 heads at
 * head_dim 128, 8 at 64: the heads one workgroup covers), else 256 tokens.
 * With 512-token partitions, at most 256 sequences and at most 65,536
 * (sequence, partition) slots, the workspace also holds one 32-bit claim flag
 * per (backed-up item, head group): the last quarter of the launch's work
 * items get a second workgroup on another XCD, and the flag lets exactly one
 * of the two compute the item (at the first 256-byte boundary after the
 * partials; ceil(num_seqs * partitions / 4) * ceil(num_heads / G) flags). Returns 0
 * when no sequence can span more than one partition or when the arguments
 * are invalid.
 */
size_t paged_attention_workspace_size(int num_seqs, int num_heads, int head_dim,
                                      int max_blocks_per_seq, int block_size);

/*
 * Single-query decode attention over the paged cache [P3 §3.1.3 translation;
 * P1 §3.3.1 "显存访问模式的优化": work organised by physical block, all
 * sequences in one launch]. For every sequence s and head h:
 *     x_t = scale * <query[s][h], K_t>  for tokens t in [0, context_lens[s])
 *     out[s][h] = sum_t softmax(x)_t * V_t
 * where K_t and V_t are token t's rows of head h, found through block_tables[s].
 * Accumulation is fp32; the output is rounded to nearest-even into `dtype`.
 * Contexts are split into partitions of 256 or 512 tokens (the rule at
 * paged_attention_workspace_size) whose partial results are merged by
 * log-sum-exp; the reduction order depends only
 * on logical token positions, so relabelling physical blocks leaves `out`
 * bit-identical.
 * `workspace` (>= paged_attention_workspace_size(...) bytes) may be NULL
 * when that size is 0. Any content gives the correct result. Claim flags that
 * start at zero are left at zero, so zeroing the workspace once when it is
 * allocated lets the first of an item's two workgroups compute it in every
 * call (from other values the second one does). Calls that
 * share a workspace must be ordered (one stream). num_seqs == 0 is a no-op
 * (pointers may then be NULL).
 * Equivalent to paged_attention_decode_partitions followed by
 * paged_attention_decode_merge on the same stream.
 */
int paged_attention_decode(void* out, const void* query,
                           const void* key_cache, const void* value_cache,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int num_seqs, int num_heads, int head_dim, int num_blocks,
                           int block_size, int max_blocks_per_seq, float scale, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments and result as paged_attention_decode (the same kernels, so the
 * output is bit-identical), without a workspace: the split-K partials go to
 * a fixed device array of PKV_NOALLOC_SCRATCH_BYTES (64 MiB) that the library
 * holds on each GPU it runs on until the process ends. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine). A call whose
 * partials need more than that (paged_attention_workspace_size(...) >
 * PKV_NOALLOC_SCRATCH_BYTES) returns PKV_ERR_SCRATCH before touching the
 * device. Every call on one GPU shares that GPU's array and leaves its
 * partials in it; nothing in it must start at zero (the claim flags give the
 * correct result from any content). Calls that overlap on one
 * GPU (on different streams, or from several threads without ordering) race
 * on the array and may return wrong results: order them on one stream.
 */
int paged_attention_decode_noalloc(void* out, const void* query,
                                   const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   int num_seqs, int num_heads, int head_dim, int num_blocks,
                                   int block_size, int max_blocks_per_seq, float scale,
                                   int dtype, void* stream);

/*
 * First of the two launches of paged_attention_decode: one workgroup per
 * (sequence, context partition, group of heads). Sequences whose context fits one
 * partition get their final `out` here; the others leave partials in
 * `workspace`. Exposed so that callers can schedule or time the two launches
 * separately; the arguments mean the same as for paged_attention_decode.
 */
int paged_attention_decode_partitions(void* out, const void* query,
                                      const void* key_cache, const void* value_cache,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      int num_seqs, int num_heads, int head_dim, int num_blocks,
                                      int block_size, int max_blocks_per_seq, float scale,
                                      int dtype, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Second launch: log-sum-exp merge of the partials left by
 * paged_attention_decode_partitions for sequences longer than one partition,
 * writing their `out`. Must follow that call on the same stream, with the
 * same out, context_lens, sizes and workspace. Does nothing (and launches
 * nothing) when max_blocks_per_seq*block_size <= 256.
 */
int paged_attention_decode_merge(void* out, const int32_t* context_lens,
                                 int num_seqs, int num_heads, int head_dim,
                                 int block_size, int max_blocks_per_seq, int dtype,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes paged_attention_decode_grouped needs: fp32 partials of every
 * shared-prefix chunk (128 tokens) and every tail partition (512 tokens) of
 * every (sequence, head), then one int32 per sequence. Returns 0 when the arguments
 * are invalid.
 */
size_t paged_attention_grouped_workspace_size(int num_seqs, int num_heads, int head_dim,
                                              int max_blocks_per_seq, int block_size);

/*
 * Decode attention for sequences that share prefix blocks, e.g. the samples of
 * one prompt in parallel sampling or the beams of a beam search [P2 "Copy-on-
 * Write共享解码的显存优化原理": sequences with a common prefix map it to the same
 * physical blocks; P4 "Memory Sharing与写时复制"]. Same result as
 * paged_attention_decode (within rounding; the summation order differs), but
 * each shared block is read once per group and its attention for all the
 * group's queries runs on the MFMA matrix cores.
 *   group_start    int32 [num_groups + 1], device: group g is sequences
 *                  [group_start[g], group_start[g+1]); group_start[0] = 0,
 *                  nondecreasing, group_start[num_groups] = num_seqs.
 *   shared_blocks  int32 [num_groups], device: the first shared_blocks[g]
 *                  block-table entries are identical for every member of
 *                  group g and are full blocks of every member's context
 *                  (shared_blocks[g] * block_size <= context_lens[s]).
 * Groups of any size are allowed (queries are processed 16 at a time). The
 * MFMA units cover the shared tokens rounded down to a multiple of 16 (at
 * block_size 8 an odd last shared block goes with the tails); a group with
 * shared_blocks 0 runs entirely on the tail partitions.
 * Two launches on `stream`: shared-prefix chunks and tail partitions in one
 * grid, then the merge.
 * `workspace` needs paged_attention_grouped_workspace_size(...) bytes.
 */
int paged_attention_decode_grouped(void* out, const void* query,
                                   const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   const int32_t* group_start, const int32_t* shared_blocks,
                                   int num_groups, int num_seqs, int num_heads, int head_dim,
                                   int num_blocks, int block_size, int max_blocks_per_seq,
                                   float scale, int dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Multi-token (prefill / chunked-prefill) attention over the paged cache, on
 * the MFMA matrix cores [P1 §3.3.2 "动态页面分配机制": a prompt's pages are
 * allocated in one go at prefill; P3 §3.1.3: the same address translation as
 * decode]. The pages give no formula; the reading is causal scaled
 * dot-product attention. Sequence s's query rows are
 * query[query_start[s] .. query_start[s+1]) ([rows][num_heads][head_dim], the
 * same layout for `out`): its last q_len = query_start[s+1] - query_start[s]
 * tokens, at positions context_lens[s] - q_len .. context_lens[s] - 1, whose
 * K/V must already be in the cache (reshape_and_cache first). Query i attends
 * over tokens 0 .. context_lens[s] - q_len + i of its sequence. q_len =
 * context_lens[s] is a whole prompt, a smaller q_len a chunk after a cached
 * prefix, q_len = 0 skips the sequence.
 *   query_start  int32 [num_seqs + 1], device: 0, nondecreasing; the rows of
 *                query and out are query_start[num_seqs].
 *   max_query_len  host bound on every q_len (sizes the grid; rows of a longer
 *                chunk beyond it are not computed). <= max_blocks_per_seq *
 *                block_size.
 * Preconditions as for decode, plus q_len <= context_lens[s]. No workspace;
 * one launch on `stream`; output rounded to nearest even from fp32.
 */
int paged_attention_prefill(void* out, const void* query, const void* key_cache,
                            const void* value_cache, const int32_t* block_tables,
                            const int32_t* context_lens, const int32_t* query_start,
                            int num_seqs, int max_query_len, int num_heads, int head_dim,
                            int num_blocks, int block_size, int max_blocks_per_seq, float scale,
                            int dtype, void* stream);

/*
 * Slot-mapped cache write [P2 "Copy-on-Write共享解码的显存优化原理": the new
 * token's K/V is written into its block; P1 §3.3.2 "动态页面分配机制"]. For each
 * token i with slot_mapping[i] >= 0:
 *     key_cache[slot / block_size][slot % block_size] = key[i]   ([num_heads][head_dim])
 *     value_cache[...]                                 = value[i]
 * A negative slot marks a padding token and is skipped. key and value are
 * [num_tokens][num_heads][head_dim]. The copy is bit-exact. num_tokens == 0 is
 * a no-op (pointers may then be NULL).
 */
int reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                      const int64_t* slot_mapping, int num_tokens, int num_heads, int head_dim,
                      int num_blocks, int block_size, int dtype, void* stream);

/*
 * Copy-on-write block copy [P2 "Python 演示" copy_on_write: the caller copies
 * the data into the newly allocated block; P3 §3.1.5 "CoW机制的实现" step 3;
 * P4 "Memory Sharing与写时复制"]. For each pair (src, dst) in block_mapping,
 * the whole block dst of both pools becomes a bit-exact copy of block src.
 * num_pairs == 0 is a no-op (pointers may then be NULL).
 */
int copy_blocks(void* key_cache, void* value_cache, const int32_t* block_mapping, int num_pairs,
                int num_heads, int head_dim, int num_blocks, int block_size, int dtype,
                void* stream);

/*
 * Swap-out / swap-in of whole blocks between a device pool and a pool in
 * pinned host memory [P1 §3.3.3 "显存不足时的处理策略", CPU Swap: the blocks of
 * a sequence being swapped out are copied block by block into pre-allocated
 * host buffers and its device blocks are freed; swapping in copies them back
 * into newly allocated device blocks; P2 "vLLM高性能推理架构的工程落地考量":
 * the cost is bound by the host link]. For each pair (src, dst) in
 * block_mapping, block dst of (dst_key, dst_value) becomes a bit-exact copy
 * of block src of (src_key, src_value); both pools are laid out
 * [num_blocks][block_size][num_heads][head_dim].
 *   Swap-out: src = the device pools, dst = the host pools.
 *   Swap-in:  src = the host pools,   dst = the device pools.
 * Each pool, and block_mapping (int32 [num_pairs][2]), must be device memory
 * of the current device or pinned host memory (hipHostMalloc, e.g. a torch
 * tensor made with pin_memory=True); anything else, or a pool smaller than
 * its num_blocks, returns PKV_ERR_MEMORY before any launch (checked with
 * hipPointerGetAttributes and hipMemGetAddressRange). One launch on `stream`
 * moves every pair; host memory is read and written by the kernel over the
 * host link, and the kernel's writes are visible to the host once `stream`
 * has been synchronised (when the destination pools are host memory, every
 * workgroup ends with a system-scope release; device destinations need none).
 * Preconditions: src ids < src_num_blocks, dst ids <
 * dst_num_blocks and unique. num_pairs == 0 is a no-op (pointers may then
 * be NULL).
 */
int swap_blocks(const void* src_key, const void* src_value, void* dst_key, void* dst_value,
                const int32_t* block_mapping, int num_pairs, int num_heads, int head_dim,
                int src_num_blocks, int dst_num_blocks, int block_size, int dtype, void* stream);

/*
 * The same block moves as swap_blocks, done by the DMA engines instead of a
 * kernel [P1 §3.3.3 "CPU Swap策略": swap is page-granular and runs as DMA
 * transfers between device and host]: one hipMemcpyAsync per pool for each
 * run of pairs whose source and destination ids both step by one, in
 * mapping order, on `stream`. block_mapping (int32 [num_pairs][2]) is HOST
 * memory here (any host memory), read during the call; every id is checked
 * against its pool (PKV_ERR_SHAPE) before the first copy. Pools as for
 * swap_blocks (PKV_ERR_MEMORY otherwise). A failed enqueue returns
 * PKV_ERR_LAUNCH; copies enqueued before it still run.
 */
int swap_blocks_dma(const void* src_key, const void* src_value, void* dst_key, void* dst_value,
                    const int32_t* block_mapping, int num_pairs, int num_heads, int head_dim,
                    int src_num_blocks, int dst_num_blocks, int block_size, int dtype,
                    void* stream);

/*
 * Swap-in through a device staging buffer: the same block moves as
 * swap_blocks / swap_blocks_dma (typically src = pinned host pools, dst =
 * device pools), done as DMA of each run of consecutive source ids into
 * consecutive staging slots (hipMemcpyAsync), then one block-copy launch that
 * scatters the slots to their destination blocks. Swapped-out sequences sit
 * in consecutive host blocks while their device blocks are scattered, so the
 * DMA moves long runs instead of one block per copy. Pairs are processed in
 * mapping order in chunks that fit `staging`, all on `stream`.
 *   block_mapping  int32 [num_pairs][2], HOST memory, read during the call;
 *                  every id is checked against its pool (PKV_ERR_SHAPE).
 *   staging        device memory, 256-byte aligned: a chunk of
 *                  staging_bytes / (2 * block_bytes) K slots followed by as
 *                  many V slots (block_bytes = block_size * num_heads *
 *                  head_dim * 2); at least one slot, else PKV_ERR_WORKSPACE.
 * The destination ids of each scatter launch travel in the launch's own
 * kernel arguments (up to 896 pairs per launch), so no host buffer outlives
 * the call and the enqueued work may be captured in a HIP graph.
 * Pools and staging as for swap_blocks (PKV_ERR_MEMORY otherwise).
 */
int swap_blocks_staged(const void* src_key, const void* src_value, void* dst_key,
                       void* dst_value, const int32_t* block_mapping, int num_pairs,
                       int num_heads, int head_dim, int src_num_blocks, int dst_num_blocks,
                       int block_size, int dtype, void* staging, size_t staging_bytes,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H */
