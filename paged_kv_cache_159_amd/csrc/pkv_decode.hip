// Paged decode attention for gfx950: one query per (sequence, head) attends
// over that sequence's tokens, which live in physical blocks of 16 tokens (or
// 8 or 32) reached through the sequence's block table.
//
// Pages: [P3] "3.1 PagedAttention的核心原理" §3.1.3 (logical block = t / 16,
// offset = t % 16, physical = block_table[logical]; the flat table is indexed
// directly) and "页面访问优化" (all sequences in one launch; computation
// organised by physical block so reads within a block coalesce); [P1] "3.3
// 页面级显存管理" §3.3.1 "显存访问模式的优化" (16 consecutive tokens of a block
// are contiguous; one sequence's blocks visited close together in time).
// Block size: 16 is the default the pages settle on; larger blocks mean fewer
// table entries and lookups, smaller ones less waste in each sequence's last
// block ([P2] "KV Cache逻辑块物理块映射机制" and "vLLM高性能推理架构的工程落地考量";
// [P4] "PagedAttention: 页式管理内存"; [P1] §3.3.5 "自动调优策略" item 4). The
// kernels are built for 8, 16 and 32.
//
// Work decomposition. One workgroup (8 waves) per (sequence, context
// partition of PT tokens, group of HG heads). With the pool laid out
// [block][token][head][dim], one token row holds all heads side by side, so
// a head group's slice of a row is contiguous: HG = 4 heads x 128 dims (8 x 64)
// = 1 KB, exactly one wave-wide 16-byte load. Lane (hl, c) holds 8 elements
// of head hl. Wave w reads rows w, w+8, ... of every block of the partition
// (1, 2 or 4 rows at block size 8, 16, 32), so the 8 waves read a block's
// rows side by side. A block's physical id
// is a wave-uniform scalar load; row addresses are that block base plus a
// 32-bit lane offset. Workgroup ids run head groups fastest, so neighbouring
// workgroups read neighbouring pieces of the same token rows.
// Measured on MI355X (paged pool at the LLaMA-7B shape): 1 KB row pieces read
// faster than one head's 256 B pieces per workgroup, and whole 8 KB rows per
// workgroup leave too few workgroups at short contexts. Each workgroup's final
// stores (output or partials) cost far more than their bytes, so workgroups
// should be few and fast: 8 waves over 256-token partitions (512 when tables
// span more than 4096 tokens) beat 4 waves over 64-token partitions by ~8%.
//
// Arithmetic. q.k of one row and head: packed dot2 over the lane's 8 elements,
// then a DPP butterfly over the head's 16 (8) lanes. Each (wave, head) keeps a
// running (max, sum, accumulator) over its rows, online softmax in the log2
// domain with the scale pre-multiplied by log2 e; the 8 waves' streams are
// merged by log-sum-exp through LDS. A sequence that fits one partition writes
// its output directly; longer ones write (max, sum, normalised output)
// partials that the merge kernel combines. The reduction order depends only
// on logical token positions, never on physical block ids.

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_partition.h"

namespace pkv {

// LDS bytes that cap the partition kernel at two workgroups per CU (160 KiB
// of LDS per CU holds two of them, not three).
constexpr int kPartitionOccupancyLds = 60 * 1024;

template <typename T, int D, int PT, int BS, bool TAIL, bool BACKUP>
__global__ void __launch_bounds__(kWaves * 64)
decode_partition_kernel(uint16_t* __restrict__ out, float* __restrict__ ws_ml,
                        float* __restrict__ ws_o, const uint16_t* __restrict__ query,
                        const uint16_t* __restrict__ key_cache,
                        const uint16_t* __restrict__ value_cache,
                        const int32_t* __restrict__ block_tables,
                        const int32_t* __restrict__ context_lens, int num_seqs, int num_heads,
                        int max_blocks, int num_parts, float scale_log2,
                        const int32_t* __restrict__ group_start,
                        const int32_t* __restrict__ shared_blocks, int num_groups,
                        int slot_base, int32_t* __restrict__ seq_tok0,
                        uint32_t* __restrict__ flags, int backup_items) {
  // The LDS array is sized so that two 8-wave workgroups fit on a CU (the
  // kernel itself needs partition_lds_bytes): with four resident workgroups
  // per CU the LLaMA-7B and long-context decodes measured ~1% slower.
  constexpr int kLds = partition_lds_bytes<D>() > kPartitionOccupancyLds ? partition_lds_bytes<D>()
                                                                        : kPartitionOccupancyLds;
  __shared__ __align__(16) uint8_t lds[kLds];
  partition_body<T, D, PT, BS, TAIL, BACKUP>(blockIdx.x, out, ws_ml, ws_o, query, key_cache, value_cache,
                                     block_tables, context_lens, num_seqs, num_heads, max_blocks,
                                     num_parts, scale_log2, group_start, shared_blocks,
                                     num_groups, slot_base, seq_tok0, lds, flags, backup_items);
}

// Log-sum-exp merge of the partials of one (sequence, head). Partials live in
// slots [0, n0) and [slot_base, slot_base + n1) of the sequence's slot row
// (the plain call uses only the first range; the grouped call puts the
// shared-prefix chunks in the first and the tail partitions in the second).
// THREADS threads: thread (k, d) merges slots k, k + K, ... for output element
// d (K = THREADS / D) in one online pass, then the K states meet in LDS (one
// barrier). The loads of different slots are independent, so many are in
// flight. Few slots per (sequence, head) take 128 threads (one 128-dim head
// per thread row, so the whole grid fits the machine at once: ~2% faster at
// the shared-prefix workload); many take 1024 (eight streams per output
// element at head size 128, so a 64-slot merge is two rounds of four loads
// per thread: 8 x 32K tokens 626.3 -> 623.9 us for the decode call on
// MI355X, against 624.7 with 512 threads; the whole grid of 256 (sequence,
// head) workgroups is one per CU).
constexpr int kMergeSlotsFor128 = 16;
constexpr int kMergeThreadsMany = 1024;

template <typename T, int D, bool GROUPED, int THREADS>
__global__ void __launch_bounds__(THREADS)
decode_merge_kernel(uint16_t* __restrict__ out, const float* __restrict__ ws_ml,
                    const float* __restrict__ ws_o, const int32_t* __restrict__ context_lens,
                    int num_heads, int num_parts, int part_tokens,
                    const int32_t* __restrict__ seq_tok0, int slot_base) {
  using E = Elem<T>;
  constexpr int K = THREADS / D;
  const int H = num_heads;
  const int h = blockIdx.x % H;
  const int s = blockIdx.x / H;
  const int ctx = context_lens[s];
  int n0, n1;
  if constexpr (GROUPED) {
    constexpr int chunk_tokens = kSharedChunkTiles * kTileTokens;
    const int st = seq_tok0[s];   // shared-prefix tokens, written by the main launch
    n0 = (st + chunk_tokens - 1) / chunk_tokens;
    n1 = (ctx - st + part_tokens - 1) / part_tokens;
  } else {
    n0 = (ctx + part_tokens - 1) / part_tokens;
    n1 = 0;
    if (n0 <= 1) return;  // written directly by the partition launch
  }
  const int n = n0 + n1;
  auto slot = [&](int i) { return i < n0 ? i : slot_base + (i - n0); };
  const size_t base = ((size_t)s * H + h) * num_parts;
  const int d = threadIdx.x % D;
  const int k = threadIdx.x / D;
  // One pass: each thread keeps a running (max, weight sum, output) over its
  // partials, so a partial's (m, l) pair and output element are loaded
  // together. Every partial covers at least one token, so its m is finite;
  // the first one turns the running max from -inf into a number (weight
  // 2^-inf = 0 for the empty state).
  float M = -INFINITY, L = 0.f, o = 0.f;
#pragma unroll 4
  for (int i = k; i < n; i += K) {
    const size_t pi = base + slot(i);
    const float mi = ws_ml[pi * 2];
    const float li = ws_ml[pi * 2 + 1];
    const float oi = ws_o[pi * D + d];
    const float mn = fmaxf(M, mi);
    const float a = fast_exp2(M - mn);
    const float w = li * fast_exp2(mi - mn);
    L = L * a + w;
    o = o * a + w * oi;
    M = mn;
  }
  __shared__ float s_o[THREADS], s_m[K], s_l[K];
  s_o[threadIdx.x] = o;
  if (d == 0) {
    s_m[k] = M;
    s_l[k] = L;
  }
  __syncthreads();
  if (k == 0) {
    float mx = s_m[0];
#pragma unroll
    for (int j = 1; j < K; ++j) mx = fmaxf(mx, s_m[j]);
    float oo = 0.f, ll = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      // a thread with no partials (n < K) holds M = -inf and weight 0
      const float c = s_m[j] == -INFINITY ? 0.f : fast_exp2(s_m[j] - mx);
      oo += s_o[j * D + d] * c;
      ll += s_l[j] * c;
    }
    out[((size_t)s * H + h) * D + d] = E::round(oo / ll);
  }
}

// The same merge for calls with at most kMergeSlotsFor128 partial slots per
// (sequence, head), packed: one 256-thread workgroup per (sequence, block of
// MH heads), thread (head, quad) merging four consecutive output elements
// with 16-byte partial loads (MH = 8 at head size 128, 16 at 64). A
// (sequence, head) in 2-wave workgroups took 4,096 workgroups at the
// shared-prefix workload; this takes 512. Per element the arithmetic is the
// single-chain pass above, so the outputs are the same bits.
template <typename T, int D, bool GROUPED>
__global__ void __launch_bounds__(256)
decode_merge_packed_kernel(uint16_t* __restrict__ out, const float* __restrict__ ws_ml,
                           const float* __restrict__ ws_o, const int32_t* __restrict__ context_lens,
                           int num_heads, int num_parts, int part_tokens,
                           const int32_t* __restrict__ seq_tok0, int slot_base) {
  using E = Elem<T>;
  constexpr int QPH = D / 4;       // threads per head
  constexpr int MH = 256 / QPH;    // heads per workgroup
  const int H = num_heads;
  const int hblocks = (H + MH - 1) / MH;
  const int s = blockIdx.x / hblocks;
  const int h = (blockIdx.x % hblocks) * MH + (int)threadIdx.x / QPH;
  const int q = threadIdx.x % QPH;
  if (h >= H) return;
  const size_t base = ((size_t)s * H + h) * num_parts;
  // The first kMergeAhead slots of this (sequence, head), and in the grouped
  // call its first tail slot, are loaded before the lengths that say which of
  // them hold partials arrive (all lie inside the row; unused ones are
  // dropped): the lengths' round trip then overlaps the partials'.
  constexpr int kMergeAhead = 4;
  float2 aml[kMergeAhead + 1];
  float4 ao[kMergeAhead + 1];
#pragma unroll
  for (int j = 0; j <= kMergeAhead; ++j) {
    const int slot = j < kMergeAhead ? j : slot_base;
    if ((j < kMergeAhead || GROUPED) && slot < num_parts) {
      aml[j] = *reinterpret_cast<const float2*>(ws_ml + (base + slot) * 2);
      ao[j] = *reinterpret_cast<const float4*>(ws_o + (base + slot) * D + 4 * q);
    }
  }
  const int ctx = context_lens[s];
  int n0, n1;
  if constexpr (GROUPED) {
    constexpr int chunk_tokens = kSharedChunkTiles * kTileTokens;
    const int st = seq_tok0[s];
    n0 = (st + chunk_tokens - 1) / chunk_tokens;
    n1 = (ctx - st + part_tokens - 1) / part_tokens;
    // keeps the compiler from sinking the length load past the first folds,
    // which put its round trip at the end
    asm volatile("" ::"s"(n1));
  } else {
    n0 = (ctx + part_tokens - 1) / part_tokens;
    n1 = 0;
    if (n0 <= 1) return;  // written directly by the partition launch
  }
  float M = -INFINITY, L = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fold = [&](const float2 ml, const float4 oi) {
    const float mn = fmaxf(M, ml.x);
    const float a = fast_exp2(M - mn);
    const float w = ml.y * fast_exp2(ml.x - mn);
    L = L * a + w;
    o.x = o.x * a + w * oi.x;
    o.y = o.y * a + w * oi.y;
    o.z = o.z * a + w * oi.z;
    o.w = o.w * a + w * oi.w;
    M = mn;
  };
  // slots 0 .. n0 - 1, then slot_base .. slot_base + n1 - 1, in that order
#pragma unroll
  for (int j = 0; j < kMergeAhead; ++j)
    if (j < n0) fold(aml[j], ao[j]);
#pragma unroll 4
  for (int i = kMergeAhead; i < n0; ++i)
    fold(*reinterpret_cast<const float2*>(ws_ml + (base + i) * 2),
         *reinterpret_cast<const float4*>(ws_o + (base + i) * D + 4 * q));
  if constexpr (GROUPED) {
    if (n1 > 0) fold(aml[kMergeAhead], ao[kMergeAhead]);
#pragma unroll 4
    for (int i = 1; i < n1; ++i)
      fold(*reinterpret_cast<const float2*>(ws_ml + (base + slot_base + i) * 2),
           *reinterpret_cast<const float4*>(ws_o + (base + slot_base + i) * D + 4 * q));
  }
  const uint2 r = make_uint2(E::pack2(o.x / L, o.y / L), E::pack2(o.z / L, o.w / L));
  *reinterpret_cast<uint2*>(out + ((size_t)s * H + h) * D + 4 * q) = r;
}

int decode_partition_tokens(int num_seqs, int num_heads, int head_dim, int max_blocks_per_seq,
                            int block_size) {
  // 512 tokens when tables span more than 4096 tokens, or when 256-token
  // partitions would make a grid of 8192 or more (sequence, partition, head
  // group) slots; 256 otherwise. Measured on MI355X (32 heads x 128, fp16,
  // decode call, 256 -> 512): 64 sequences of U[128, 2048] 167.1 -> 170.5 us
  // and 64 of Exp(512) 89.2 -> 94.6 us (4096 slots: 256 stays), but 128 of
  // U[128, 2048] 368.5 -> 364.4, 256 of Exp(512) 358.1 -> 350.4 and 256 of
  // U[128, 2048] 694.0 -> 684.5 (8192 and 16384 slots): large batches have
  // items enough to balance, and fewer partials to write and merge.
  const int64_t tokens = (int64_t)max_blocks_per_seq * block_size;
  if (tokens > 4096) return 512;
  const int64_t head_groups = (num_heads + 64 / (head_dim / 8) - 1) / (64 / (head_dim / 8));
  const int64_t slots = (int64_t)num_seqs * head_groups * ((tokens + 255) / 256);
  return slots >= kLargeGridSlots ? 512 : 256;
}

size_t decode_workspace_bytes(int num_seqs, int num_heads, int head_dim, int num_parts) {
  const size_t n = (size_t)num_seqs * num_heads * num_parts;
  const size_t ml = (n * 2 * sizeof(float) + 255) & ~(size_t)255;
  return ml + n * head_dim * sizeof(float);
}

void decode_workspace_split(void* ws, int num_seqs, int num_heads, int num_parts, float** ml,
                            float** o) {
  const size_t n = (size_t)num_seqs * num_heads * num_parts;
  const size_t mlb = (n * 2 * sizeof(float) + 255) & ~(size_t)255;
  *ml = static_cast<float*>(ws);
  *o = reinterpret_cast<float*>(static_cast<char*>(ws) + mlb);
}

namespace {
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D, int PT, int BS, bool TAIL, bool BACKUP>
hipError_t partitions_t(const DecodeArgs& a, hipStream_t st) {
  constexpr int HG = 64 / (D / 8);
  const unsigned groups = (unsigned)(a.num_heads + HG - 1) / HG;
  unsigned grid = (unsigned)a.num_seqs * groups * (unsigned)a.tail_parts;
  if (BACKUP) grid += (unsigned)a.backup_items * groups;   // backup workgroups of the last items
  hipLaunchKernelGGL((decode_partition_kernel<T, D, PT, BS, TAIL, BACKUP>), dim3(grid), dim3(kWaves * 64), 0, st,
                     static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o,
                     static_cast<const uint16_t*>(a.query),
                     static_cast<const uint16_t*>(a.key_cache),
                     static_cast<const uint16_t*>(a.value_cache), a.block_tables, a.context_lens,
                     a.num_seqs, a.num_heads, a.max_blocks_per_seq, a.num_parts,
                     a.scale * kLog2e, a.group_start, a.shared_blocks, a.num_groups, a.slot_base,
                     a.ws_seq, BACKUP ? a.flags : nullptr, BACKUP ? a.backup_items : 0);
  return hipGetLastError();
}

template <typename T, int D, int BS>
hipError_t partitions_b(const DecodeArgs& a, hipStream_t st) {
  const bool tail = a.group_start != nullptr;
  // backups only where the host gave claim flags: planned orders over
  // 512-token partitions
  const bool backup = !tail && a.flags != nullptr && plan_fits(a.num_seqs, a.num_parts);
  if (a.part_tokens == 256)
    return tail ? partitions_t<T, D, 256, BS, true, false>(a, st)
                : partitions_t<T, D, 256, BS, false, false>(a, st);
  if (tail) return partitions_t<T, D, 512, BS, true, false>(a, st);
  return backup ? partitions_t<T, D, 512, BS, false, true>(a, st)
                : partitions_t<T, D, 512, BS, false, false>(a, st);
}

template <typename T, int D>
hipError_t partitions_d(const DecodeArgs& a, hipStream_t st) {
  if (a.block_size == 8) return partitions_b<T, D, 8>(a, st);
  if (a.block_size == 32) return partitions_b<T, D, 32>(a, st);
  return partitions_b<T, D, 16>(a, st);
}

template <typename T, int D, int THREADS>
hipError_t merge_n(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.num_seqs * a.num_heads;
  if (a.ws_seq != nullptr) {
    hipLaunchKernelGGL((decode_merge_kernel<T, D, true, THREADS>), dim3(grid), dim3(THREADS), 0,
                       st, static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o, a.context_lens,
                       a.num_heads, a.num_parts, a.part_tokens, a.ws_seq, a.slot_base);
  } else {
    hipLaunchKernelGGL((decode_merge_kernel<T, D, false, THREADS>), dim3(grid), dim3(THREADS), 0,
                       st, static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o, a.context_lens,
                       a.num_heads, a.num_parts, a.part_tokens, nullptr, 0);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t merge_packed(const DecodeArgs& a, hipStream_t st) {
  constexpr int MH = 256 / (D / 4);
  const unsigned grid = (unsigned)a.num_seqs * (unsigned)((a.num_heads + MH - 1) / MH);
  if (a.ws_seq != nullptr) {
    hipLaunchKernelGGL((decode_merge_packed_kernel<T, D, true>), dim3(grid), dim3(256), 0, st,
                       static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o, a.context_lens,
                       a.num_heads, a.num_parts, a.part_tokens, a.ws_seq, a.slot_base);
  } else {
    hipLaunchKernelGGL((decode_merge_packed_kernel<T, D, false>), dim3(grid), dim3(256), 0, st,
                       static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o, a.context_lens,
                       a.num_heads, a.num_parts, a.part_tokens, nullptr, 0);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t merge_t(const DecodeArgs& a, hipStream_t st) {
  return a.num_parts <= kMergeSlotsFor128 ? merge_packed<T, D>(a, st) : merge_n<T, D, kMergeThreadsMany>(a, st);
}
}  // namespace

hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 0) return a.head_dim == 64 ? partitions_d<F16, 64>(a, st) : partitions_d<F16, 128>(a, st);
  return a.head_dim == 64 ? partitions_d<BF16, 64>(a, st) : partitions_d<BF16, 128>(a, st);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 0) return a.head_dim == 64 ? merge_t<F16, 64>(a, st) : merge_t<F16, 128>(a, st);
  return a.head_dim == 64 ? merge_t<BF16, 64>(a, st) : merge_t<BF16, 128>(a, st);
}

}  // namespace pkv
