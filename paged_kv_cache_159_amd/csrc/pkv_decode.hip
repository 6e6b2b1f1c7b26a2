// Paged decode attention for gfx950: one query per (sequence, head) attends
// over that sequence's tokens, which live in 16-token physical blocks reached
// through the sequence's block table.
//
// Pages: [P3] "3.1 PagedAttention的核心原理" §3.1.3 (logical block = t / 16,
// offset = t % 16, physical = block_table[logical]; the flat table is indexed
// directly) and "页面访问优化" (all sequences in one launch; computation
// organised by physical block so reads within a block coalesce); [P1] "3.3
// 页面级显存管理" §3.3.1 "显存访问模式的优化" (16 consecutive tokens of a block
// are contiguous; one sequence's blocks visited close together in time).
//
// Work decomposition. One workgroup (8 waves) per (sequence, context
// partition of PT tokens, group of HG heads). With the pool laid out
// [block][token][head][dim], one token row holds all heads side by side, so
// a head group's slice of a row is contiguous: HG = 4 heads x 128 dims (8 x 64)
// = 1 KB, exactly one wave-wide 16-byte load. Lane (hl, c) holds 8 elements
// of head hl. Wave w reads rows w and w+8 of every block of the partition, so
// the 8 waves read the 16 rows of a block side by side. A block's physical id
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

namespace pkv {

constexpr int kWaves = 8;
constexpr int kRowsPerWave = kBlockSize / kWaves;  // rows of a block each wave reads

// TAIL = true is the grouped call's second launch: each sequence starts after
// its group's shared blocks (those are handled by the shared-prefix kernel),
// its partitions go to partial slots slot_base + p, and every partition
// writes a partial (the merge always runs).
template <typename T, int D, int PT, bool TAIL>
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
                        int slot_base) {
  using E = Elem<T>;
  constexpr int LPR = D / 8;         // lanes per head row (16 bytes each)
  constexpr int HG = 64 / LPR;       // heads per wave-wide load
  static_assert(PT % kBlockSize == 0, "partition is whole blocks");

  const int H = num_heads;
  const int groups = (H + HG - 1) / HG;
  const int g = blockIdx.x % groups;
  const int sp = blockIdx.x / groups;
  const int s = sp % num_seqs;
  const int p = sp / num_seqs;
  const int ctx = context_lens[s];
  int tok0 = 0;   // first token this launch covers for sequence s
  if constexpr (TAIL) tok0 = shared_blocks[group_of(s, group_start, num_groups)] * kBlockSize;
  const int tok_begin = tok0 + p * PT;
  if (tok_begin >= ctx) return;
  const int tok_end = min(ctx, tok_begin + PT);
  const int blk_begin = tok_begin / kBlockSize;
  const int nblk = (tok_end - tok_begin + kBlockSize - 1) / kBlockSize;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int hl = lane / LPR;          // head within the group
  const int c = lane % LPR;           // 8-element column chunk
  const int h = g * HG + hl;
  const bool head_ok = h < H;
  const int hr = head_ok ? h : 0;     // lanes past the last head read head 0 and are ignored

  const uint4 qv = *reinterpret_cast<const uint4*>(query + ((size_t)s * H + hr) * D + c * 8);
  const int32_t* bt = block_tables + (size_t)s * max_blocks + blk_begin;
  const uint32_t kv_dim = (uint32_t)H * D;
  const size_t blk_bytes = (size_t)kBlockSize * kv_dim * sizeof(uint16_t);
  const uint32_t col_bytes = ((uint32_t)hr * D + (uint32_t)c * 8) * sizeof(uint16_t);
  const char* kpool = reinterpret_cast<const char*>(key_cache);
  const char* vpool = reinterpret_cast<const char*>(value_cache);

  float m = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  for (int b = 0; b < nblk; ++b) {
    const int phys = bt[b];
    const int rows = min(kBlockSize, ctx - (blk_begin + b) * kBlockSize);
    const char* kb = kpool + (size_t)phys * blk_bytes;
    const char* vb = vpool + (size_t)phys * blk_bytes;
    // Rows past the context re-read row 0 of the block (a valid token, a
    // cache hit) instead of branching; their weight is exactly 0 below.
    uint4 kr[kRowsPerWave], vr[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int row = wave + i * kWaves;
      const uint32_t rr = row < rows ? (uint32_t)row : 0u;
      const uint32_t off = rr * kv_dim * (uint32_t)sizeof(uint16_t) + col_bytes;
      kr[i] = *reinterpret_cast<const uint4*>(kb + off);
      vr[i] = *reinterpret_cast<const uint4*>(vb + off);
    }
    float sc[kRowsPerWave];
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      float d = E::dot2(kr[i].x, qv.x, 0.f);
      d = E::dot2(kr[i].y, qv.y, d);
      d = E::dot2(kr[i].z, qv.z, d);
      d = E::dot2(kr[i].w, qv.w, d);
      d = group_sum<LPR>(d);
      sc[i] = (wave + i * kWaves < rows) ? d * scale_log2 : -INFINITY;
    }
    float bm = sc[0];
#pragma unroll
    for (int i = 1; i < kRowsPerWave; ++i) bm = fmaxf(bm, sc[i]);
    const float mn = fmaxf(m, bm);
    // While a stream has seen no valid row, m and mn are -inf; using 0 as the
    // reference then makes every weight 2^-inf = 0 without a branch (a
    // divergent branch here would make the compiler wait for all loads).
    const float ref = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(m - ref);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const float pw = fast_exp2(sc[i] - ref);
      l += pw;
      acc[0] += pw * E::lo(vr[i].x);
      acc[1] += pw * E::hi(vr[i].x);
      acc[2] += pw * E::lo(vr[i].y);
      acc[3] += pw * E::hi(vr[i].y);
      acc[4] += pw * E::lo(vr[i].z);
      acc[5] += pw * E::hi(vr[i].z);
      acc[6] += pw * E::lo(vr[i].w);
      acc[7] += pw * E::hi(vr[i].w);
    }
    m = mn;
  }

  // Merge the waves' streams of each head through LDS.
  __shared__ float s_m[kWaves][HG], s_l[kWaves][HG];
  __shared__ float s_acc[kWaves][HG * D];
#pragma unroll
  for (int j = 0; j < 8; ++j) s_acc[wave][hl * D + c * 8 + j] = acc[j];
  if (c == 0) {
    s_m[wave][hl] = m;
    s_l[wave][hl] = l;
  }
  __syncthreads();
  const int parts_s = TAIL ? 0 : (ctx + PT - 1) / PT;
  for (int o = threadIdx.x; o < HG * D; o += kWaves * 64) {
    const int ol = o / D;
    const int d = o % D;
    const int oh = g * HG + ol;
    if (oh >= H) break;   // o grows, so later o are past H too
    float M = s_m[0][ol];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][ol]);
    float L = 0.f, val = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float cw = (s_m[w][ol] == -INFINITY) ? 0.f : fast_exp2(s_m[w][ol] - M);
      L += s_l[w][ol] * cw;
      val += s_acc[w][o] * cw;
    }
    if (parts_s == 1) {
      out[((size_t)s * H + oh) * D + d] = E::round(val / L);
    } else {
      const size_t pi = ((size_t)s * H + oh) * num_parts + slot_base + p;
      ws_o[pi * D + d] = val / L;
      if (d == 0) {
        ws_ml[pi * 2] = M;
        ws_ml[pi * 2 + 1] = L;
      }
    }
  }
}

// Log-sum-exp merge of the partials of one (sequence, head). Partials live in
// slots [0, n0) and [slot_base, slot_base + n1) of the sequence's slot row
// (the plain call uses only the first range; the grouped call puts the
// shared-prefix chunks in the first and the tail partitions in the second).
// 256 threads: thread (k, d) sums slots k, k + K, ... for output element d
// (K = 256 / D), then the K partial sums meet in LDS. The loads of different
// slots are independent, so many are in flight.
constexpr int kMergeThreads = 256;

template <typename T, int D, bool GROUPED>
__global__ void __launch_bounds__(kMergeThreads)
decode_merge_kernel(uint16_t* __restrict__ out, const float* __restrict__ ws_ml,
                    const float* __restrict__ ws_o, const int32_t* __restrict__ context_lens,
                    int num_heads, int num_parts, int part_tokens,
                    const int32_t* __restrict__ group_start,
                    const int32_t* __restrict__ shared_blocks, int num_groups, int chunk_blocks,
                    int slot_base) {
  using E = Elem<T>;
  constexpr int K = kMergeThreads / D;
  const int H = num_heads;
  const int h = blockIdx.x % H;
  const int s = blockIdx.x / H;
  const int ctx = context_lens[s];
  int n0, n1;
  if constexpr (GROUPED) {
    const int sb = shared_blocks[group_of(s, group_start, num_groups)];
    n0 = (sb + chunk_blocks - 1) / chunk_blocks;
    n1 = (ctx - sb * kBlockSize + part_tokens - 1) / part_tokens;
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
  __shared__ float s_red[kMergeThreads];
  float M = -INFINITY;
  for (int i = threadIdx.x; i < n; i += kMergeThreads) M = fmaxf(M, ws_ml[(base + slot(i)) * 2]);
  s_red[threadIdx.x] = M;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) s_red[threadIdx.x] = fmaxf(s_red[threadIdx.x], s_red[threadIdx.x + w]);
    __syncthreads();
  }
  M = s_red[0];
  __syncthreads();
  float L = 0.f, o = 0.f;
#pragma unroll 4
  for (int i = k; i < n; i += K) {
    const size_t pi = base + slot(i);
    const float cw = ws_ml[pi * 2 + 1] * fast_exp2(ws_ml[pi * 2] - M);
    L += cw;
    o += cw * ws_o[pi * D + d];
  }
  __shared__ float s_o[kMergeThreads], s_l[K];
  s_o[threadIdx.x] = o;
  if (d == 0) s_l[k] = L;
  __syncthreads();
  if (k == 0) {
    float oo = 0.f, ll = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      oo += s_o[j * D + d];
      ll += s_l[j];
    }
    out[((size_t)s * H + h) * D + d] = E::round(oo / ll);
  }
}

int decode_partition_tokens(int max_blocks_per_seq, int block_size) {
  // 256 tokens while tables span at most 4096 tokens; 512 beyond, where the
  // grid is large anyway and fewer partials mean less merge traffic.
  const int64_t tokens = (int64_t)max_blocks_per_seq * block_size;
  return tokens <= 4096 ? 256 : 512;
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

template <typename T, int D, int PT, bool TAIL>
hipError_t partitions_t(const DecodeArgs& a, hipStream_t st) {
  constexpr int HG = 64 / (D / 8);
  const unsigned groups = (unsigned)(a.num_heads + HG - 1) / HG;
  const unsigned grid = (unsigned)a.num_seqs * groups * (unsigned)a.tail_parts;
  hipLaunchKernelGGL((decode_partition_kernel<T, D, PT, TAIL>), dim3(grid), dim3(kWaves * 64), 0, st,
                     static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o,
                     static_cast<const uint16_t*>(a.query),
                     static_cast<const uint16_t*>(a.key_cache),
                     static_cast<const uint16_t*>(a.value_cache), a.block_tables, a.context_lens,
                     a.num_seqs, a.num_heads, a.max_blocks_per_seq, a.num_parts,
                     a.scale * kLog2e, a.group_start, a.shared_blocks, a.num_groups, a.slot_base);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t partitions_d(const DecodeArgs& a, hipStream_t st) {
  const bool tail = a.group_start != nullptr;
  if (a.part_tokens == 256)
    return tail ? partitions_t<T, D, 256, true>(a, st) : partitions_t<T, D, 256, false>(a, st);
  return tail ? partitions_t<T, D, 512, true>(a, st) : partitions_t<T, D, 512, false>(a, st);
}

template <typename T, int D>
hipError_t merge_t(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.num_seqs * a.num_heads;
  if (a.group_start != nullptr) {
    hipLaunchKernelGGL((decode_merge_kernel<T, D, true>), dim3(grid), dim3(kMergeThreads), 0, st,
                       static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o, a.context_lens, a.num_heads,
                       a.num_parts, a.part_tokens, a.group_start, a.shared_blocks, a.num_groups,
                       kSharedChunkBlocks, a.slot_base);
  } else {
    hipLaunchKernelGGL((decode_merge_kernel<T, D, false>), dim3(grid), dim3(kMergeThreads), 0, st,
                       static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o, a.context_lens, a.num_heads,
                       a.num_parts, a.part_tokens, a.group_start, a.shared_blocks, a.num_groups,
                       kSharedChunkBlocks, 0);
  }
  return hipGetLastError();
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
