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
// Work decomposition. One workgroup (4 waves) per (sequence, head, 512-token
// partition); workgroup ids run heads fastest, so the 32 workgroups of one
// (sequence, partition) read the same blocks' token rows side by side. Inside
// a workgroup, wave w takes blocks w, w+4, ... of the partition. A token row
// of one head is head_dim 16-bit elements: 16 lanes x 16 bytes at head_dim
// 128 (8 lanes at 64), so one wave-wide 16-byte load covers 4 (8) rows and a
// block takes 4 (2) loads for K and as many for V, each coalesced. The block's
// physical id is a wave-uniform scalar load; the row addresses are that base
// plus a 32-bit lane offset.
//
// Arithmetic. q.k of one row: packed dot2 over the lane's 8 elements, then a
// 4-step DPP butterfly over the row's 16 lanes. Each group of lanes that
// shares rows keeps its own running (max, sum, accumulator) over its rows
// (online softmax in the log2 domain, scale pre-multiplied by log2 e), so the
// block loop needs no cross-row communication; the streams are merged by
// log-sum-exp at the end (shuffles inside a wave, LDS across waves). A
// sequence that fits one partition writes its output directly; longer ones
// write (max, sum, normalised output) partials that the merge kernel combines.
// Reduction order depends only on logical positions, never on physical ids.
//
// The next block's K and V rows are loaded before the current block is
// processed, so each wave keeps two blocks of loads in flight.

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kWaves = 4;

template <typename T, int D>
__global__ void __launch_bounds__(kWaves * 64)
decode_partition_kernel(uint16_t* __restrict__ out, float* __restrict__ ws_ml,
                        float* __restrict__ ws_o, const uint16_t* __restrict__ query,
                        const uint16_t* __restrict__ key_cache,
                        const uint16_t* __restrict__ value_cache,
                        const int32_t* __restrict__ block_tables,
                        const int32_t* __restrict__ context_lens, int num_seqs, int num_heads,
                        int max_blocks, int num_parts, float scale_log2) {
  using E = Elem<T>;
  constexpr int LPR = D / 8;     // lanes per token row
  constexpr int RPL = 64 / LPR;  // token rows per wave-wide load
  constexpr int NL = kBlockSize / RPL;  // wave-wide loads per block (K or V)

  const int H = num_heads;
  const int h = blockIdx.x % H;
  const int sp = blockIdx.x / H;
  const int s = sp % num_seqs;
  const int p = sp / num_seqs;
  const int ctx = context_lens[s];
  const int tok_begin = p * kPartitionTokens;
  if (tok_begin >= ctx) return;
  const int tok_end = min(ctx, tok_begin + kPartitionTokens);
  const int blk_begin = tok_begin / kBlockSize;
  const int nblk = (tok_end - tok_begin + kBlockSize - 1) / kBlockSize;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int r = lane / LPR;  // row group
  const int c = lane % LPR;  // 8-element column chunk

  const uint4 qv = *reinterpret_cast<const uint4*>(query + ((size_t)s * H + h) * D + c * 8);
  const int32_t* bt = block_tables + (size_t)s * max_blocks + blk_begin;
  const uint32_t kv_dim = (uint32_t)H * D;
  const size_t blk_bytes = (size_t)kBlockSize * kv_dim * sizeof(uint16_t);
  const uint32_t col_bytes = ((uint32_t)h * D + (uint32_t)c * 8) * sizeof(uint16_t);
  const char* kpool = reinterpret_cast<const char*>(key_cache);
  const char* vpool = reinterpret_cast<const char*>(value_cache);

  float m = -INFINITY, l = 0.f;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  auto valid_rows = [&](int b) { return min(kBlockSize, ctx - (blk_begin + b) * kBlockSize); };

  // Issue the K and V loads of block b. Every lane loads unconditionally; a
  // row past the context re-reads row 0 of the same block (always a valid
  // token, a cache hit), and process_block gives it weight 0.
  auto issue_block = [&](int b, uint4 (&kr)[NL], uint4 (&vr)[NL]) {
    const int phys = bt[b];
    const int rows = valid_rows(b);
    const char* kb = kpool + (size_t)phys * blk_bytes;
    const char* vb = vpool + (size_t)phys * blk_bytes;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const uint32_t row = (r + i * RPL < rows) ? (uint32_t)(r + i * RPL) : 0u;
      const uint32_t off = row * kv_dim * (uint32_t)sizeof(uint16_t) + col_bytes;
      kr[i] = *reinterpret_cast<const uint4*>(kb + off);
      vr[i] = *reinterpret_cast<const uint4*>(vb + off);
    }
  };

  // rows = number of valid token rows of the block (0 for a padding step).
  auto process_block = [&](int rows, const uint4 (&kr)[NL], const uint4 (&vr)[NL]) {
    float sc[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      float d = E::dot2(kr[i].x, qv.x, 0.f);
      d = E::dot2(kr[i].y, qv.y, d);
      d = E::dot2(kr[i].z, qv.z, d);
      d = E::dot2(kr[i].w, qv.w, d);
      d = group_sum<LPR>(d);
      sc[i] = (r + i * RPL < rows) ? d * scale_log2 : -INFINITY;
    }
    float bm = sc[0];
#pragma unroll
    for (int i = 1; i < NL; ++i) bm = fmaxf(bm, sc[i]);
    const float mn = fmaxf(m, bm);
    // While a row group has seen no valid row, m and mn are -inf; using 0 as
    // the reference then makes every weight 2^-inf = 0 without a branch (a
    // divergent branch here would split the compiler's load-wait tracking).
    const float ref = (mn == -INFINITY) ? 0.f : mn;
    const float alpha = fast_exp2(m - ref);
    l *= alpha;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= alpha;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
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
  };

  // This wave's blocks are wave, wave + kWaves, ...; my_n of them. Two register
  // sets alternate (explicit 2x unroll, no copies), and the next block's loads
  // are always issued before the current block is processed. The loop runs
  // whole pairs with no exit in between: a step past the wave's last block
  // re-reads that block (a cache hit) and is processed with zero valid rows,
  // which leaves (m, l, acc) unchanged. Branches around loads or an early exit
  // make the compiler wait for every outstanding load, prefetch included.
  const int my_n = (nblk > wave) ? (nblk - wave + kWaves - 1) / kWaves : 0;
  if (my_n > 0) {
    auto blk = [&](int j) { return wave + min(j, my_n - 1) * kWaves; };
    auto rows_of = [&](int j) { return j < my_n ? valid_rows(wave + j * kWaves) : 0; };
    uint4 kA[NL], vA[NL], kB[NL], vB[NL];
    issue_block(blk(0), kA, vA);
    for (int j = 0; j < my_n; j += 2) {
      issue_block(blk(j + 1), kB, vB);
      process_block(rows_of(j), kA, vA);
      issue_block(blk(j + 2), kA, vA);
      process_block(rows_of(j + 1), kB, vB);
    }
  }

  // Merge the row groups of this wave (lanes that differ only in row-group bits).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float mn = fmaxf(m, m2);
    const float ca = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
    const float cb = (m2 == -INFINITY) ? 0.f : fast_exp2(m2 - mn);
    l = l * ca + l2 * cb;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a2 = __shfl_xor(acc[j], off);
      acc[j] = acc[j] * ca + a2 * cb;
    }
    m = mn;
  }

  // Merge the waves through LDS.
  __shared__ float s_m[kWaves], s_l[kWaves];
  __shared__ float s_acc[kWaves][D];
  if (lane < LPR) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s_acc[wave][c * 8 + j] = acc[j];
  }
  if (lane == 0) {
    s_m[wave] = m;
    s_l[wave] = l;
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    float M = s_m[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float cw = (s_m[w] == -INFINITY) ? 0.f : fast_exp2(s_m[w] - M);
      L += s_l[w] * cw;
      o += s_acc[w][d] * cw;
    }
    const int parts_s = (ctx + kPartitionTokens - 1) / kPartitionTokens;
    if (parts_s == 1) {
      out[((size_t)s * H + h) * D + d] = E::round(o / L);
    } else {
      const size_t pi = ((size_t)s * H + h) * num_parts + p;
      ws_o[pi * D + d] = o / L;
      if (d == 0) {
        ws_ml[pi * 2] = M;
        ws_ml[pi * 2 + 1] = L;
      }
    }
  }
}

// Log-sum-exp merge of the partition partials of one (sequence, head); one
// thread per output element.
template <typename T, int D>
__global__ void __launch_bounds__(D)
decode_merge_kernel(uint16_t* __restrict__ out, const float* __restrict__ ws_ml,
                    const float* __restrict__ ws_o, const int32_t* __restrict__ context_lens,
                    int num_heads, int num_parts) {
  using E = Elem<T>;
  const int H = num_heads;
  const int h = blockIdx.x % H;
  const int s = blockIdx.x / H;
  const int ctx = context_lens[s];
  const int np = (ctx + kPartitionTokens - 1) / kPartitionTokens;
  if (np <= 1) return;
  const size_t base = ((size_t)s * H + h) * num_parts;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ws_ml[(base + p) * 2]);
  const int d = threadIdx.x;
  float L = 0.f, o = 0.f;
  for (int p = 0; p < np; ++p) {
    const float cw = ws_ml[(base + p) * 2 + 1] * fast_exp2(ws_ml[(base + p) * 2] - M);
    L += cw;
    o += cw * ws_o[(base + p) * D + d];
  }
  out[((size_t)s * H + h) * D + d] = E::round(o / L);
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

template <typename T, int D>
hipError_t partitions_t(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.num_seqs * a.num_heads * a.num_parts;
  hipLaunchKernelGGL((decode_partition_kernel<T, D>), dim3(grid), dim3(kWaves * 64), 0, st,
                     static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o,
                     static_cast<const uint16_t*>(a.query),
                     static_cast<const uint16_t*>(a.key_cache),
                     static_cast<const uint16_t*>(a.value_cache), a.block_tables, a.context_lens,
                     a.num_seqs, a.num_heads, a.max_blocks_per_seq, a.num_parts,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t merge_t(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.num_seqs * a.num_heads;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(grid), dim3(D), 0, st,
                     static_cast<uint16_t*>(a.out), a.ws_ml, a.ws_o, a.context_lens, a.num_heads,
                     a.num_parts);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_partitions(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 0) return a.head_dim == 64 ? partitions_t<F16, 64>(a, st) : partitions_t<F16, 128>(a, st);
  return a.head_dim == 64 ? partitions_t<BF16, 64>(a, st) : partitions_t<BF16, 128>(a, st);
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 0) return a.head_dim == 64 ? merge_t<F16, 64>(a, st) : merge_t<F16, 128>(a, st);
  return a.head_dim == 64 ? merge_t<BF16, 64>(a, st) : merge_t<BF16, 128>(a, st);
}

}  // namespace pkv
