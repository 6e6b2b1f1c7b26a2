// Grouped decode, first launch: attention of several queries over the prefix
// blocks their sequences share, on the MFMA matrix cores of gfx950.
//
// Pages: sharing a prefix maps several sequences' logical blocks to the same
// physical blocks, with a reference count per block ([P2] "vLLM三大核心技术分页
// 内存与共享解码", "Copy-on-Write共享解码的显存优化原理"; [P1] "3.3 页面级显存管理",
// "Copy-on-Write页面共享机制"; parallel sampling and beam search in [P4]
// "Memory Sharing与写时复制"). A shared block is then read once for all its
// readers instead of once per sequence, and the work on a shared tile of 16
// tokens becomes a dense contraction: Q_group [n x D] against K_tile [16 x D]
// and V_tile [16 x D]. A tile is a whole 16-token block, half a 32-token
// block or two 8-token blocks; the tile is gathered through the block table
// row by row, so the MFMA shape is the same at every block size.
//
// One 8-wave workgroup per (group, chunk of kSharedChunkTiles shared tiles,
// head); up to 16 queries per MFMA tile (larger groups loop over tiles).
//   S^T = K Q^T with v_mfma_f32_16x16x32 (M = 16 tokens, N = 16 queries,
//   K = 32 dims per instruction), A operand (lane l: token l%16, 8 dims) read
//   from the K rows staged in LDS, B operand (query l%16) from Q. Lane group
//   q = l/16 covers dims [q*D/4, (q+1)*D/4).
//   The accumulator holds S^T[token 4*(l/16)+v][query l%16] (v < 4): exactly
//   the B-operand layout P^T needs for O^T = V^T P^T with v_mfma_f32_16x16x16
//   (K = 16 tokens), so P never moves between lanes.
//   V^T's A operand wants 4 tokens of one dim per lane, a transposed read from
//   the V rows staged in LDS (rows padded to spread banks).
//   P is split into hi + lo 16-bit parts (two MFMAs), so the 16-bit operand
//   costs no accuracy next to the fp32 softmax.
// The unit writes (max, sum, normalised output) partials for its chunk; the
// merge kernel combines them with the sequences' tail partitions, which run in
// the same launch (decode_grouped_kernel).

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_mfma.h"
#include "pkv_partition.h"

namespace pkv {

constexpr int kQueryTile = 16;
constexpr int kGroupedWaves = 8;   // same workgroup shape as the partition kernel

// LDS bytes of one shared-prefix unit: K and V rows of one head for one tile,
// double-buffered, rows padded by 16 bytes to spread LDS banks.
template <int D>
constexpr int shared_row_bytes() { return 2 * D + 16; }
template <int D>
constexpr int shared_lds_bytes() { return 2 * 2 * kTileTokens * shared_row_bytes<D>(); }

// One shared-prefix unit (group g, chunk of kSharedChunkTiles shared tiles,
// head h) on an 8-wave workgroup over blocks of BS tokens. Tiles go through
// LDS one at a time: each thread holds one 16-byte piece of the head's K or V
// rows of the next tile in registers while the waves compute on the current
// one, so a tile's load overlaps the previous tile's MFMAs, with one barrier
// per tile. Every wave computes S^T = K Q^T per tile (a few MFMAs, identical
// in every wave) and its own 16 output dims of O^T = V^T P^T, so registers
// stay low. Groups larger than 16 run the chunk once per 16-query tile (the
// re-reads hit L2).
template <typename T, int D, int BS>
__device__ __forceinline__ void shared_unit(
    int g, int chunk, int h, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const uint16_t* __restrict__ query, const uint16_t* __restrict__ key_cache,
    const uint16_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ group_start, const int32_t* __restrict__ shared_blocks,
    int H, int max_blocks, int num_parts, float scale_log2, uint8_t* lds) {
  using E = Elem<T>;
  using M = Mfma<T>;
  constexpr int NQK = D / 32;        // S MFMAs (32 dims each)
  constexpr int NPV = D / 16;        // 16-dim output chunks; wave w owns chunk w
  constexpr int SPAN = D / 4;        // dims per lane group in the S contraction
  constexpr int ROW = shared_row_bytes<D>();
  constexpr int PIECES = kTileTokens * D / 8;  // 16-byte pieces of one head's K (or V) tile
  constexpr int BUF = 2 * kTileTokens * ROW;   // one buffer: K rows, then V rows
  static_assert(2 * PIECES <= kGroupedWaves * 64, "one piece per thread per tile");
  const int st = shared_prefix_tokens(shared_blocks[g], BS);
  const int t0_chunk = chunk * kSharedChunkTiles * kTileTokens;
  if (t0_chunk >= st) return;
  const int nt = min(kSharedChunkTiles, (st - t0_chunk) / kTileTokens);
  const int s0 = group_start[g];
  const int s1 = group_start[g + 1];
  if (s1 <= s0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const uint32_t kv_dim = (uint32_t)H * D;
  // The group's first member's table: the shared entries are the same in all.
  const int32_t* bt = block_tables + (size_t)s0 * max_blocks;
  const bool pv_wave = wave < NPV;

  // This thread's piece: tensor `which` (0 = K, 1 = V), token row r of the
  // tile, 16-byte column cc; it lands at LDS byte (which * 16 + r) * ROW +
  // cc * 16 of a buffer. Token t of the prefix is at slot
  // block_table[t / BS] * BS + t % BS, whose row starts at element slot * kv_dim.
  const int pc = threadIdx.x;
  const bool loader = pc < 2 * PIECES;
  const int which = pc / PIECES;
  const int r = (pc % PIECES) / (D / 8);
  const int cc = pc % (D / 8);
  const uint16_t* src = (which ? value_cache : key_cache) + (size_t)h * D + cc * 8;
  const int dst = (which * kTileTokens + r) * ROW + cc * 16;
  auto load_piece = [&](int tile) {
    const int t = t0_chunk + tile * kTileTokens + r;
    const size_t slot = (size_t)bt[t / BS] * BS + (t % BS);
    return *reinterpret_cast<const uint4*>(src + slot * kv_dim);
  };

  for (int t0 = s0; t0 < s1; t0 += kQueryTile) {
    const int sq = t0 + col;
    const bool q_ok = sq < s1;
    uint4 qf[NQK];
#pragma unroll
    for (int i = 0; i < NQK; ++i)
      qf[i] = q_ok ? *reinterpret_cast<const uint4*>(query + ((size_t)sq * H + h) * D +
                                                     grp * SPAN + 8 * i)
                   : make_uint4(0, 0, 0, 0);
    uint4 piece = make_uint4(0, 0, 0, 0);
    if (loader) piece = load_piece(0);
    f4_t acc = {0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    for (int b = 0; b < nt; ++b) {
      // The buffer written here was last read in tile b - 2's step; every
      // wave has passed tile b - 1's barrier since.
      uint8_t* buf = lds + (b & 1) * BUF;
      if (loader) *reinterpret_cast<uint4*>(buf + dst) = piece;
      __syncthreads();
      if (loader && b + 1 < nt) piece = load_piece(b + 1);
      const uint8_t* s_k = buf;
      const uint8_t* s_v = buf + kTileTokens * ROW;
      f4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        const uint4 kf =
            *reinterpret_cast<const uint4*>(s_k + col * ROW + (grp * SPAN + 8 * i) * 2);
        sacc = M::k32(kf, qf[i], sacc);
      }
      // sacc[v] = S^T[token 4*grp + v][query col]; shared tiles are full.
      float x[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) x[v] = sacc[v] * scale_log2;
      float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bm = lane_group4_max(bm);
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);
      float pr[4], ps = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        pr[v] = fast_exp2(x[v] - mn);
        ps += pr[v];
      }
      ps = lane_group4_sum(ps);
      l = l * alpha + ps;
      m = mn;
      acc *= alpha;
      if (pv_wave) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          hi[v] = E::round(pr[v]);
          lo[v] = E::round(pr[v] - M::widen(hi[v]));
        }
        const uint2 bhi = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
        const uint2 blo = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
        const uint8_t* vp = s_v + (4 * grp) * ROW + (16 * wave + col) * 2;
        const uint32_t a0 = *reinterpret_cast<const uint16_t*>(vp);
        const uint32_t a1 = *reinterpret_cast<const uint16_t*>(vp + ROW);
        const uint32_t a2 = *reinterpret_cast<const uint16_t*>(vp + 2 * ROW);
        const uint32_t a3 = *reinterpret_cast<const uint16_t*>(vp + 3 * ROW);
        const uint2 av = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
        acc = M::k16(av, bhi, acc);
        acc = M::k16(av, blo, acc);
      }
    }
    // acc[v] = O^T[dim 16*wave + 4*grp + v][query col], unnormalised
    if (q_ok) {
      const size_t pi = ((size_t)sq * H + h) * num_parts + chunk;
      const float inv = 1.f / l;
      if (pv_wave)
        *reinterpret_cast<float4*>(ws_o + pi * D + 16 * wave + 4 * grp) =
            make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
      if (wave == 0 && grp == 0) {
        ws_ml[pi * 2] = m;
        ws_ml[pi * 2 + 1] = l;
      }
    }
    // The next query tile's first store goes to buffer 0, which this query
    // tile's last even token tile may still be reading: wait for every wave.
    __syncthreads();
  }
}

// The grouped call's main launch: workgroups [0, tail_wgs) run tail partitions
// exactly as the partition kernel does in TAIL mode; the rest run shared-prefix
// units (head fastest, then chunk, then group). Both kinds share one grid, so
// they overlap on the machine; the tails (several blocks per sequence and head
// group) are dispatched first and the short shared units fill in behind them.
template <typename T, int D, int PT, int BS>
__global__ void __launch_bounds__(kGroupedWaves * 64, 8)
decode_grouped_kernel(float* __restrict__ ws_ml, float* __restrict__ ws_o,
                      const uint16_t* __restrict__ query, const uint16_t* __restrict__ key_cache,
                      const uint16_t* __restrict__ value_cache,
                      const int32_t* __restrict__ block_tables,
                      const int32_t* __restrict__ context_lens,
                      const int32_t* __restrict__ group_start,
                      const int32_t* __restrict__ shared_blocks, int num_groups, int num_seqs,
                      int num_heads, int max_blocks, int num_parts, int chunk_slots,
                      int tail_wgs, float scale_log2, int32_t* __restrict__ seq_tok0) {
  constexpr int kLds = shared_lds_bytes<D>() > partition_lds_bytes<D>() ? shared_lds_bytes<D>()
                                                                         : partition_lds_bytes<D>();
  __shared__ __align__(16) uint8_t lds[kLds];
  if ((int)blockIdx.x < tail_wgs) {
    partition_body<T, D, PT, BS, true>(blockIdx.x, nullptr, ws_ml, ws_o, query, key_cache,
                                   value_cache, block_tables, context_lens, num_seqs, num_heads,
                                   max_blocks, num_parts, scale_log2, group_start, shared_blocks,
                                   num_groups, chunk_slots, seq_tok0, lds);
  } else {
    const int u = blockIdx.x - tail_wgs;
    const int h = u % num_heads;
    const int gc = u / num_heads;
    shared_unit<T, D, BS>(gc / chunk_slots, gc % chunk_slots, h, ws_ml, ws_o, query, key_cache,
                      value_cache, block_tables, group_start, shared_blocks, num_heads,
                      max_blocks, num_parts, scale_log2, lds);
  }
}

namespace {
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D, int PT, int BS>
hipError_t grouped_t(const DecodeArgs& a, hipStream_t st) {
  constexpr int HG = 64 / (D / 8);
  const int chunk_slots = a.slot_base;  // shared chunks occupy slots [0, slot_base)
  const long shared_wgs = (long)a.num_groups * chunk_slots * a.num_heads;
  const long head_groups = (a.num_heads + HG - 1) / HG;
  const long tail_wgs = (long)a.num_seqs * head_groups * a.tail_parts;
  hipLaunchKernelGGL((decode_grouped_kernel<T, D, PT, BS>), dim3((unsigned)(shared_wgs + tail_wgs)),
                     dim3(kGroupedWaves * 64), 0, st, a.ws_ml, a.ws_o,
                     static_cast<const uint16_t*>(a.query),
                     static_cast<const uint16_t*>(a.key_cache),
                     static_cast<const uint16_t*>(a.value_cache), a.block_tables, a.context_lens,
                     a.group_start, a.shared_blocks, a.num_groups, a.num_seqs, a.num_heads,
                     a.max_blocks_per_seq, a.num_parts, chunk_slots, (int)tail_wgs,
                     a.scale * kLog2e, a.ws_seq);
  return hipGetLastError();
}

template <typename T, int D, int BS>
hipError_t grouped_b(const DecodeArgs& a, hipStream_t st) {
  return a.part_tokens == 256 ? grouped_t<T, D, 256, BS>(a, st) : grouped_t<T, D, 512, BS>(a, st);
}

template <typename T, int D>
hipError_t grouped_d(const DecodeArgs& a, hipStream_t st) {
  if (a.block_size == 8) return grouped_b<T, D, 8>(a, st);
  if (a.block_size == 32) return grouped_b<T, D, 32>(a, st);
  return grouped_b<T, D, 16>(a, st);
}
}  // namespace

hipError_t launch_decode_grouped(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 0) return a.head_dim == 64 ? grouped_d<F16, 64>(a, st) : grouped_d<F16, 128>(a, st);
  return a.head_dim == 64 ? grouped_d<BF16, 64>(a, st) : grouped_d<BF16, 128>(a, st);
}

}  // namespace pkv
