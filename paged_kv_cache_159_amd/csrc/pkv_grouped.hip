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

// Heads per shared-prefix unit: PKV_SHARED_ROW_BYTES / (2 D), so one token
// row of the unit's heads is that many contiguous bytes of K (or V); a single
// head's 256-byte slices at the pool's token stride stream far slower from
// HBM. The waves split the heads, then each head's output dims.
#ifndef PKV_SHARED_ROW_BYTES
#define PKV_SHARED_ROW_BYTES 512
#endif
template <int D>
constexpr int shared_heads() { return PKV_SHARED_ROW_BYTES / (2 * D); }

// LDS bytes of one shared-prefix unit: K and V rows of its heads for one tile,
// rows padded by 16 bytes to spread LDS banks.
template <int D>
constexpr int shared_row_bytes() { return 2 * D + 16; }
template <int D>
constexpr int shared_lds_bytes() { return 2 * shared_heads<D>() * kTileTokens * shared_row_bytes<D>(); }

// One shared-prefix unit (group g, chunk of kSharedChunkTiles shared tiles,
// head group hg of shared_heads<D>() heads) on an 8-wave workgroup over
// blocks of BS tokens. The chunk's tiles stream through one LDS tile buffer:
// each thread holds its four 16-byte pieces of the next tile in registers
// while the waves compute on the current one (two barriers per tile). Wave w
// takes head w / (8 / HU) of the group: S^T = K Q^T for that head (the few
// MFMAs are repeated by the head's other wave) and 64 output dims of
// O^T = V^T P^T. Groups larger than 16 run the chunk once per 16-query tile
// (the re-reads hit L2).
template <typename T, int D, int BS>
__device__ __forceinline__ void shared_unit(
    int g, int chunk, int hg, float* __restrict__ ws_ml, float* __restrict__ ws_o,
    const uint16_t* __restrict__ query, const uint16_t* __restrict__ key_cache,
    const uint16_t* __restrict__ value_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ group_start, const int32_t* __restrict__ shared_blocks,
    int H, int max_blocks, int num_parts, float scale_log2, uint8_t* lds) {
  using E = Elem<T>;
  using M = Mfma<T>;
  constexpr int HU = shared_heads<D>();
  constexpr int WPH = kGroupedWaves / HU;      // waves per head
  constexpr int NQK = D / 32;                  // S MFMAs (32 dims each)
  constexpr int NPV = D / 16 / WPH;            // 16-dim output chunks per wave (4)
  constexpr int SPAN = D / 4;                  // dims per lane group in the S contraction
  constexpr int ROW = shared_row_bytes<D>();
  constexpr int THREADS = kGroupedWaves * 64;
  constexpr int ROW_PIECES = HU * D / 8;       // 16-byte pieces of one token row of the heads
  constexpr int TILE_PIECES = 2 * kTileTokens * ROW_PIECES;   // K and V of one tile
  constexpr int PPT = TILE_PIECES / THREADS;   // pieces per thread per tile
  constexpr int V_OFF = HU * kTileTokens * ROW;  // LDS byte offset of the V rows
  static_assert(64 % ROW_PIECES == 0 && PPT * THREADS == TILE_PIECES,
                "whole row segments per wave load");
  static_assert(WPH * HU == kGroupedWaves && NPV * 16 * WPH == D, "waves split heads and dims");
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
  const int hw = wave / WPH;                   // this wave's head within the unit
  const int h = hg * HU + hw;
  const bool head_ok = h < H;                  // wave-uniform
  const int dim0 = (wave % WPH) * (NPV * 16);  // first output dim of this wave

  // This thread's pieces of a tile: piece e = threadIdx.x % ROW_PIECES of the
  // row segment (head e / (D / 8), column e % (D / 8)) in token rows
  // r_j = threadIdx.x / ROW_PIECES + j * RSTEP, j < RPT, of both K and V.
  // Token t of the prefix is at slot block_table[t / BS] * BS + t % BS, whose
  // row starts at byte slot * kv_dim * 2; the unit's heads start at hg * HU * D.
  constexpr int RPT = PPT / 2;                 // token rows per thread per tile
  constexpr int RSTEP = THREADS / ROW_PIECES;  // rows covered by one pass of the threads
  static_assert(RPT * RSTEP == kTileTokens, "the threads cover the tile's rows");
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 pk[RPT], pv[RPT];
  const int e = threadIdx.x % ROW_PIECES;
  const int r0 = threadIdx.x / ROW_PIECES;
  const bool piece_ok = hg * HU + e / (D / 8) < H;
  const char* kbase = reinterpret_cast<const char*>(key_cache + (size_t)hg * HU * D);
  const char* vbase = reinterpret_cast<const char*>(value_cache + (size_t)hg * HU * D);
  const size_t row_bytes = (size_t)kv_dim * sizeof(uint16_t);
  auto load_tile = [&](int b) {
    const int tb = t0_chunk + b * kTileTokens;   // a multiple of 16
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int t = tb + r0 + j * RSTEP;
      // At block sizes >= 16 the whole tile is in the block of tb.
      const int32_t phys = bt[(BS >= kTileTokens ? tb : t) / BS];
      const size_t off = ((size_t)phys * BS + (t % BS)) * row_bytes + e * 16;
      if (piece_ok) {
        pk[j] = *reinterpret_cast<const u32x4*>(kbase + off);
        pv[j] = *reinterpret_cast<const u32x4*>(vbase + off);
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int at = ((e / (D / 8)) * kTileTokens + r0 + j * RSTEP) * ROW + (e % (D / 8)) * 16;
      if (piece_ok) {
        *reinterpret_cast<u32x4*>(lds + at) = pk[j];
        *reinterpret_cast<u32x4*>(lds + V_OFF + at) = pv[j];
      }
    }
  };
  const uint8_t* s_k = lds + hw * kTileTokens * ROW;
  const uint8_t* s_v = lds + V_OFF + hw * kTileTokens * ROW;

  for (int t0 = s0; t0 < s1; t0 += kQueryTile) {
    const int sq = t0 + col;
    const bool q_ok = sq < s1 && head_ok;
    u32x4 qf[NQK];
#pragma unroll
    for (int i = 0; i < NQK; ++i)
      qf[i] = q_ok ? *reinterpret_cast<const u32x4*>(query + ((size_t)sq * H + h) * D +
                                                     grp * SPAN + 8 * i)
                   : u32x4{0u, 0u, 0u, 0u};
    f4_t acc[NPV];
#pragma unroll
    for (int c = 0; c < NPV; ++c) acc[c] = f4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;
    load_tile(0);
    for (int b = 0; b < nt; ++b) {
      // Every wave is done with the buffer's previous tile (and, at b = 0,
      // with the previous query tile's last one).
      __syncthreads();
      store_tile();
      __syncthreads();
      if (b + 1 < nt) load_tile(b + 1);
      f4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        const uint4 kf =
            *reinterpret_cast<const uint4*>(s_k + col * ROW + (grp * SPAN + 8 * i) * 2);
        sacc = M::k32(kf, __builtin_bit_cast(uint4, qf[i]), sacc);
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
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        hi[v] = E::round(pr[v]);
        lo[v] = E::round(pr[v] - M::widen(hi[v]));
      }
      const uint2 bhi = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
      const uint2 blo = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
#pragma unroll
      for (int c = 0; c < NPV; ++c) {
        const uint8_t* vp = s_v + (4 * grp) * ROW + (dim0 + 16 * c + col) * 2;
        const uint32_t a0 = *reinterpret_cast<const uint16_t*>(vp);
        const uint32_t a1 = *reinterpret_cast<const uint16_t*>(vp + ROW);
        const uint32_t a2 = *reinterpret_cast<const uint16_t*>(vp + 2 * ROW);
        const uint32_t a3 = *reinterpret_cast<const uint16_t*>(vp + 3 * ROW);
        const uint2 av = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
        acc[c] = M::k16(av, bhi, acc[c] * alpha);
        acc[c] = M::k16(av, blo, acc[c]);
      }
    }
    // acc[c][v] = O^T[dim dim0 + 16c + 4*grp + v][query col], unnormalised
    if (q_ok) {
      const size_t pi = ((size_t)sq * H + h) * num_parts + chunk;
      const float inv = 1.f / l;
#pragma unroll
      for (int c = 0; c < NPV; ++c)
        *reinterpret_cast<float4*>(ws_o + pi * D + dim0 + 16 * c + 4 * grp) =
            make_float4(acc[c][0] * inv, acc[c][1] * inv, acc[c][2] * inv, acc[c][3] * inv);
      if (dim0 == 0 && grp == 0) {
        ws_ml[pi * 2] = m;
        ws_ml[pi * 2 + 1] = l;
      }
    }
  }
}

// The grouped call's main launch: workgroups [0, tail_wgs) run tail partitions
// exactly as the partition kernel does in TAIL mode; the rest run shared-prefix
// units (head fastest, then chunk, then group). Both kinds share one grid, so
// they overlap on the machine; the tails (several blocks per sequence and head
// group) are dispatched first and the short shared units fill in behind them.
template <typename T, int D, int PT, int BS>
//
// Registers: the budget of 6 waves per SIMD (up to 80). Head size 128 then
// takes ~70 (7 waves per SIMD, 3 workgroups per CU); the 64 of 8 waves per
// SIMD made the shared-prefix units spill, and the shared-prefix workload
// ran ~5% slower with 4 workgroups per CU than with 3 (with 2, the same).
__global__ void __launch_bounds__(kGroupedWaves * 64, 6)
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
    const int head_groups = (num_heads + shared_heads<D>() - 1) / shared_heads<D>();
    const int u = blockIdx.x - tail_wgs;
    const int hg = u % head_groups;
    const int gc = u / head_groups;
    shared_unit<T, D, BS>(gc / chunk_slots, gc % chunk_slots, hg, ws_ml, ws_o, query, key_cache,
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
  constexpr int HU = shared_heads<D>();
  const long shared_wgs = (long)a.num_groups * chunk_slots * ((a.num_heads + HU - 1) / HU);
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
