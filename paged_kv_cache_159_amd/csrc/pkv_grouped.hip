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
// group of heads); up to 16 queries per MFMA tile (larger groups loop over
// tiles).
//   S^T = K Q^T with v_mfma_f32_16x16x32 (M = 16 tokens, N = 16 queries,
//   K = 32 dims per instruction), A operand (lane l: token l%16, 8 dims) read
//   from the K rows staged in LDS, B operand (query l%16) from Q. Lane group
//   q = l/16 covers dims [q*D/4, (q+1)*D/4).
//   The accumulator holds S^T[token 4*(l/16)+v][query l%16] (v < 4): exactly
//   the B-operand layout P^T needs for O^T = V^T P^T with v_mfma_f32_16x16x16
//   (K = 16 tokens), so P never moves between lanes.
//   V^T's A operand wants 4 tokens of one dim per lane: one transposing LDS
//   read (ds_read_b64_tr_b16) from the row-major V rows.
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

// Bytes of one token row of a shared-prefix unit's heads: the unit takes
// kSharedRowBytes / (2 D) heads (2 at D = 128, 4 at D = 64), so one token row
// of its heads is that many contiguous bytes of K (or V); a single head's
// 256-byte slices at the pool's token stride stream far slower from HBM. The
// waves split the heads, then each head's output dims.
constexpr int kSharedRowBytes = 512;
template <int D>
constexpr int shared_heads() { return kSharedRowBytes / (2 * D); }

// LDS of one shared-prefix unit: a ring of kSharedBuffers tile buffers, each
// the K rows then the V rows of the unit's heads for one 16-token tile
// (unpadded 512-byte rows of XOR-swizzled 16-byte pieces).
constexpr int kSharedBuffers = 3;
constexpr int kSharedTileBytes = 2 * kTileTokens * kSharedRowBytes;
constexpr int kSharedLdsBytes = kSharedBuffers * kSharedTileBytes;

// One shared-prefix unit (group g, chunk of kSharedChunkTiles shared tiles,
// head group hg of shared_heads<D>() heads) on an 8-wave workgroup over
// blocks of BS tokens.
// Staging: the tiles go from global memory straight into the LDS ring
// (global_load_lds_dwordx4), two tiles ahead of the one being computed, so a
// unit keeps 32 KiB in flight without staging registers. Wave w loads token
// rows 2w and 2w + 1 of a tile, K and V one instruction each: lane l fills
// slot l % 32 of row r = 2w + l / 32 with the row's piece slot ^ swizzle(r).
// K swizzles by r & 15 (the 16 rows one S^T operand read touches land on
// distinct banks), V by 2 (r & 7) (the transposing reads take 4 rows x 4
// dims per 16 lanes). XOR on the low four bits keeps a piece in its half row.
// Compute: wave w takes head w / (8 / HU) of the unit: S^T = K Q^T for that
// head (the few MFMAs are repeated by the head's other waves) and NPV 16-dim
// chunks of O^T = V^T P^T, whose A operand (4 tokens of one dim per lane) is
// one transposing LDS read (ds_read_b64_tr_b16). Groups larger than 16 run
// the chunk once per 16-query tile (the re-reads hit L2).
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
  constexpr int NPV = D / 16 / WPH;            // 16-dim output chunks per wave
  constexpr int SPAN = D / 4;                  // dims per lane group in the S contraction
  constexpr int HP = D / 8;                    // 16-byte pieces of one head's row
  constexpr int ROWB = kSharedRowBytes;
  constexpr int V_OFF = kTileTokens * ROWB;    // V rows after the K rows of a tile buffer
  static_assert(HU * HP == 32 && 2 * kGroupedWaves == kTileTokens,
                "a wave's load instruction is two whole token rows of the unit");
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
  const size_t kv_dim = (size_t)H * D;
  const int hw = wave / WPH;                   // this wave's head within the unit
  const int h = hg * HU + hw;
  const bool head_ok = h < H;                  // wave-uniform
  const int dim0 = (wave % WPH) * (NPV * 16);  // first output dim of this wave

  // The chunk's table entries (the group's first member's table: the shared
  // entries are the same in all), one per lane, read with v_readlane. A chunk
  // starts on a multiple of 128 tokens, so on a block boundary.
  const int32_t* bt = block_tables + (size_t)s0 * max_blocks;
  const int blk0 = t0_chunk / BS;
  const int nblk = (nt * kTileTokens + BS - 1) / BS;   // <= 16
  const int32_t table_lane = lane < nblk ? bt[blk0 + lane] : 0;
  // This lane's load: row lrow of each tile, the pieces the K and V swizzles
  // put in its slot. Pieces of heads past H (a partial last head group)
  // re-read the unit's first head; nothing reads their slots.
  const int lrow = 2 * wave + (lane >> 5);
  auto piece_elems = [&](int p) {
    return (uint32_t)(hg * HU * D + (hg * HU + p / HP < H ? p : p % HP) * 8);
  };
  const uint32_t k_elem = piece_elems((lane & 31) ^ (lrow & 15));
  const uint32_t v_elem = piece_elems((lane & 31) ^ (2 * (lrow & 7)));
  // byte offsets of this lane's piece from its tile row pair's first row
  const uint32_t k_off = ((uint32_t)(lane >> 5) * (uint32_t)kv_dim + k_elem) * (uint32_t)sizeof(uint16_t);
  const uint32_t v_off = ((uint32_t)(lane >> 5) * (uint32_t)kv_dim + v_elem) * (uint32_t)sizeof(uint16_t);
  auto lds_addr = [](const uint8_t* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(p);
  };
  // Tile b of the chunk into ring buffer buf. Rows 2w and 2w + 1 lie in one
  // block (tiles start on multiples of 16 tokens, blocks hold 8 or more).
  // The loads are inline asm so that the compiler does not treat them as LDS
  // writes every later LDS read must wait for; the loop below waits for them
  // itself (s_waitcnt vmcnt, then a barrier) before a buffer is read. They are
  // non-temporal (nt): each prefix row is read once per launch.
  auto issue_tile = [&](int b, uint8_t* buf) {
    const int tw = t0_chunk + b * kTileTokens + 2 * wave;   // wave-uniform
    const int32_t phys = __builtin_amdgcn_readlane(table_lane, tw / BS - blk0);
    const size_t row = ((size_t)phys * BS + (tw % BS)) * kv_dim;   // wave-uniform
    const uint16_t* kb = key_cache + row;
    const uint16_t* vb = value_cache + row;
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :: "s"(lds_addr(buf + 2 * wave * ROWB)), "v"(k_off), "s"(kb) : "memory", "m0");
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :: "s"(lds_addr(buf + V_OFF + 2 * wave * ROWB)), "v"(v_off), "s"(vb) : "memory", "m0");
  };
  // s_waitcnt vmcnt(n) with expcnt and lgkmcnt left at their maxima.
  constexpr int kWaitVmcnt0 = 0x0F70, kWaitVmcnt2 = 0x0F72;
  // LDS reads of this lane: S^T operand i at row col, piece hw HP + grp SPAN / 8
  // + i; V^T operand of chunk c: lane 4 k4 + q of its 16-lane group points at
  // dims dim0 + 16 c + 4 q .. + 3 of row 4 grp + k4 and receives dim
  // dim0 + 16 c + col of those 4 rows (tokens 4 grp .. 4 grp + 3).
  const int k4 = (lane & 15) >> 2, q4 = lane & 3;
  const int vr = 4 * grp + k4;

  for (int t0 = s0; t0 < s1; t0 += kQueryTile) {
    const int sq = t0 + col;
    const bool q_ok = sq < s1 && head_ok;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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
    issue_tile(0, lds);
    if (nt > 1) issue_tile(1, lds + kSharedTileBytes);
    for (int b = 0; b < nt; ++b) {
      // Tile b has landed once this wave's loads up to it are done (only tile
      // b + 1's two may still fly: loads complete in order) and every wave
      // has passed the barrier.
      if (b + 1 < nt)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt2);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
      // Tile b + 2 goes to the buffer tile b - 1 used; every wave finished
      // reading it before the barrier.
      if (b + 2 < nt) issue_tile(b + 2, lds + ((b + 2) % kSharedBuffers) * kSharedTileBytes);
      const uint8_t* s_k = lds + (b % kSharedBuffers) * kSharedTileBytes;
      const uint8_t* s_v = s_k + V_OFF;
      f4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NQK; ++i) {
        const int p = hw * HP + grp * (SPAN / 8) + i;
        const uint4 kf = *reinterpret_cast<const uint4*>(s_k + col * ROWB + 16 * (p ^ col));
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
        const int p = hw * HP + (dim0 + 16 * c) / 8 + (q4 >> 1);
        typedef short s4_lds __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s4_lds lds_s4;
        const s4_lds t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4*)(s_v + vr * ROWB + 16 * (p ^ (2 * (vr & 7))) + 8 * (q4 & 1)));
        const uint2 av = __builtin_bit_cast(uint2, t);
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
    // The next query tile's first loads overwrite the ring.
    __syncthreads();
  }
}

// The grouped call's main launch: workgroups [0, tail_wgs) run tail partitions
// exactly as the partition kernel does in TAIL mode; the rest run shared-prefix
// units (head fastest, then group, then chunk). Both kinds share one grid, so
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
  constexpr int kLds = kSharedLdsBytes > partition_lds_bytes<D>() ? kSharedLdsBytes
                                                                  : partition_lds_bytes<D>();
  __shared__ __align__(16) uint8_t lds[kLds];
  // Grid order: the first tail partition of every (sequence, head group),
  // then the shared-prefix units, then the later tail partitions (needed only
  // by tails longer than PT tokens). Later partitions placed between the
  // first ones and the shared units held the units back: at the shared-prefix
  // workload (tails of 9-264 tokens) its 1,024 empty workgroups were
  // dispatched first and the units started only at 37 of 66 us.
  const int head_groups = (num_heads + shared_heads<D>() - 1) / shared_heads<D>();
  const int first_wgs = num_seqs * ((num_heads + 64 / (D / 8) - 1) / (64 / (D / 8)));
  const int shared_wgs = num_groups * chunk_slots * head_groups;
  const int wg = blockIdx.x;
  if (wg < first_wgs || wg >= first_wgs + shared_wgs) {
    partition_body<T, D, PT, BS, true>(wg < first_wgs ? wg : wg - shared_wgs, nullptr, ws_ml,
                                       ws_o, query, key_cache, value_cache, block_tables,
                                       context_lens, num_seqs, num_heads, max_blocks, num_parts,
                                       scale_log2, group_start, shared_blocks, num_groups,
                                       chunk_slots, seq_tok0, lds);
  } else {
    // Chunk-major: every group's first chunk, then every group's second, ...
    // so the short last chunks and the empty chunk slots come last.
    const int u = wg - first_wgs;
    const int hg = u % head_groups;
    const int gc = u / head_groups;
    shared_unit<T, D, BS>(gc % num_groups, gc / num_groups, hg, ws_ml, ws_o, query, key_cache,
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
  // tail partitions are always 512 tokens
  return a.part_tokens == 512 ? grouped_t<T, D, 512, BS>(a, st) : hipErrorInvalidValue;
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
