// Multi-token (prefill / chunked-prefill) paged attention for gfx950 on the
// MFMA matrix cores.
//
// Pages: a prompt's KV goes into pages allocated in one go at prefill ([P1]
// "3.3 页面级显存管理" §3.3.2 "动态页面分配机制": a 320-token prompt takes 20
// pages), read back through the block table with the same translation as
// decode ([P3] "3.1 PagedAttention的核心原理" §3.1.3); prefix pages may be shared
// at prefill as at decode ([P2] "Copy-on-Write共享解码的显存优化原理"). The pages
// give no attention formula; the reading taken is causal scaled dot-product
// attention: sequence s's chunk of q_len new tokens sits at positions
// ctx - q_len .. ctx - 1 (its K/V already written to the cache), and query i
// attends over tokens 0 .. ctx - q_len + i through the block table. q_len = ctx
// is a whole prompt, q_len < ctx a chunk after a cached prefix.
//
// Work decomposition. One 8-wave workgroup per (sequence, tile of 256 chunk
// rows, head); each wave owns 32 query rows as two 16-column MFMA tiles. Tiles
// are dispatched last-first (the causal work of a tile grows with its
// position). Keys are staged through LDS 64 at a time, gathered row by row
// through the block table (any block size): K row-major (rows padded by 16
// bytes), V transposed (V^T[dim][key]). At head size 128 the transpose runs
// in registers (a 4 x 4 word exchange across lane groups) and each lane
// stores two 16-byte V^T pieces; other head sizes store 2-byte elements. The
// next stage's rows are held in registers while the waves compute on the
// current one, in a second LDS buffer (one barrier per stage).
//
// Arithmetic, per 32 keys and 16 queries:
//   S^T = K Q^T with v_mfma_f32_16x16x32 (A = 16 key rows, B = the queries'
//   rows), two 16-key tiles; the accumulator holds S^T[key 4g+v][query l%16].
//   Causal mask (key position > query position -> -inf; only on steps that
//   reach past the wave's first query), online softmax per query column in
//   the log2 domain (max and sum across the 4 lane groups by gfx950's
//   row-swap instructions), against a reference that moves only when a score
//   exceeds it by more than 2^8, so most steps skip the rescale.
//   O^T += V^T P^T with one v_mfma_f32_16x16x32 per 16 output dims: its K index
//   8g+e runs over keys 4g+e of the first tile (e < 4) and 16+4g+(e-4) of the
//   second, which is exactly where the two S^T accumulators already hold P^T,
//   so P never moves between lanes; V^T's operand is one 16-byte LDS read
//   at head size 128 (the two 4-key groups stored side by side), two 8-byte
//   reads otherwise.
//   fp16: P is rounded once to fp16 (11-bit significand; the sum l stays
//   fp32). bf16: rounding P to bf16's 8 bits made ~0.1% of outputs miss half
//   an output ulp against the exact result, so P is split into hi + lo bf16
//   parts and V^T P^T takes two MFMAs per 16 dims.

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_mfma.h"

namespace pkv {

// Shape measured on MI355X (LLaMA-7B heads, 8 prompts of 1.3k-3.8k tokens):
// 8 waves x 2 query tiles x 64-key stages ~400 TFLOP/s fp16; 4 waves x 2
// tiles (one wave per SIMD at 274 registers) 222; 8 x 1 373; 128-key stages
// 330; the table copied to LDS, or V^T operands read once for both query
// tiles, no gain.
#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
#ifndef PKV_PREFILL_QW
#define PKV_PREFILL_QW 2
#endif
#ifndef PKV_PREFILL_KEYS
#define PKV_PREFILL_KEYS 64
#endif
constexpr int kPrefillWaves = PKV_PREFILL_WAVES;
constexpr int kPrefillQW = PKV_PREFILL_QW;                           // 16-row tiles per wave
constexpr int kPrefillRows = 16 * kPrefillQW * kPrefillWaves;        // rows per workgroup
constexpr int kPrefillKeys = PKV_PREFILL_KEYS;                       // keys per LDS stage
// Bytes of one V^T row: the keys plus padding that keeps the 8-byte operand
// reads of 32 lanes (16 dims x 2 key groups) on distinct LDS banks.
constexpr int kVtRow = kPrefillKeys * 2 + (kPrefillKeys == 64 ? 8 : 16);
#ifndef PKV_VT_SWIZZLE
#define PKV_VT_SWIZZLE 1
#endif
// Byte offset of key k in V^T row d: groups of 4 keys (one 8-byte MFMA
// operand read) are XOR-swizzled by bits 5..6 of d, so the transposed 2-byte
// stores of a wave (16 column pieces of 8 dims each, 4 keys) fall on distinct
// LDS banks; the 16 lanes of an operand read share d >> 5, hence one swizzle.
__device__ __forceinline__ int vt_key_offset(int d, int k) {
  if (PKV_VT_SWIZZLE) return ((((k >> 2) ^ ((d >> 5) & 3)) << 2) | (k & 3)) * 2;
  return k * 2;
}

template <int D>
constexpr int prefill_krow() { return 2 * D + 16; }

// Paired V^T layout (head size 128, 64-key stages, 8 waves). The P.V operand
// of one lane is 8 keys of one dim: keys 4g..4g+3 and 16+4g..16+4g+3 of a
// 32-key step (lane group g). They sit side by side as one 16-byte unit
// u = 4 * step + g of the dim's row, so an operand is one 16-byte read. A row
// is 8 units plus 16 bytes of padding, and unit u of row d is stored at
// u ^ ((d >> 4) & 7). Reads (16 consecutive dims, one unit) and the stores
// below (16 column pieces, one unit) then fall on distinct LDS banks.
constexpr int kPairedVtRow = 8 * 16 + 16;

// 4 x 4 transpose of 32-bit words across the lane groups (lanes l, l + 16,
// l + 32, l + 48): afterwards word k of lane group g is word g of lane group
// k. v_permlane32_swap exchanges the upper half of its first operand with
// the lower half of its second; v_permlane16_swap the odd 16-lane rows of its
// first operand with the even rows of its second.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lane_group_transpose4(u32x4_t& x) {
  const auto a = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto e = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  x = u32x4_t{c[0], c[1], e[0], e[1]};
}

int prefill_rows_per_tile() { return kPrefillRows; }

// Largest log2 gap between a step's max score and the softmax reference that
// keeps the reference (weights then stay at most 2^8).
constexpr float kRefSlack = 8.f;

template <typename T, int D, int BS>
__global__ void __launch_bounds__(kPrefillWaves * 64)
prefill_kernel(uint16_t* __restrict__ out, const uint16_t* __restrict__ query,
               const uint16_t* __restrict__ key_cache, const uint16_t* __restrict__ value_cache,
               const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens,
               const int32_t* __restrict__ query_start, int num_heads, int max_blocks,
               int q_tiles, float scale_log2) {
  using E = Elem<T>;
  using M = Mfma<T>;
  constexpr int KROW = prefill_krow<D>();
  constexpr int NK = D / 32;                      // S^T MFMAs per 16 keys
  constexpr int NC = D / 16;                      // 16-dim output chunks
  constexpr int QW = kPrefillQW;
  constexpr int THREADS = kPrefillWaves * 64;
  constexpr int PIECES = kPrefillKeys * D / 8;    // 16-byte pieces of K (or V) per stage
  constexpr int PER_THREAD = PIECES / THREADS;
  static_assert(PIECES % THREADS == 0, "whole pieces per thread");
#ifndef PKV_PREFILL_DBUF
#define PKV_PREFILL_DBUF 1
#endif
  constexpr int NBUF = PKV_PREFILL_DBUF ? 2 : 1;
  __shared__ __align__(16) uint8_t s_kbuf[NBUF][kPrefillKeys * KROW];
  constexpr bool kPaired = D == 128 && kPrefillKeys == 64 && kPrefillWaves == 8;
  constexpr int VTROW = kPaired ? kPairedVtRow : kVtRow;
  __shared__ __align__(16) uint8_t s_vtbuf[NBUF][D * VTROW];

  const int H = num_heads;
  const int h = blockIdx.x % H;
  const int tile = q_tiles - 1 - (int)(blockIdx.x / H);
  const int s = blockIdx.y;
  const int q0 = query_start[s];
  const int qn = query_start[s + 1] - q0;
  if (tile * kPrefillRows >= qn) return;
  const int ctx = context_lens[s];
  const int first = ctx - qn;                     // position of chunk row 0
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int wrow0 = tile * kPrefillRows + wave * 16 * QW;   // this wave's first chunk row
  const int wend = min(wrow0 + 16 * QW, qn);
  const int wave_last_pos = first + wend - 1;               // meaningful when wrow0 < qn
  const int nkeys = first + min(tile * kPrefillRows + kPrefillRows, qn);  // keys [0, nkeys)

  uint4 qf[QW][NK];
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    const int row = wrow0 + 16 * j + col;
#pragma unroll
    for (int i = 0; i < NK; ++i)
      qf[j][i] = row < qn ? *reinterpret_cast<const uint4*>(
                                query + ((size_t)(q0 + row) * H + h) * D + 32 * i + 8 * grp)
                          : make_uint4(0, 0, 0, 0);
  }
  f4_t acc[QW][NC];
  float m[QW], l[QW];
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[j][c] = f4_t{0.f, 0.f, 0.f, 0.f};
  }

  const size_t kv_dim = (size_t)H * D;
  const int32_t* bt = block_tables + (size_t)s * max_blocks;
  // Piece it of this thread: key row r = q / (D/8) of the stage, 16-byte
  // column cc = q % (D/8), q = threadIdx.x + it * THREADS. Keys past the
  // last needed one re-read it (valid, a cache hit); the mask drops them.
  // Native 4-lane vectors: the compiler keeps them in registers across the
  // stage loop (HIP's struct uint4 here ended up in scratch memory, which made
  // every stage wait for its K loads as soon as they were issued).
  typedef u32x4_t u32x4;
  u32x4 pk[PER_THREAD], pv[PER_THREAD];
  // Piece it of this thread: key row r of the stage, 16-byte column piece cc.
  // Plain layout: q = threadIdx.x + it * THREADS, r = q / (D/8), cc = q % (D/8).
  // Paired layout: wave w reads key groups 4 * kg .. 4 * kg + 3 with
  // kg = 8 * (w / 4) + w % 4 + 4 * it (the two halves of unit w), lane group g
  // the key 4 * kg + g, and the 16 lanes of a group the pieces of that key
  // row in the order cc = 2 * (l % 8) + (l / 8) % 2.
  auto piece_row = [&](int it) {
    if constexpr (kPaired)
      return 4 * (8 * (wave >> 2) + (wave & 3) + 4 * it) + (lane >> 4);
    else
      return (int)(threadIdx.x + it * THREADS) / (D / 8);
  };
  auto piece_col = [&](int it) {
    if constexpr (kPaired)
      return ((lane & 7) << 1) | ((lane >> 3) & 1);
    else
      return (int)(threadIdx.x + it * THREADS) % (D / 8);
  };
  // Keys past the last needed one re-read it (valid, a cache hit); the mask
  // drops them.
  auto load_stage = [&](int st) {
#pragma unroll
    for (int it = 0; it < PER_THREAD; ++it) {
      const int r = piece_row(it);
      const int cc = piece_col(it);
      const int kpos = min(st * kPrefillKeys + r, nkeys - 1);
      const size_t slot = (size_t)bt[kpos / BS] * BS + (kpos % BS);
      const size_t off = slot * kv_dim + (size_t)h * D + cc * 8;
      pk[it] = *reinterpret_cast<const u32x4*>(key_cache + off);
      pv[it] = *reinterpret_cast<const u32x4*>(value_cache + off);
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* s_k = s_kbuf[buf];
    uint8_t* s_vt = s_vtbuf[buf];
#pragma unroll
    for (int it = 0; it < PER_THREAD; ++it)
      *reinterpret_cast<u32x4*>(s_k + piece_row(it) * KROW + piece_col(it) * 16) = pk[it];
    if constexpr (kPaired) {
      // After the transpose, word k of piece it holds dims (2g, 2g + 1) of
      // the column piece for key 4 * kg + k: dim 8 cc + 2g gets the low
      // halves, dim 8 cc + 2g + 1 the high halves, 8 keys each (one unit).
      u32x4 x0 = pv[0], x1 = pv[1];
      lane_group_transpose4(x0);
      lane_group_transpose4(x1);
      const int cc = piece_col(0);
      const int d = cc * 8 + 2 * (lane >> 4);
      const int unit = 16 * (wave ^ ((d >> 4) & 7));     // d and d + 1 share d >> 4
      const u32x4 lo = {(x0[0] & 0xffffu) | (x0[1] << 16), (x0[2] & 0xffffu) | (x0[3] << 16),
                        (x1[0] & 0xffffu) | (x1[1] << 16), (x1[2] & 0xffffu) | (x1[3] << 16)};
      const u32x4 hi = {(x0[0] >> 16) | (x0[1] & 0xffff0000u), (x0[2] >> 16) | (x0[3] & 0xffff0000u),
                        (x1[0] >> 16) | (x1[1] & 0xffff0000u), (x1[2] >> 16) | (x1[3] & 0xffff0000u)};
      *reinterpret_cast<u32x4*>(s_vt + d * VTROW + unit) = lo;
      *reinterpret_cast<u32x4*>(s_vt + (d + 1) * VTROW + unit) = hi;
    } else {
#pragma unroll
      for (int it = 0; it < PER_THREAD; ++it) {
        const int r = piece_row(it);
        const int cc = piece_col(it);
        const u32x4 w = pv[it];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint16_t*>(s_vt + (cc * 8 + e) * VTROW +
                                       vt_key_offset(cc * 8 + e, r)) =
              (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
      }
    }
  };

  const int nstages = (nkeys + kPrefillKeys - 1) / kPrefillKeys;
  load_stage(0);
  if constexpr (NBUF == 2) {
    store_stage(0);
    __syncthreads();
    if (nstages > 1) load_stage(1);
  }
  for (int st = 0; st < nstages; ++st) {
    if constexpr (NBUF == 1) {
      __syncthreads();                // every wave is done with the previous stage
      store_stage(0);
      __syncthreads();
      if (st + 1 < nstages) load_stage(st + 1);
    }
    const uint8_t* s_k = s_kbuf[NBUF == 2 ? (st & 1) : 0];
    const uint8_t* s_vt = s_vtbuf[NBUF == 2 ? (st & 1) : 0];
    if (wrow0 < qn) {                 // a wave past the chunk's end only helps staging
#pragma unroll
    for (int kp = 0; kp < kPrefillKeys / 32; ++kp) {
      const int kbase = st * kPrefillKeys + kp * 32;     // first key of this 32-key step
      if (kbase > wave_last_pos) break;                  // wave-uniform
      const int lk = kp * 32;
      // One 32-key step for all QW query tiles, as one branch-free block: the
      // S^T products of every tile first, then the softmax updates, then the
      // P.V products, so one tile's VALU work can overlap another's MFMAs.
      // Rows past the chunk's end (zero queries) are computed and dropped at
      // the store. Only steps reaching past the wave's first query position
      // take the causal mask (instantiated apart, so the others skip it).
      auto step = [&](auto mask_tag) {
        constexpr bool kMask = decltype(mask_tag)::value;
        uint4 ka[NK], kb[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          ka[i] = *reinterpret_cast<const uint4*>(s_k + (lk + col) * KROW + (32 * i + 8 * grp) * 2);
          kb[i] = *reinterpret_cast<const uint4*>(s_k + (lk + 16 + col) * KROW +
                                                  (32 * i + 8 * grp) * 2);
        }
        // Wave priority: the softmax (a chain of dependent VALU work) runs
        // at priority 1 and the MFMA blocks at 0, so on a SIMD the wave in
        // its softmax wins issue slots while the other wave's MFMAs run.
        __builtin_amdgcn_s_setprio(0);
        f4_t sa[QW], sb[QW];
#pragma unroll
        for (int j = 0; j < QW; ++j) {
          sa[j] = f4_t{0.f, 0.f, 0.f, 0.f};
          sb[j] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < NK; ++i) {
            sa[j] = M::k32(ka[i], qf[j][i], sa[j]);
            sb[j] = M::k32(kb[i], qf[j][i], sb[j]);
          }
        }
        constexpr bool kSplit = std::is_same<T, BF16>::value;
        uint4 bhi[QW], blo[QW];
        float mnew[QW], psum[QW];
        bool moved = false;
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < QW; ++j) {
          // Scaled scores in the log2 domain (products are canonical floats,
          // so the max below needs no quieting of its inputs).
          float x[8];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            x[v] = sa[j][v] * scale_log2;
            x[4 + v] = sb[j][v] * scale_log2;
          }
          if constexpr (kMask) {
            const int qpos = first + wrow0 + 16 * j + col;   // this lane's query position
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              if (kbase + 4 * grp + v > qpos) x[v] = -INFINITY;
              if (kbase + 16 + 4 * grp + v > qpos) x[4 + v] = -INFINITY;
            }
          }
          float bm = x[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) bm = fmaxf(bm, x[e]);
          bm = lane_group4_max(bm);
          // Reference for the weights: raised to the step's max only when
          // that exceeds it by more than kRefSlack (log2 units), so every
          // weight stays at most 2^kRefSlack, well inside the 16-bit range.
          // Softmax does not depend on the reference, and most steps keep
          // it, which skips the rescale of the accumulators below. The first
          // step holds key 0, which every query sees, so the reference is
          // finite from then on; a step whose keys are all masked for a
          // query keeps it.
          mnew[j] = (bm > m[j] + kRefSlack) ? bm : m[j];
          moved |= mnew[j] != m[j];
          const float nm = -mnew[j];
          float p[8], ps = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = fast_exp2(x[e] + nm);
#pragma unroll
          for (int e = 0; e < 8; ++e) ps += p[e];
          psum[j] = lane_group4_sum(ps);
          uint32_t hi[4], lo[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hi[e] = E::pack2(p[2 * e], p[2 * e + 1]);
            if constexpr (kSplit)
              lo[e] = E::pack2(p[2 * e] - M::widen(hi[e] & 0xffffu), p[2 * e + 1] - M::widen(hi[e] >> 16));
          }
          bhi[j] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
          blo[j] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
        }
        if (__builtin_expect(__any(moved), 0)) {         // wave-uniform, rare
#pragma unroll
          for (int j = 0; j < QW; ++j) {
            const float alpha = fast_exp2(m[j] - mnew[j]);  // exactly 1 where kept
            l[j] *= alpha;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[j][c] *= alpha;
          }
        }
#pragma unroll
        for (int j = 0; j < QW; ++j) {
          l[j] += psum[j];
          m[j] = mnew[j];
        }
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int d = 16 * c + col;
          const uint8_t* vrow = s_vt + d * VTROW;
          uint4 a;
          if constexpr (kPaired) {
            a = *reinterpret_cast<const uint4*>(vrow + 16 * ((kp * 4 + grp) ^ (c & 7)));
          } else {
            const uint2 va = *reinterpret_cast<const uint2*>(vrow + vt_key_offset(d, lk + 4 * grp));
            const uint2 vb =
                *reinterpret_cast<const uint2*>(vrow + vt_key_offset(d, lk + 16 + 4 * grp));
            a = make_uint4(va.x, va.y, vb.x, vb.y);
          }
#pragma unroll
          for (int j = 0; j < QW; ++j) {
            f4_t t = M::k32(a, bhi[j], acc[j][c]);
            if constexpr (kSplit) t = M::k32(a, blo[j], t);
            acc[j][c] = t;
          }
        }
        __builtin_amdgcn_s_setprio(1);
      };
      if (kbase + 31 > first + wrow0)
        step(std::true_type{});
      else
        step(std::false_type{});
    }
    }
    if constexpr (NBUF == 2) {
      // The other buffer was last read in stage st - 1; every wave has
      // passed the barrier that ended it.
      if (st + 1 < nstages) store_stage((st + 1) & 1);
      __syncthreads();
      if (st + 2 < nstages) load_stage(st + 2);
    }
  }

  // acc[j][c][v] = O^T[dim 16c + 4g + v][row wrow0 + 16j + l%16], unnormalised
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    const int row = wrow0 + 16 * j + col;
    if (row >= qn) continue;
    const float inv = 1.f / l[j];
    uint16_t* o = out + ((size_t)(q0 + row) * H + h) * D + 4 * grp;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint32_t r0 = E::round(acc[j][c][0] * inv), r1 = E::round(acc[j][c][1] * inv);
      const uint32_t r2 = E::round(acc[j][c][2] * inv), r3 = E::round(acc[j][c][3] * inv);
      *reinterpret_cast<uint2*>(o + 16 * c) = make_uint2(r0 | (r1 << 16), r2 | (r3 << 16));
    }
  }
}

namespace {
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D, int BS>
hipError_t prefill_t(const PrefillArgs& a, hipStream_t st) {
  const int q_tiles = (a.max_query_len + kPrefillRows - 1) / kPrefillRows;
  const dim3 grid((unsigned)(a.num_heads * q_tiles), (unsigned)a.num_seqs);
  hipLaunchKernelGGL((prefill_kernel<T, D, BS>), grid, dim3(kPrefillWaves * 64), 0, st,
                     static_cast<uint16_t*>(a.out), static_cast<const uint16_t*>(a.query),
                     static_cast<const uint16_t*>(a.key_cache),
                     static_cast<const uint16_t*>(a.value_cache), a.block_tables, a.context_lens,
                     a.query_start, a.num_heads, a.max_blocks_per_seq, q_tiles,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t prefill_d(const PrefillArgs& a, hipStream_t st) {
  if (a.block_size == 8) return prefill_t<T, D, 8>(a, st);
  if (a.block_size == 32) return prefill_t<T, D, 32>(a, st);
  return prefill_t<T, D, 16>(a, st);
}
}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.dtype == 0) return a.head_dim == 64 ? prefill_d<F16, 64>(a, st) : prefill_d<F16, 128>(a, st);
  return a.head_dim == 64 ? prefill_d<BF16, 64>(a, st) : prefill_d<BF16, 128>(a, st);
}

}  // namespace pkv
