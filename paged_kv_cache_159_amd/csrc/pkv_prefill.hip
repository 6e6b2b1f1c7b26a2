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
// through the block table (any block size); one barrier per stage. At head
// size 128 the rows go from global memory straight into a ring of four LDS
// buffers (global_load_lds_dwordx4; the next three stages arrive while the
// waves compute on the current one), K and V both row-major with
// XOR-swizzled 16-byte pieces, and P.V reads its V^T operands with gfx950's
// transposing LDS read (ds_read_b64_tr_b16). Other head sizes stage through
// registers into two buffers: K rows padded by 16 bytes, V transposed into
// V^T[dim][key] element by element.
//
// Arithmetic, per 32 keys and 16 queries:
//   S^T = K Q^T with v_mfma_f32_16x16x32 (A = 16 key rows, B = the queries'
//   rows), two 16-key tiles; the accumulator holds S^T[key 4g+v][query l%16].
//   Causal mask (key position > query position -> -inf; only on steps that
//   reach past the wave's first query), online softmax per query column in
//   the log2 domain against a reference that moves only when a score
//   exceeds it by more than 8 (log2 units): the exponent of a score is one
//   FMA, and each lane tests its own scores against the slack; only a step
//   that moves the reference takes the max across the 4 lane groups
//   (gfx950's row-swap instructions) and rescales.
//   O^T += V^T P^T with one v_mfma_f32_16x16x32 per 16 output dims: its K index
//   8g+e runs over keys 4g+e of the first tile (e < 4) and 16+4g+(e-4) of the
//   second, which is exactly where the two S^T accumulators already hold P^T,
//   so P never moves between lanes; V^T's operand is two 8-byte LDS reads
//   (transposing reads of the row-major V at head size 128).
//   The row sums of the weights come from one more MFMA per tile: the same P
//   operand against all-ones rows (so the denominator sums exactly the
//   weights the numerator used).
//   fp16: P is rounded once to fp16 (11-bit significand). bf16: rounding P to
//   bf16's 8 bits made ~0.1% of outputs miss half an output ulp against the
//   exact result, so P is split into hi + lo bf16 parts and V^T P^T takes
//   two MFMAs per 16 dims.

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
constexpr int kPrefillWaves = 8;
constexpr int kPrefillQW = 2;                                        // 16-row tiles per wave
constexpr int kPrefillRows = 16 * kPrefillQW * kPrefillWaves;        // rows per workgroup
constexpr int kPrefillKeys = 64;                                     // keys per LDS stage
// Bytes of one V^T row: the keys plus padding that keeps the 8-byte operand
// reads of 32 lanes (16 dims x 2 key groups) on distinct LDS banks.
constexpr int kVtRow = kPrefillKeys * 2 + 8;
// Byte offset of key k in V^T row d: groups of 4 keys (one 8-byte MFMA
// operand read) are XOR-swizzled by bits 5..6 of d, so the transposed 2-byte
// stores of a wave (16 column pieces of 8 dims each, 4 keys) fall on distinct
// LDS banks; the 16 lanes of an operand read share d >> 5, hence one swizzle.
__device__ __forceinline__ int vt_key_offset(int d, int k) {
  return ((((k >> 2) ^ ((d >> 5) & 3)) << 2) | (k & 3)) * 2;
}

template <int D>
constexpr int prefill_krow() { return 2 * D + 16; }

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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
  constexpr int NBUF = 2;   // register-staged stages alternate between two buffers
  constexpr bool kPrio = !std::is_same<T, BF16>::value;   // wave priorities (below)
  // Direct staging (head size 128): K and V rows go from global memory
  // straight into LDS (one 16-byte load per lane, lane l landing at the
  // instruction's base + 16 l), unpadded 256-byte rows with XOR-swizzled
  // 16-byte pieces; V stays row-major and P.V operands come from transposing
  // LDS reads. Other head sizes stage through registers into padded K rows
  // and a 2-byte-element V^T.
  constexpr bool kDirect = D == 128;
  constexpr int kDirectRow = 2 * D;                       // 256 bytes
  constexpr int kDirectStage = 2 * kPrefillKeys * kDirectRow;   // K rows, then V rows
  // A ring of four stage buffers: the loads of stages st + 1 .. st + 3 fly
  // while stage st is computed (the kernel's registers allow one workgroup
  // per CU, so its LDS can take 128 KiB). Three buffers measured 1-3% slower
  // (fp16 chunks 373.0 vs 361.0 us, bf16 whole prompts 685.8 vs 665.2 us with
  // the priorities below).
  __shared__ __align__(16) uint8_t s_d0[kDirect ? kDirectStage : 16];
  __shared__ __align__(16) uint8_t s_d1[kDirect ? kDirectStage : 16];
  __shared__ __align__(16) uint8_t s_d2[kDirect ? kDirectStage : 16];
  __shared__ __align__(16) uint8_t s_d3[kDirect ? kDirectStage : 16];
  __shared__ __align__(16) uint8_t s_kbuf[kDirect ? 1 : NBUF][kDirect ? 16 : kPrefillKeys * KROW];
  constexpr int VTROW = kVtRow;
  __shared__ __align__(16) uint8_t s_vtbuf[kDirect ? 1 : NBUF][kDirect ? 16 : D * VTROW];

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
  // m: softmax reference per query row (log2 domain); lsum: the row sums of
  // the weights, accumulated by an MFMA against an all-ones operand (every
  // element of lsum[j] holds lane's query row sum).
  float m[QW];
  f4_t lsum[QW];
#pragma unroll
  for (int j = 0; j < QW; ++j) {
    m[j] = -INFINITY;
    lsum[j] = f4_t{0.f, 0.f, 0.f, 0.f};
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
  // Piece it of this thread: q = threadIdx.x + it * THREADS is key row
  // r = q / (D/8) of the stage, 16-byte column piece cc = q % (D/8).
  auto piece_row = [&](int it) { return (int)(threadIdx.x + it * THREADS) / (D / 8); };
  auto piece_col = [&](int it) { return (int)(threadIdx.x + it * THREADS) % (D / 8); };
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
  };

  const int nstages = (nkeys + kPrefillKeys - 1) / kPrefillKeys;
  // Direct staging of stage st into buffer b: wave w issues 4 loads, each 4
  // rows of K or V (64 lanes x 16 bytes). Lane l takes row r = r0 + l / 16 and
  // LDS slot l % 16 of it, i.e. the row's piece (l % 16) ^ swizzle(r): K rows
  // swizzle by r & 15 (16 consecutive rows read one piece column on distinct
  // banks), V rows by 2 (r & 7) (the transposing reads take 8 rows x 2
  // pieces at a time). A 16-lane row segment is one coalesced 256-byte read.
  auto issue_stage = [&](int st, uint8_t* buf) {
    // Table lookups and addresses of all four loads first, then the loads
    // back to back (a lookup between them would wait for the loads before it).
    // Each load takes a wave-uniform 64-bit base (the block's first row of
    // this head, in SGPRs) and a 32-bit per-lane byte offset: against a
    // 64-bit address per lane this frees VGPRs and VALU address arithmetic
    // (fp16 whole prompts 537.4 -> 525.7 us, chunks 379.8 -> 359.7 us; bf16
    // within 1%).
    const uint16_t* sbase[4];
    uint32_t voff[4];
    uint32_t lds_base[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tensor = j >> 1;
      const int r0 = 4 * (wave + 8 * (j & 1));
      const int r = r0 + (lane >> 4);
      const int piece = (lane & 15) ^ (tensor ? 2 * (r & 7) : (r & 15));
      const int kpos = min(st * kPrefillKeys + r, nkeys - 1);
      // The instruction's 4 rows (clamped or not) lie in one block, so its
      // table entry is a scalar load (not a vector load, whose wait would
      // also wait for the stage loads in flight).
      const int32_t phys = bt[min(st * kPrefillKeys + r0, nkeys - 1) / BS];
      sbase[j] = (tensor ? value_cache : key_cache) + (size_t)phys * BS * kv_dim + (size_t)h * D;
      voff[j] = (uint32_t)(((kpos % BS) * kv_dim + piece * 8) * sizeof(uint16_t));
      lds_base[j] = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(
          buf + tensor * kPrefillKeys * kDirectRow + r0 * kDirectRow);
    }
    // global_load_lds_dwordx4 with the wave-uniform LDS base in M0. Written
    // as inline asm so the compiler does not treat the loads as LDS writes
    // that every later LDS read must wait for: the loads go to a buffer the
    // current stage does not read, and the stage loop waits for them itself
    // (s_waitcnt vmcnt, then a barrier) before that buffer is read. Loads
    // unknown to the compiler only make its own vmcnt waits more
    // conservative (vector loads complete in order). m0 (the DMA's LDS
    // address) is set in the same statement and used by nothing else here.
#pragma unroll
    for (int j = 0; j < 4; ++j)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(lds_base[j]), "v"(voff[j]), "s"(sbase[j]) : "memory", "m0");
  };

  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), as the
  // builtin so the compiler's own wait placement sees it.
  constexpr int kWaitVmcnt0 = 0x0F70;
  // s_waitcnt vmcnt(4) / vmcnt(8): all but the last one / two stages' four
  // loads of this wave done.
  constexpr int kWaitVmcnt4 = 0x0F74;
  constexpr int kWaitVmcnt8 = 0x0F78;
  if constexpr (kDirect) {
    // Stage 0 and the query rows first (waited for here, so the compiler
    // knows the query registers are ready and puts no wait of its own in
    // the loop, where it would also wait for the stages in flight).
    issue_stage(0, s_d0);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (nstages > 1) issue_stage(1, s_d1);
    if (nstages > 2) issue_stage(2, s_d2);
    __syncthreads();
  } else {
    load_stage(0);
    store_stage(0);
    __syncthreads();
    if (nstages > 1) load_stage(1);
  }
  for (int st = 0; st < nstages; ++st) {
    const uint8_t* s_k;
    const uint8_t* s_vt;
    if constexpr (kDirect) {
      const int b = st & 3;
      uint8_t* cur = b == 0 ? s_d0 : (b == 1 ? s_d1 : (b == 2 ? s_d2 : s_d3));
      uint8_t* nxt3 = b == 0 ? s_d3 : (b == 1 ? s_d0 : (b == 2 ? s_d1 : s_d2));
      // Stage st + 3's loads go to the buffer stage st - 1 used (every wave
      // finished reading it before the barrier that ended stage st - 1) and
      // fly during the math of this stage and the next two.
      if (st + 3 < nstages) issue_stage(st + 3, nxt3);
      s_k = cur;
      s_vt = cur + kPrefillKeys * kDirectRow;
    } else {
      s_k = s_kbuf[st & 1];
      s_vt = s_vtbuf[st & 1];
    }
    // A wave computes a stage if some of its keys are visible to the wave's
    // rows (a wave past the chunk's end only helps staging). Within a stage
    // both 32-key steps run: a step wholly past the wave's last row is fully
    // masked and adds exact zeros. Skipping it instead (a branch out of the
    // step loop) joined two definitions of the accumulators, and the compiler
    // then copied all 64 accumulator registers twice per stage (~76 moves):
    // the unconditional second step measured 10% faster (fp16 whole prompts
    // 587.6 -> 528.1 us, chunks 405.1 -> 368.1 us; bf16 733.2 -> 690.6 and
    // 505.4 -> 470.6 us).
    if (wrow0 < qn && st * kPrefillKeys <= wave_last_pos) {
#pragma unroll
    for (int kp = 0; kp < kPrefillKeys / 32; ++kp) {
      const int kbase = st * kPrefillKeys + kp * 32;     // first key of this 32-key step
      const int lk = kp * 32;
      // One 32-key step for all QW query tiles, as one branch-free block: the
      // S^T products of every tile first, then the softmax updates, then the
      // P.V products, so one tile's VALU work can overlap another's MFMAs.
      // Rows past the chunk's end (zero queries) are computed and dropped at
      // the store. Only steps reaching past the wave's first query position
      // take the causal mask (instantiated apart, so the others skip it).
      auto step = [&](auto mask_tag) {
        constexpr bool kMask = decltype(mask_tag)::value;
        // Wave priority (fp16): the softmax (a chain of dependent VALU work)
        // runs at priority 1 and the MFMA blocks at 0, so on a SIMD the wave
        // in its softmax wins issue slots while the other wave's MFMAs run.
        // bf16, whose split P doubles the P.V MFMAs, ran 3-4% faster without
        // the priorities; fp16 1-2% slower. Set before the K reads, so that
        // the reads and the MFMAs form one scheduling region (below).
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
        uint4 ka[NK], kb[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          if constexpr (kDirect) {
            // rows lk + col and lk + 16 + col both swizzle by col
            const int sw = 16 * ((4 * i + grp) ^ col);
            ka[i] = *reinterpret_cast<const uint4*>(s_k + (lk + col) * kDirectRow + sw);
            kb[i] = *reinterpret_cast<const uint4*>(s_k + (lk + 16 + col) * kDirectRow + sw);
          } else {
            ka[i] = *reinterpret_cast<const uint4*>(s_k + (lk + col) * KROW + (32 * i + 8 * grp) * 2);
            kb[i] = *reinterpret_cast<const uint4*>(s_k + (lk + 16 + col) * KROW +
                                                    (32 * i + 8 * grp) * 2);
          }
        }
        // S^T by K piece (32 dims) across the query tiles; each tile's sums
        // still run over the pieces in order. The schedule below issues the
        // reads of pieces 0 and 1, then each piece's MFMAs with the reads of
        // the piece two ahead, so only the first reads are waited for before
        // the matrix cores start (all eight reads first, then a wait for all
        // of them: fp16 whole prompts 1-2% slower on three boxes).
        f4_t sa[QW], sb[QW];
#pragma unroll
        for (int j = 0; j < QW; ++j) {
          sa[j] = f4_t{0.f, 0.f, 0.f, 0.f};
          sb[j] = f4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < NK; ++i) {
#pragma unroll
          for (int j = 0; j < QW; ++j) {
            sa[j] = M::k32(ka[i], qf[j][i], sa[j]);
            sb[j] = M::k32(kb[i], qf[j][i], sb[j]);
          }
        }
        // Scheduling groups (mask 0x100: LDS reads, 0x008: MFMA).
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < NK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2 * QW, 0);
          if (i + 2 < NK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        constexpr bool kSplit = std::is_same<T, BF16>::value;
        uint4 bhi[QW], blo[QW];
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
        // Exponents against the current reference: y = s * scale - m in the
        // log2 domain, one FMA per score (masked keys -inf). The reference
        // stays unless some score of the step exceeds it by more than
        // kRefSlack, which each lane tests on its own 8 scores (no cross-lane
        // max in the common case). Every weight is then at most 2^kRefSlack,
        // well inside the 16-bit range; softmax does not depend on the
        // reference.
        float y[QW][8];
        bool over = false;
#pragma unroll
        for (int j = 0; j < QW; ++j) {
          const float nm = -m[j];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            y[j][v] = __builtin_fmaf(sa[j][v], scale_log2, nm);
            y[j][4 + v] = __builtin_fmaf(sb[j][v], scale_log2, nm);
          }
          if constexpr (kMask) {
            const int qpos = first + wrow0 + 16 * j + col;   // this lane's query position
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              if (kbase + 4 * grp + v > qpos) y[j][v] = -INFINITY;
              if (kbase + 16 + 4 * grp + v > qpos) y[j][4 + v] = -INFINITY;
            }
          }
          float lm = y[j][0];
#pragma unroll
          for (int e = 1; e < 8; ++e) lm = fmaxf(lm, y[j][e]);
          over |= lm > kRefSlack;
        }
        // Weights and the 16-bit P operands from y.
        auto weights = [&]() {
#pragma unroll
          for (int j = 0; j < QW; ++j) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = fast_exp2(y[j][e]);
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
        };
        // O^T += V^T P^T. Written once and placed on both sides of the rare
        // rescale below, so that each side ends in the MFMAs that update the
        // accumulators in place (a rescale joining a shared P.V block made
        // the compiler copy all 64 accumulator registers every step).
        auto pv_block = [&]() {
          if constexpr (kPrio) __builtin_amdgcn_s_setprio(0);
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int d = 16 * c + col;
            const uint8_t* vrow = s_vt + d * VTROW;
            uint4 a;
            if constexpr (kDirect) {
              // Two transposing reads: in each 16-lane group, lane 4k + q points
              // at dims 16c + 4q .. + 3 of key row lk + 16 half + 4 grp + k, and
              // lane L receives dim 16c + L of those 4 keys: A[dim][8 grp + e].
              const int k4 = (lane & 15) >> 2, q = lane & 3;
              const int rr = 4 * grp + k4;                   // row within the 16-key tile
              const int off = 16 * ((2 * c + (q >> 1)) ^ (2 * (rr & 7))) + 8 * (q & 1);
              typedef short s4_lds __attribute__((ext_vector_type(4)));
              typedef __attribute__((address_space(3))) s4_lds lds_s4;
              const s4_lds t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_s4*)(s_vt + (lk + rr) * kDirectRow + off));
              const s4_lds t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (lds_s4*)(s_vt + (lk + 16 + rr) * kDirectRow + off));
              const uint2 u0 = __builtin_bit_cast(uint2, t0), u1 = __builtin_bit_cast(uint2, t1);
              a = make_uint4(u0.x, u0.y, u1.x, u1.y);
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
          // Row sums: the same P operands against all-ones rows.
          constexpr uint32_t kOne2 = std::is_same<T, BF16>::value ? 0x3F803F80u : 0x3C003C00u;
          const uint4 ones = make_uint4(kOne2, kOne2, kOne2, kOne2);
#pragma unroll
          for (int j = 0; j < QW; ++j) {
            f4_t t = M::k32(ones, bhi[j], lsum[j]);
            if constexpr (kSplit) t = M::k32(ones, blo[j], t);
            lsum[j] = t;
          }
        };
        if (__builtin_expect(__any(over), 0)) {          // wave-uniform, rare
          // Some score exceeds the reference by more than the slack (or this
          // is the first step, whose reference is -inf): raise the reference
          // of each query whose step max exceeds it by more than kRefSlack to
          // that max, rescale its sums and accumulators, recompute y. The
          // first step holds key 0, which every query sees, so the reference
          // is finite from then on; a step whose keys are all masked for a
          // query keeps it.
#pragma unroll
          for (int j = 0; j < QW; ++j) {
            float x[8];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              x[v] = sa[j][v] * scale_log2;
              x[4 + v] = sb[j][v] * scale_log2;
            }
            if constexpr (kMask) {
              const int qpos = first + wrow0 + 16 * j + col;
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
            const float mnew = (bm > m[j] + kRefSlack) ? bm : m[j];
            const float alpha = fast_exp2(m[j] - mnew);    // exactly 1 where kept
            lsum[j] *= alpha;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[j][c] *= alpha;
            m[j] = mnew;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[j][e] = x[e] - mnew;
          }
          weights();
          pv_block();
        } else {
          weights();
          pv_block();
        }
        if constexpr (kPrio) __builtin_amdgcn_s_setprio(1);
      };
      if (kbase + 31 > first + wrow0)
        step(std::true_type{});
      else
        step(std::false_type{});
    }
    }
    if constexpr (kDirect) {
      // Stage st + 1 has landed once this wave's loads up to it are done
      // (only those of stages st + 2 and st + 3 may still fly: loads complete
      // in order) and every wave has passed the barrier.
      if (st + 3 < nstages)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt8);
      else if (st + 2 < nstages)
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt4);
      else
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
      __syncthreads();
    } else {
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
    const float inv = 1.f / lsum[j][0];
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
