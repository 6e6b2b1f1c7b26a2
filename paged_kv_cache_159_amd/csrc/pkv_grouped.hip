// Grouped decode, first launch: attention of several queries over the prefix
// blocks their sequences share, on the MFMA matrix cores of gfx950.
//
// Pages: sharing a prefix maps several sequences' logical blocks to the same
// physical blocks, with a reference count per block ([P2] "vLLM三大核心技术分页
// 内存与共享解码", "Copy-on-Write共享解码的显存优化原理"; [P1] "3.3 页面级显存管理",
// "Copy-on-Write页面共享机制"; parallel sampling and beam search in [P4]
// "Memory Sharing与写时复制"). A shared block is then read once for all its
// readers instead of once per sequence, and the per-block work becomes a dense
// contraction: Q_group [n x D] against K_block [16 x D] and V_block [16 x D].
//
// One wave per (group, chunk of kSharedChunkBlocks shared blocks, head); up to
// 16 queries per MFMA tile (larger groups loop over tiles).
//   S^T = K Q^T with v_mfma_f32_16x16x32 (M = 16 tokens, N = 16 queries,
//   K = 32 dims per instruction). The K block's rows load straight from HBM in
//   the A-operand layout (lane l: token l%16, 8 dims), Q likewise in the B
//   layout. Lane group q = l/16 covers dims [q*D/4, (q+1)*D/4), so a lane's
//   four loads are one contiguous 64-byte piece of its row.
//   The accumulator holds S^T[token 4*(l/16)+v][query l%16] (v < 4): exactly
//   the B-operand layout P^T needs for O^T = V^T P^T with v_mfma_f32_16x16x16
//   (K = 16 tokens), so P never moves between lanes.
//   V^T's A operand wants 4 tokens of one dim per lane, a transposed read:
//   the block's V rows go through LDS (rows padded to spread banks).
//   P is split into hi + lo 16-bit parts (two MFMAs), so the 16-bit operand
//   costs no accuracy next to the fp32 softmax.
// Each wave writes (max, sum, normalised output) partials for its chunk; the
// merge kernel combines them with the sequences' tail partitions.

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Mfma;

template <> struct Mfma<F16> {
  static __device__ __forceinline__ f4_t qk(uint4 a, uint4 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                  __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4_t pv(uint2 a, uint2 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4_t, a),
                                                 __builtin_bit_cast(h4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float widen(uint32_t x) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)x);
  }
};

template <> struct Mfma<BF16> {
  static __device__ __forceinline__ f4_t qk(uint4 a, uint4 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a),
                                                   __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f4_t pv(uint2 a, uint2 b, f4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4_t, a),
                                                     __builtin_bit_cast(s4_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float widen(uint32_t x) { return __uint_as_float(x << 16); }
};

constexpr int kQueryTile = 16;

template <typename T, int D>
__global__ void __launch_bounds__(64)
decode_shared_kernel(float* __restrict__ ws_ml, float* __restrict__ ws_o,
                     const uint16_t* __restrict__ query, const uint16_t* __restrict__ key_cache,
                     const uint16_t* __restrict__ value_cache,
                     const int32_t* __restrict__ block_tables,
                     const int32_t* __restrict__ group_start,
                     const int32_t* __restrict__ shared_blocks, int num_heads, int max_blocks,
                     int num_parts, int chunk_slots, float scale_log2) {
  using E = Elem<T>;
  using M = Mfma<T>;
  constexpr int NQK = D / 32;        // S MFMAs (32 dims each)
  constexpr int NPV = D / 16;        // O MFMAs (16 dims each)
  constexpr int SPAN = D / 4;        // dims per lane group in the S contraction
  constexpr int VROW = 2 * D + 16;   // padded LDS row of V, bytes
  constexpr int VPIECES = 16 * D / 8;  // 16-byte pieces of one head's V block

  const int H = num_heads;
  const int h = blockIdx.x % H;
  const int gc = blockIdx.x / H;
  const int chunk = gc % chunk_slots;
  const int g = gc / chunk_slots;
  const int sb = shared_blocks[g];
  const int b0 = chunk * kSharedChunkBlocks;
  if (b0 >= sb) return;
  const int nb = min(kSharedChunkBlocks, sb - b0);
  const int s0 = group_start[g];
  const int s1 = group_start[g + 1];
  if (s1 <= s0) return;

  const int lane = threadIdx.x;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const uint32_t kv_dim = (uint32_t)H * D;
  const size_t blk_elems = (size_t)kBlockSize * kv_dim;
  // the shared entries are identical in every member's table: read the first's
  const int32_t* bt = block_tables + (size_t)s0 * max_blocks + b0;
  __shared__ __align__(16) uint8_t s_v[kBlockSize * VROW];

  for (int t0 = s0; t0 < s1; t0 += kQueryTile) {
    const int sq = t0 + col;
    const bool q_ok = sq < s1;
    uint4 qf[NQK];
#pragma unroll
    for (int i = 0; i < NQK; ++i)
      qf[i] = q_ok ? *reinterpret_cast<const uint4*>(query + ((size_t)sq * H + h) * D +
                                                     grp * SPAN + 8 * i)
                   : make_uint4(0, 0, 0, 0);
    f4_t acc[NPV];
#pragma unroll
    for (int j = 0; j < NPV; ++j) acc[j] = f4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    for (int b = 0; b < nb; ++b) {
      const int phys = bt[b];
      const uint16_t* kb = key_cache + (size_t)phys * blk_elems + (size_t)h * D;
      const uint16_t* vb = value_cache + (size_t)phys * blk_elems + (size_t)h * D;
      uint4 kf[NQK];
#pragma unroll
      for (int i = 0; i < NQK; ++i)
        kf[i] = *reinterpret_cast<const uint4*>(kb + (size_t)col * kv_dim + grp * SPAN + 8 * i);
#pragma unroll
      for (int pc = lane; pc < VPIECES; pc += 64) {
        const int r = pc / (D / 8);
        const int cc = pc % (D / 8);
        const uint4 v = *reinterpret_cast<const uint4*>(vb + (size_t)r * kv_dim + cc * 8);
        *reinterpret_cast<uint4*>(s_v + r * VROW + cc * 16) = v;
      }

      f4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NQK; ++i) sacc = M::qk(kf[i], qf[i], sacc);
      // sacc[v] = S^T[token 4*grp + v][query col]; shared blocks are full, so
      // every token is valid and the block maximum is finite.
      float x[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) x[v] = sacc[v] * scale_log2;
      float bm = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(m, bm);
      const float alpha = fast_exp2(m - mn);
      float p[4], ps = 0.f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[v] = fast_exp2(x[v] - mn);
        ps += p[v];
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l = l * alpha + ps;
      m = mn;
#pragma unroll
      for (int j = 0; j < NPV; ++j) acc[j] *= alpha;
      uint32_t hi[4], lo[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        hi[v] = E::round(p[v]);
        lo[v] = E::round(p[v] - M::widen(hi[v]));
      }
      const uint2 bhi = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
      const uint2 blo = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
      __syncthreads();  // V block visible in LDS
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        const uint8_t* vp = s_v + (4 * grp) * VROW + (16 * j + col) * 2;
        const uint32_t a0 = *reinterpret_cast<const uint16_t*>(vp);
        const uint32_t a1 = *reinterpret_cast<const uint16_t*>(vp + VROW);
        const uint32_t a2 = *reinterpret_cast<const uint16_t*>(vp + 2 * VROW);
        const uint32_t a3 = *reinterpret_cast<const uint16_t*>(vp + 3 * VROW);
        const uint2 av = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
        acc[j] = M::pv(av, bhi, acc[j]);
        acc[j] = M::pv(av, blo, acc[j]);
      }
      __syncthreads();  // reads done before the next block overwrites s_v
    }

    // acc[j][v] = O^T[dim 16j + 4*grp + v][query col], unnormalised
    if (q_ok) {
      const size_t pi = ((size_t)sq * H + h) * num_parts + chunk;
      const float inv = 1.f / l;
#pragma unroll
      for (int j = 0; j < NPV; ++j) {
        *reinterpret_cast<float4*>(ws_o + pi * D + 16 * j + 4 * grp) =
            make_float4(acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv);
      }
      if (grp == 0) {
        ws_ml[pi * 2] = m;
        ws_ml[pi * 2 + 1] = l;
      }
    }
  }
}

namespace {
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D>
hipError_t shared_t(const DecodeArgs& a, hipStream_t st) {
  const int chunk_slots = a.slot_base;  // shared chunks occupy slots [0, slot_base)
  const unsigned grid = (unsigned)a.num_groups * (unsigned)chunk_slots * (unsigned)a.num_heads;
  hipLaunchKernelGGL((decode_shared_kernel<T, D>), dim3(grid), dim3(64), 0, st, a.ws_ml, a.ws_o,
                     static_cast<const uint16_t*>(a.query),
                     static_cast<const uint16_t*>(a.key_cache),
                     static_cast<const uint16_t*>(a.value_cache), a.block_tables, a.group_start,
                     a.shared_blocks, a.num_heads, a.max_blocks_per_seq, a.num_parts, chunk_slots,
                     a.scale * kLog2e);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode_shared(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == 0) return a.head_dim == 64 ? shared_t<F16, 64>(a, st) : shared_t<F16, 128>(a, st);
  return a.head_dim == 64 ? shared_t<BF16, 64>(a, st) : shared_t<BF16, 128>(a, st);
}

}  // namespace pkv
