// Device-side helpers shared by the gfx950 kernels: 16-bit element types,
// packed dot products, DPP reductions inside a token row, fp32 -> 16-bit
// rounding.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

namespace pkv {

// Tokens per block the kernels are built for (the pages' default of 16 and the
// smaller and larger sizes they weigh against it).
constexpr bool supported_block_size(int bs) { return bs == 8 || bs == 16 || bs == 32; }

// Tokens per tile of the grouped path's MFMA contraction (M = 16).
constexpr int kTileTokens = 16;

// Shared-prefix tokens the grouped path's MFMA units cover for a group whose
// first `shared_blocks` blocks are shared: the shared tokens rounded down to
// whole 16-token tiles. The rest (an odd last block at block size 8) is read
// with the sequence's own tail.
__host__ __device__ __forceinline__ int shared_prefix_tokens(int shared_blocks, int block_size) {
  return (shared_blocks * block_size) & ~(kTileTokens - 1);
}

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

struct F16 {};
struct BF16 {};

// Element-type operations on 32-bit words holding two elements (element 2i in
// the low half, 2i+1 in the high half: the little-endian memory order).
template <typename T> struct Elem;

template <> struct Elem<F16> {
  // v_dot2_f32_f16: fp32 result of a.lo*b.lo + a.hi*b.hi + c.
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b), c,
                                  false);
  }
  static __device__ __forceinline__ float lo(uint32_t w) {
    return (float)__builtin_bit_cast(half2_t, w).x;
  }
  static __device__ __forceinline__ float hi(uint32_t w) {
    return (float)__builtin_bit_cast(half2_t, w).y;
  }
  // Round to nearest even (the hardware default rounding mode).
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
  }
  // round(a) in the low half, round(b) in the high half (one packed convert).
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){a, b}, half2_t));
  }
};

template <> struct Elem<BF16> {
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, a),
                                           __builtin_bit_cast(bf162_t, b), c, false);
  }
  // bf16 is the upper half of an fp32, so widening is a shift or a mask.
  static __device__ __forceinline__ float lo(uint32_t w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
  static __device__ __forceinline__ uint16_t round(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2_t){a, b}, bf162_t));
  }
};

// DPP lane moves within a 16-lane row (gfx9 DPP control codes).
enum : int {
  kDppXor1 = 0xB1,        // quad_perm [1,0,3,2]
  kDppXor2 = 0x4E,        // quad_perm [2,3,0,1]
  kDppHalfMirror = 0x141, // lane i <- lane 7-i within each half row
  kDppMirror = 0x140,     // lane i <- lane 15-i within each row
};

template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane of a group gets
// the same, bit-identical sum (each step adds a pair symmetrically).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp_move<kDppXor1>(x);
  x += dpp_move<kDppXor2>(x);
  x += dpp_move<kDppHalfMirror>(x);
  if constexpr (N == 16) x += dpp_move<kDppMirror>(x);
  return x;
}

// DPP lane moves for a wave-wide prefix sum (gfx9 control codes): shift right
// by n lanes within each 16-lane row, and the broadcast of lane 15 (31) of a
// row to the rows after it.
enum : int {
  kDppRowShr1 = 0x111,
  kDppRowShr2 = 0x112,
  kDppRowShr4 = 0x114,
  kDppRowShr8 = 0x118,
  kDppRowBcast15 = 0x142,
  kDppRowBcast31 = 0x143,
};

// Inclusive prefix sum of x over lanes 0 .. this lane, with DPP moves only
// (no LDS round trips): a scan inside each 16-lane row, then row 0's total
// into row 1 and row 2's into row 3, then lane 31's running total into rows 2
// and 3. Lanes whose DPP source lies outside the row add 0.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr2, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr4, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr8, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xC, 0xF, false);
  return x;
}

// Maximum of x over the wave's 64 lanes, with the same DPP moves as the
// prefix sum (a running maximum, read from lane 63).
__device__ __forceinline__ int wave_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, kDppRowShr1, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, kDppRowShr2, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, kDppRowShr4, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, kDppRowShr8, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, kDppRowBcast15, 0xA, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, kDppRowBcast31, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(x, 63);
}

// Lane holding the (j + 1)-th set bit of the wave-uniform mask m (j <
// popcount(m)), found by ranking the set lanes with mbcnt and one ballot.
__device__ __forceinline__ int nth_set_lane(uint64_t m, int j) {
  const int lane = threadIdx.x & 63;
  const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  const uint64_t sel = __ballot((((m >> lane) & 1ull) != 0) && (int)rank == j);
  return __ffsll((unsigned long long)sel) - 1;
}

// 2^x with the hardware instruction (v_exp_f32); 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Shared blocks of sequence s's group: shared_blocks[g] for the largest
// g < num_groups with group_start[g] <= s (group_start is nondecreasing from 0
// to num_seqs, so that g has group_start[g] <= s < group_start[g + 1],
// skipping empty groups). Called by a whole wave with the same s: lane i loads
// entry i of each 64-entry chunk of both arrays at once, a ballot counts the
// starts <= s (a prefix of the chunk), and the last such lane's shared_blocks
// entry is read across lanes. One memory round trip per 64 groups, with no
// load waiting on another.
__device__ __forceinline__ int group_shared_blocks(int s, const int32_t* __restrict__ group_start,
                                                   const int32_t* __restrict__ shared_blocks,
                                                   int num_groups) {
  const int lane = threadIdx.x & 63;
  int sb = 0;
  for (int base = 0; base < num_groups; base += 64) {
    const int g = base + lane;
    const bool in = g < num_groups;
    const int gs = in ? group_start[g] : 0;
    const int sbv = in ? shared_blocks[g] : 0;
    const int c = __popcll(__ballot(in && gs <= s));   // wave-uniform
    if (c > 0) sb = __builtin_amdgcn_readlane(sbv, c - 1);
    if (c < 64) break;                                  // later starts are past s
  }
  return sb;
}

}  // namespace pkv
