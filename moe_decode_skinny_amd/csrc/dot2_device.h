// Device helpers of the GEMM kernels whose lanes run along K (the DOT2
// (VALU) path and the 16-block MFMA path): the eight-product bf16 dot and
// the cross-lane reduce-scatters of a wave.  Included by the single-call and
// the ring kernels only.
#pragma once

#include "device.h"

namespace skinny {
namespace dot2 {

constexpr int kDot2MaxThreads = 512;  // launch bound of the DOT2 kernels' 8-wave form

// Eight bf16 products accumulated in FP32 by four v_dot2_f32_bf16.  The
// operands are split with vector shuffles of a whole-vector bit cast (a bit
// cast of a single vector element does not lower correctly).
__device__ __forceinline__ float dot8(u32x4 a, u32x4 b, float c) {
  const bf16x8 av = __builtin_bit_cast(bf16x8, a);
  const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 0, 1),
                                      __builtin_shufflevector(bv, bv, 0, 1), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 2, 3),
                                      __builtin_shufflevector(bv, bv, 2, 3), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 4, 5),
                                      __builtin_shufflevector(bv, bv, 4, 5), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(av, av, 6, 7),
                                      __builtin_shufflevector(bv, bv, 6, 7), c, false);
  return c;
}

// Cross-lane reduce-scatter of R values per lane (R a power of two, <= 64)
// over the 64 lanes of a wave.  Six exchange steps pair lane l with l ^ 32,
// l ^ 16, l ^ 15, l ^ 7, l ^ 3 and l ^ 1 (gfx950 v_permlane32_swap /
// v_permlane16_swap, then DPP row_mirror, row_half_mirror and two quad
// permutations; no LDS traffic).  While a lane holds more than one value,
// each step halves them: the lane keeps the low or high half according to
// bit 5, 4, 3, 2, 1, 0 of its index and adds its partner's copy of that
// half; once one value is left the remaining steps add the partner's value.
// The six masks are linearly independent, so every lane ends with a full sum
// over all 64 lanes, in an order fixed by the lane layout, of value index
// lane >> (6 - log2 R).
__device__ __forceinline__ unsigned as_u(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ __forceinline__ float as_f(unsigned u) { return __builtin_bit_cast(float, u); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <int C, int D>  // D = 32 or 16: the permlane swap steps
__device__ __forceinline__ void swap_step(float *v) {
  if constexpr (C >= 2) {
#pragma unroll
    for (int j = 0; j < C / 2; ++j) {
      const auto p = D == 32 ? __builtin_amdgcn_permlane32_swap(as_u(v[j]), as_u(v[j + C / 2]), false, false)
                             : __builtin_amdgcn_permlane16_swap(as_u(v[j]), as_u(v[j + C / 2]), false, false);
      v[j] = as_f(p[0]) + as_f(p[1]);
    }
  } else {
    const auto p = D == 32 ? __builtin_amdgcn_permlane32_swap(as_u(v[0]), as_u(v[0]), false, false)
                           : __builtin_amdgcn_permlane16_swap(as_u(v[0]), as_u(v[0]), false, false);
    v[0] = as_f(p[0]) + as_f(p[1]);
  }
}

template <int C, int CTRL, int BIT>  // steps inside a 16-lane row, by DPP
__device__ __forceinline__ void dpp_step(float *v, int lane) {
  const bool hi = (lane & BIT) != 0;
  if constexpr (C >= 2) {
#pragma unroll
    for (int j = 0; j < C / 2; ++j) {
      const float keep = hi ? v[j + C / 2] : v[j];
      const float give = hi ? v[j] : v[j + C / 2];
      v[j] = keep + dpp<CTRL>(give);
    }
  } else {
    v[0] = v[0] + dpp<CTRL>(v[0]);
  }
}

constexpr int halve(int c) { return c > 1 ? c / 2 : 1; }
constexpr int log2i(int c) { return c <= 1 ? 0 : 1 + log2i(c / 2); }

template <int R>
__device__ __forceinline__ void wave_reduce_scatter(float *v, int lane) {
  static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "R must be a power of two <= 64");
  constexpr int c0 = R, c1 = halve(c0), c2 = halve(c1), c3 = halve(c2), c4 = halve(c3),
                c5 = halve(c4);
  swap_step<c0, 32>(v);
  swap_step<c1, 16>(v);
  dpp_step<c2, 0x140, 8>(v, lane);  // row_mirror: l ^ 15
  dpp_step<c3, 0x141, 4>(v, lane);  // row_half_mirror: l ^ 7
  dpp_step<c4, 0x1B, 2>(v, lane);   // quad_perm [3, 2, 1, 0]: l ^ 3
  dpp_step<c5, 0xB1, 1>(v, lane);   // quad_perm [1, 0, 3, 2]: l ^ 1
}

// l ^ 4 inside each 8-lane half row: DPP row_half_mirror (l ^ 7) followed
// by quad_perm [3, 2, 1, 0] (l ^ 3).
__device__ __forceinline__ float dpp_xor4(float x) { return dpp<0x1B>(dpp<0x141>(x)); }

template <int C>
__device__ __forceinline__ void xor4_step(float *v, int lane) {
  const bool hi = (lane & 4) != 0;
  if constexpr (C >= 2) {
#pragma unroll
    for (int j = 0; j < C / 2; ++j) {
      const float keep = hi ? v[j + C / 2] : v[j];
      const float give = hi ? v[j] : v[j + C / 2];
      v[j] = keep + dpp_xor4(give);
    }
  } else {
    v[0] = v[0] + dpp_xor4(v[0]);
  }
}

// Reduce-scatter of R values per lane (R a power of two, <= 64) over the 16
// lanes that share bits 1..0 of their index (the 16 blocks of a
// v_mfma_f32_4x4x4_16b_bf16 result; bits 1..0 index a block's column).
// Steps pair lane l with l ^ 32, l ^ 16 (permlane swaps), l ^ 8 (DPP
// row_ror:8) and l ^ 4, halving the values while more than one is left, as
// in wave_reduce_scatter; afterwards a lane holds the full 16-lane sums of
// value index lane >> (6 - log2 R) for R <= 16, and for R = 32 or 64 of
// indices U (lane >> 2) + u in v[u], u < U = R / 16.
template <int R>
__device__ __forceinline__ void block_reduce_scatter(float *v, int lane) {
  static_assert(R >= 1 && R <= 64 && (R & (R - 1)) == 0, "R must be a power of two <= 64");
  constexpr int c0 = R, c1 = halve(c0), c2 = halve(c1), c3 = halve(c2);
  swap_step<c0, 32>(v);
  swap_step<c1, 16>(v);
  dpp_step<c2, 0x128, 8>(v, lane);  // row_ror:8: l ^ 8 inside a 16-lane row
  xor4_step<c3>(v, lane);
}

}  // namespace dot2
}  // namespace skinny
