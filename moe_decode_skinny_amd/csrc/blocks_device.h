// Device code of the 16-block MFMA path (SKINNY_PATH_MFMA_4X4) shared by
// the single-call and the ring kernels, so that a tile's products and sums
// are the same instructions in the same order in both.
//
// v_mfma_f32_4x4x4_16b_bf16 computes 16 independent 4 x 4 x 4 products in
// one instruction: block b (lanes 4b .. 4b + 3) takes A from lane 4b + i
// (4 bf16 of row i), B from lane 4b + j (4 bf16 of column j) and adds
// sum_k A[i][k] B[k][j] into register i of lane 4b + j.  Here row i is a
// token and column j a weight row, and every block owns its own K:
//   loads: per group of 512 K (four 128-K chunks), load p of a 4-row set
//   (weights: 4 rows of the tile; activations: 4 tokens) reads row p, lane l
//   taking 16 bytes at K offset k_w + 8 l, so every load instruction is 1 KiB
//   of one row and each 4-lane group reads 64 contiguous bytes;
//   a transpose inside every 4-lane group (two exchange steps, DPP quad
//   permutations and selects) then leaves lane 4b + j with row j at the K
//   offsets k_w + 32 b + 8 s of its four registers s = 0..3, the layout the
//   MFMA needs (all four lanes of a block at the same K);
//   chunk c = 4 g + s of a set is register s of group g, and the two halves
//   of a register feed two MFMAs.
// (Loading each block's four rows directly puts four rows, so four cache
// lines, in every 4-lane group; the load path then serves a quarter of the
// bytes per cycle, which cost 30-40% on the calls this path is picked for.)
// Per wave and (token set, row set) this leaves a 4 x 4 partial per block;
// the blocks are summed across lanes by block_reduce_scatter (lane bits
// 5..2, a fixed order) and the waves in wave order through LDS.
#pragma once

#include "dot2_device.h"

namespace skinny {
namespace blocks {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// The low (H = 0) or high (H = 1) four bf16 of a 16-byte load as an MFMA operand.
template <int H>
__device__ __forceinline__ s16x4 half4(u32x4 v) {
  const u32x2 h = H == 0 ? u32x2{v.x, v.y} : u32x2{v.z, v.w};
  return __builtin_bit_cast(s16x4, h);
}

// SETS x 4 rows of a row-major [rows][K] operand (weights: a tile's rows;
// activations: the tokens), CHUNKS / 4 groups of 512 K from k0 (this lane's
// K offset in group 0, 8 * lane past the wave's start): v[q][4 g + p] is row
// 4 q + p of group g, as loaded (transpose_sets puts it in MFMA order).
// Loads at or past K, and past the resource, read zeros.  AUX: the cache
// policy bits of the loads.  The K-tail test selects one base offset per
// group (row 4 q + p adds (4 q + p) K bytes, which keeps an out-of-range base
// out of range: 0x7FFFF000 + 30 K does not wrap for K <= 2^25, the library's
// limit).
template <int SETS, int CHUNKS, int AUX>
__device__ __forceinline__ void load_sets(u32x4 (&v)[SETS][CHUNKS], __amdgpu_buffer_rsrc_t res,
                                          int K, int k0) {
  static_assert(CHUNKS % 4 == 0, "the 16-block path loads whole 512-K groups");
#pragma unroll
  for (int g = 0; g < CHUNKS / 4; ++g) {
    const unsigned base = k0 + g * kGroupK < K ? (unsigned)(k0 + g * kGroupK) * 2u
                                               : (unsigned)kOutOfRange;
#pragma unroll
    for (int q = 0; q < SETS; ++q)
#pragma unroll
      for (int p = 0; p < 4; ++p)
        v[q][4 * g + p] = __builtin_amdgcn_raw_buffer_load_b128(
            res, (int)(base + (unsigned)((4 * q + p) * 2) * (unsigned)K), 0, AUX);
  }
}

// One exchange of the 4-lane transpose for a register pair (lo, hi) = (r,
// r | M), lane bit M: a lane with the bit clear keeps lo and takes its
// partner's lo into hi; a lane with the bit set keeps hi and takes its
// partner's hi into lo (two DPP quad permutations and two selects a dword).
template <int M, int CTRL>
__device__ __forceinline__ void quad_exchange(u32x4 &lo, u32x4 &hi, bool upper) {
  u32x4 nlo, nhi;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const unsigned from_lo =
        (unsigned)__builtin_amdgcn_update_dpp(0, (int)lo[d], CTRL, 0xF, 0xF, false);
    const unsigned from_hi =
        (unsigned)__builtin_amdgcn_update_dpp(0, (int)hi[d], CTRL, 0xF, 0xF, false);
    nlo[d] = upper ? from_hi : lo[d];
    nhi[d] = upper ? hi[d] : from_lo;
  }
  lo = nlo;
  hi = nhi;
}

// Transpose every 4-register group across the 4 lanes of each block: lane
// 4b + j, register p (row p at K slot j) -> register s (row j at K slot s).
template <int SETS, int CHUNKS>
__device__ __forceinline__ void transpose_sets(u32x4 (&v)[SETS][CHUNKS], int lane) {
  const bool odd = (lane & 1) != 0, upper_pair = (lane & 2) != 0;
#pragma unroll
  for (int q = 0; q < SETS; ++q)
#pragma unroll
    for (int g = 0; g < CHUNKS / 4; ++g) {
      u32x4 *t = &v[q][4 * g];
      quad_exchange<1, 0xB1>(t[0], t[1], odd);         // quad_perm [1, 0, 3, 2]
      quad_exchange<1, 0xB1>(t[2], t[3], odd);
      quad_exchange<2, 0x4E>(t[0], t[2], upper_pair);  // quad_perm [2, 3, 0, 1]
      quad_exchange<2, 0x4E>(t[1], t[3], upper_pair);
    }
}

// The wave's products: acc[q][r] over its K slice, chunk by chunk, low then
// high half, token sets outer, row sets inner.
template <int R4, int CHUNKS, int Q>
__device__ __forceinline__ void products(const u32x4 (&wv)[R4][CHUNKS],
                                         const u32x4 (&xv)[Q][CHUNKS], f32x4 (&acc)[Q][R4]) {
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int r = 0; r < R4; ++r) acc[q][r] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int r = 0; r < R4; ++r)
        acc[q][r] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(half4<0>(xv[q][c]),
                                                           half4<0>(wv[r][c]), acc[q][r], 0, 0, 0);
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int r = 0; r < R4; ++r)
        acc[q][r] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(half4<1>(xv[q][c]),
                                                           half4<1>(wv[r][c]), acc[q][r], 0, 0, 0);
  }
}

// Outputs of a wave: o = (t * R4 + r4) * 4 + j for token t, row 4 r4 + j.
template <int R4, int Q>
constexpr int kOutputs = 16 * Q * R4;

__device__ __forceinline__ int output_token(int o, int r4s) { return (o >> 2) / r4s; }
__device__ __forceinline__ int output_row(int o, int r4s) { return 4 * ((o >> 2) % r4s) + (o & 3); }

// Sum the wave's partials over its 16 blocks and write output o of the wave
// to red[o] (each output written by one lane).
template <int R4, int Q>
__device__ __forceinline__ void reduce_to_lds(const f32x4 (&acc)[Q][R4], float *red, int lane) {
  constexpr int kVals = 4 * Q * R4;
  float v[kVals];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < R4; ++r) v[(4 * q + i) * R4 + r] = acc[q][r][i];
  dot2::block_reduce_scatter<kVals>(v, lane);
  const int j = lane & 3;
  if constexpr (kVals >= 16) {
    constexpr int U = kVals / 16;
#pragma unroll
    for (int u = 0; u < U; ++u) red[((lane >> 2) * U + u) * 4 + j] = v[u];
  } else {
    // lanes that differ only in bits below kShift hold the same sums
    constexpr int kShift = 6 - dot2::log2i(kVals);
    if (((lane >> 2) & ((1 << (kShift - 2)) - 1)) == 0) red[(lane >> kShift) * 4 + j] = v[0];
  }
}

}  // namespace blocks
}  // namespace skinny
