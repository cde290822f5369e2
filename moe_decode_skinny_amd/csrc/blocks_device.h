// Device code of the 16-block MFMA path (SKINNY_PATH_MFMA_4X4) shared by
// the single-call and the ring kernels, so that a tile's products and sums
// are the same instructions in the same order in both.
//
// v_mfma_f32_4x4x4_16b_bf16 computes 16 independent 4 x 4 x 4 products in
// one instruction: block b (lanes 4b .. 4b + 3) takes A from lane 4b + i
// (4 bf16 of row i), B from lane 4b + j (4 bf16 of column j) and adds
// sum_k A[i][k] B[k][j] into register i of lane 4b + j.  Here row i is a
// token and column j a weight row, and every block owns its own 4 K:
//   lane 4b + j of a wave loads 16 bytes at K offset k = k_w + 8b + 128 c
//   (chunk c) of weight row j of each row set (4 rows) and of token j of
//   each token set (4 tokens), so one load instruction moves 4 rows x 256
//   contiguous bytes; the two halves of a load feed two MFMAs.
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
// activations: the tokens), CHUNKS chunks of 128 K from k0 (this lane's K
// offset in chunk 0), row j = lane & 3 of each set.  Loads at or past K, and
// past the resource, read zeros.  AUX: the cache policy bits of the loads.
// The K-tail test selects one base offset per chunk (set q adds 8 q K bytes,
// which keeps an out-of-range base out of range: 0x7FFFF000 + 24 K does not
// wrap for K <= 2^25, the library's limit).
template <int SETS, int CHUNKS, int AUX>
__device__ __forceinline__ void load_sets(u32x4 (&v)[SETS][CHUNKS], __amdgpu_buffer_rsrc_t res,
                                          int K, int k0, int j) {
  const unsigned row = (unsigned)(j * K + k0) * 2u;
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const unsigned base =
        k0 + c * kBlockK < K ? row + (unsigned)(c * kBlockK * 2) : (unsigned)kOutOfRange;
#pragma unroll
    for (int q = 0; q < SETS; ++q)
      v[q][c] = __builtin_amdgcn_raw_buffer_load_b128(res, (int)(base + (unsigned)(8 * q * K)), 0,
                                                      AUX);
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
