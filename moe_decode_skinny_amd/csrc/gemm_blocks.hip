// The 16-block MFMA path of the small-M decode GEMM y[M, N] = x[M, K] @ W[N, K]^T
// (unpooler page, module description): lanes run along K as in the DOT2
// path, the products go to the matrix cores (v_mfma_f32_4x4x4_16b_bf16; the
// lane layout and the order of the sums are in blocks_device.h).
//   wave w of workgroup (group, s) owns K range (s * waves + w) * kw,
//   kw = 128 * CHUNKS (CHUNKS 4 or 8: whole 512-K load groups), of the
//   workgroup's 4 * R4 weight rows, and all M tokens in Q sets of 4; weights
//   are loaded first, then activations, then both are transposed into the
//   MFMA layout inside each 4-lane group.
// Reduction in an order fixed by the launch shape (module description): the
// 16 blocks across lanes, waves 0..waves-1 in order through LDS, and with
// S > 1 an FP32 partial per split that split_reduce.hip sums s = 0..S-1 in
// order.
//
// Against DOT2 this replaces 4 VALU instructions per (row, token, 8 K) and a
// 64-lane reduce-scatter with one MFMA per (row set, token set, 4 K x 16
// blocks), a 16-lane reduce-scatter and 4 DPP moves and selects per loaded
// 4 bytes (the transpose); the loads are the same 1 KiB row pieces as DOT2's.
#include "blocks_device.h"
#include "internal.h"

namespace skinny {
namespace {

using namespace blocks;

template <int R4, int CHUNKS, int Q, int THREADS>
__global__ __launch_bounds__(THREADS) void gemm_blocks_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    uint16_t *__restrict__ y, float *__restrict__ partials, int M, int N, int K,
    int S, int groups, int kw, Publish pub) {
  constexpr int ROWS = 4 * R4;
  const int lane = threadIdx.x & 63;
  if (S == 1 && blockIdx.x == 0 && threadIdx.x == 0) publish_stage_word(pub);
  const int wave = wave_index();
  const int waves = blockDim.x >> 6;

  int group, s;
  const int b = blockIdx.x;
  if ((groups & 7) == 0) {  // the S workgroups of a group share an XCD
    const int xcd = b & 7, slot = b >> 3;
    group = (slot / S) * 8 + xcd;
    s = slot % S;
  } else {
    group = b / S;
    s = b % S;
  }
  const int f0 = group * ROWS;
  const int k0 = (s * waves + wave) * kw + lane * 8;

  u32x4 wv[R4][CHUNKS], xv[Q][CHUNKS];
  load_sets<R4, CHUNKS, kCacheNT>(wv, buffer_rsrc(w + (size_t)f0 * K, (unsigned)(ROWS * K * 2)),
                                  K, k0);
  __builtin_amdgcn_sched_barrier(0);
  load_sets<Q, CHUNKS, 0>(xv, buffer_rsrc(x, (unsigned)(M * K * 2)), K, k0);
  __builtin_amdgcn_sched_barrier(0);
  transpose_sets<R4, CHUNKS>(wv, lane);
  transpose_sets<Q, CHUNKS>(xv, lane);
  f32x4 acc[Q][R4];
  products<R4, CHUNKS, Q>(wv, xv, acc);

  constexpr int kOut = kOutputs<R4, Q>;
  __shared__ float red[THREADS / 64][kOut];
  reduce_to_lds<R4, Q>(acc, red[wave], lane);
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int o0 = 0; o0 < kOut; o0 += 64) {
    const int o = o0 + lane;
    if (o >= kOut) break;
    float part = red[0][o];
    for (int v2 = 1; v2 < waves; ++v2) part += red[v2][o];
    const int t = output_token(o, R4), r = output_row(o, R4);
    if (t >= M) continue;
    if (S == 1) {
      const unsigned bits = f32_to_bf16(part);
      y[(size_t)t * N + f0 + r] = (uint16_t)bits;
      if (uint16_t *slot = publish_slot(pub, N))
        slot[(size_t)t * N + f0 + r] = (uint16_t)publish_bits(bits);
    } else {  // FP32 partial of split s: partials[s][token][feature]
      partials[((size_t)s * M + t) * N + f0 + r] = part;
    }
  }
}

using BlocksKernel = void (*)(const uint16_t *, const uint16_t *, uint16_t *, float *, int,
                              int, int, int, int, int, Publish);

// Register budget per lane: weights 4 * R4 * CHUNKS, activations
// 4 * Q * CHUNKS, sums 4 * Q * R4 (160 at 512 threads, 112 at 1024).
constexpr bool fits(int r4, int chunks, int q, int threads) {
  return 4 * r4 * chunks + 4 * q * chunks + 4 * q * r4 <= (threads > 512 ? 112 : 160);
}

template <int R4, int C, int Q, int T>
constexpr BlocksKernel variant() {
  if constexpr (fits(R4, C, Q, T)) return gemm_blocks_kernel<R4, C, Q, T>;
  else return nullptr;
}

template <int R4, int C, int T>
BlocksKernel pick_q(int q) {
  switch (q) {
    case 1: return variant<R4, C, 1, T>();
    case 2: return variant<R4, C, 2, T>();
    case 4: return variant<R4, C, 4, T>();
  }
  return nullptr;
}

template <int R4, int T>
BlocksKernel pick_chunks(int chunks, int q) {
  switch (chunks) {
    case 4: return pick_q<R4, 4, T>(q);
    case 8: return pick_q<R4, 8, T>(q);
  }
  return nullptr;
}

template <int T>
BlocksKernel pick_rows(int rows, int chunks, int q) {
  switch (rows) {
    case 4: return pick_chunks<1, T>(chunks, q);
    case 8: return pick_chunks<2, T>(chunks, q);
  }
  return nullptr;
}

BlocksKernel pick(int rows, int chunks, int q, int waves) {
  return waves <= 8 ? pick_rows<512>(rows, chunks, q) : pick_rows<1024>(rows, chunks, q);
}

}  // namespace

int blocks_token_sets(int M) {
  if (M <= 4) return 1;
  if (M <= 8) return 2;
  if (M <= 16) return 4;
  return 0;
}

bool blocks_variant_exists(int rows, int chunks, int q, int waves) {
  return waves >= 1 && waves <= kBlocksMaxWaves && pick(rows, chunks, q, waves) != nullptr;
}

hipError_t launch_gemm_blocks(const uint16_t *x, const uint16_t *w, uint16_t *y, int M,
                              int N, int K, const skinny_launch &l, float *partials,
                              const Publish &pub, hipStream_t stream) {
  BlocksKernel k = pick(l.rows, l.chunks, blocks_token_sets(M), l.waves);
  const int groups = N / l.rows;
  dim3 grid(groups * l.splits), block(64 * l.waves);
  hipLaunchKernelGGL(k, grid, block, 0, stream, x, w, y, partials, M, N, K, l.splits,
                     groups, kBlockK * l.chunks, pub);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || l.splits == 1) return e;
  return launch_split_reduce(partials, y, M, N, l.splits, pub, stream);
}

}  // namespace skinny
