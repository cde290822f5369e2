// The DOT2 (VALU) path of the small-M decode GEMM y[M, N] = x[M, K] @ W[N, K]^T
// (unpooler page, module description), for few tokens.
//
// At M = 1 a 16-token MFMA tile wastes 15/16 of its work and forces 16
// features per workgroup; here lanes run along K instead, so a workgroup can
// own any number of rows and a wave-wide load is 1 KiB of one weight row:
//   wave w of workgroup (group, s) owns K range (s * waves + w) * kw,
//   kw = 512 * CHUNKS; lane l reads W[row][k + 8 l .. + 8] for each of the
//   workgroup's ROWS rows (weights first, as the pages order their loads),
//   then x[t][same k] for t < M, and accumulates 8 products per (row, token)
//   with four v_dot2_f32_bf16 (FP32 accumulation of exact bf16 products).
// Reduction in an order fixed by the launch shape (module description):
//   a reduce-scatter over the 64 lanes (dot2_device.h), waves
//   0..waves-1 in order through LDS, and with S > 1 an FP32 partial per split
//   that split_reduce.hip sums s = 0..S-1 in order.
#include "dot2_device.h"
#include "internal.h"

namespace skinny {
namespace {

using namespace dot2;

// THREADS: the launch bound, 512, or 1024 for the register-light variants
// that run 16 waves (long K at one chunk per wave).  The arguments the main
// loop needs come first, the workgroup's wave count among them: the first
// 14 argument dwords arrive preloaded in SGPRs, so the loads issue without
// waiting for a kernel-argument fetch (blockDim would be one).
template <int ROWS, int CHUNKS, int MT, int THREADS>
__global__ __launch_bounds__(THREADS) void gemm_dot2_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int M, int N, int K,
    int S, int groups, int kw, int waves, uint16_t *__restrict__ y,
    float *__restrict__ partials, Publish pub) {
  const int lane = threadIdx.x & 63;
  if (S == 1 && blockIdx.x == 0 && threadIdx.x == 0) publish_stage_word(pub);
  const int wave = wave_index();

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
  // K offset of this lane's 8 elements in chunk 0 of its slice; lanes past K
  // and tokens >= M read past their buffer resource and get zeros.
  const int k0 = (s * waves + wave) * kw + lane * 8;
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(w + (size_t)f0 * K, (unsigned)(ROWS * K * 2));
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(x, (unsigned)(M * K * 2));

  u32x4 wv[ROWS][CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const bool in = k0 + c * kDot2K < K;
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      wv[r][c] = __builtin_amdgcn_raw_buffer_load_b128(
          wres, in ? (r * K + k0 + c * kDot2K) * 2 : kOutOfRange, 0, kCacheNT);
  }
  // All loads in flight before the first wait (no sinking below the math).
  __builtin_amdgcn_sched_barrier(0);
  u32x4 xv[MT][CHUNKS];
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const bool in = k0 + c * kDot2K < K;
#pragma unroll
    for (int t = 0; t < MT; ++t)
      xv[t][c] = __builtin_amdgcn_raw_buffer_load_b128(
          xres, in ? (t * K + k0 + c * kDot2K) * 2 : kOutOfRange, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  float acc[ROWS][MT];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = 0.f;
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c)
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[r][t] = dot8(wv[r][c], xv[t][c], acc[r][t]);

  // Reduce over the wave's 64 lanes; value index r * MT + t ends in the
  // lanes whose top log2(ROWS * MT) bits equal it.
  constexpr int kOut = ROWS * MT;
  constexpr int kShift = 6 - log2i(kOut);
  float v[kOut];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) v[r * MT + t] = acc[r][t];
  wave_reduce_scatter<kOut>(v, lane);

  // Waves in order through LDS; lane i < ROWS * MT then owns (row i / MT,
  // token i % MT).
  __shared__ float red[THREADS / 64][kOut];
  if ((lane & ((1 << kShift) - 1)) == 0) red[wave][lane >> kShift] = v[0];
  __syncthreads();
  if (wave != 0) return;
  const int r = lane / MT, t = lane % MT;
  const bool live = lane < kOut && t < M;
  float part = 0.f;
  if (lane < kOut)
    part = sum_waves_in_order<THREADS / 64, float>(waves, [&](int v2) { return red[v2][lane]; });

  if (!live) return;
  if (S == 1) {
    const unsigned b = f32_to_bf16(part);
    y[(size_t)t * N + f0 + r] = (uint16_t)b;
    if (uint16_t *slot = publish_slot(pub, N)) slot[(size_t)t * N + f0 + r] = (uint16_t)publish_bits(b);
  } else  // FP32 partial of split s: partials[s][token][feature]
    partials[((size_t)s * M + t) * N + f0 + r] = part;
}

using Dot2Kernel = void (*)(const uint16_t *, const uint16_t *, int, int, int, int, int, int,
                            int, uint16_t *, float *, Publish);

// Register budget per lane: weights 4 * ROWS * CHUNKS, activations
// 4 * MT * CHUNKS, sums ROWS * MT: at most 160 for 8 waves, 112 for the
// 16-wave form (128 registers a lane, less the addresses).  Variants above
// the budget are not built.
constexpr bool fits(int rows, int chunks, int mt, int threads) {
  return 4 * rows * chunks + 4 * mt * chunks + rows * mt <= (threads > 512 ? 112 : 160);
}

template <int R, int C, int T, int THREADS>
constexpr Dot2Kernel variant() {
  if constexpr (fits(R, C, T, THREADS)) return gemm_dot2_kernel<R, C, T, THREADS>;
  else return nullptr;
}

template <int R, int C, int THREADS>
Dot2Kernel pick_mt(int mt) {
  switch (mt) {
    case 1: return variant<R, C, 1, THREADS>();
    case 2: return variant<R, C, 2, THREADS>();
    case 4: return variant<R, C, 4, THREADS>();
    case 8: return variant<R, C, 8, THREADS>();
    case 16: return variant<R, C, 16, THREADS>();
  }
  return nullptr;
}

template <int R, int THREADS>
Dot2Kernel pick_chunks(int chunks, int mt) {
  switch (chunks) {
    case 1: return pick_mt<R, 1, THREADS>(mt);
    case 2: return pick_mt<R, 2, THREADS>(mt);
    case 4: return pick_mt<R, 4, THREADS>(mt);
  }
  return nullptr;
}

template <int THREADS>
Dot2Kernel pick_rows(int rows, int chunks, int mt) {
  switch (rows) {
    case 2: return pick_chunks<2, THREADS>(chunks, mt);
    case 4: return pick_chunks<4, THREADS>(chunks, mt);
    case 8: return pick_chunks<8, THREADS>(chunks, mt);
    case 16: return pick_chunks<16, THREADS>(chunks, mt);
  }
  return nullptr;
}

// The variant for a launch of `waves` waves: the 8-wave form up to 8 waves,
// the 16-wave form beyond.
Dot2Kernel pick(int rows, int chunks, int mt, int waves) {
  if (waves >= 1 && waves <= kDot2MaxThreads / 64) return pick_rows<kDot2MaxThreads>(rows, chunks, mt);
  if (waves > kDot2MaxThreads / 64 && waves <= 16) return pick_rows<1024>(rows, chunks, mt);
  return nullptr;
}

}  // namespace

int dot2_token_tile(int M) {
  if (M <= 1) return 1;
  if (M <= 2) return 2;
  if (M <= 4) return 4;
  if (M <= 8) return 8;
  if (M <= 16) return 16;
  return 0;
}

bool dot2_variant_exists(int rows, int chunks, int mt, int waves) {
  return pick(rows, chunks, mt, waves) != nullptr;
}

int dot2_max_waves() { return 16; }

hipError_t launch_gemm_dot2(const uint16_t *x, const uint16_t *w, uint16_t *y,
                            int M, int N, int K, const skinny_launch &l,
                            const Workspace &ws, const Publish &pub, hipStream_t stream) {
  float *partials = ws.partials;
  Dot2Kernel k = pick(l.rows, l.chunks, dot2_token_tile(M), l.waves);
  const int groups = N / l.rows;
  dim3 grid(groups * l.splits), block(64 * l.waves);
  hipLaunchKernelGGL(k, grid, block, 0, stream, x, w, M, N, K, l.splits, groups,
                     kDot2K * l.chunks, l.waves, y, partials, pub);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || l.splits == 1) return e;
  return launch_split_reduce(partials, y, M, N, l.splits, pub, stream);
}

}  // namespace skinny
