// The MFMA path of the small-M decode GEMM  y[M, N] = x[M, K] @ W[N, K]^T
// (unpooler page, module description): BF16 in and out, FP32 accumulation,
// 1 <= M <= 16.
//
// gfx950 design.  The pages' SM100 kernel feeds 16 weight rows x 8 tokens to
// mma.sync; here one v_mfma_f32_16x16x32_bf16 takes 16 weight rows (A) and 16
// tokens (B, zero-padded past M) over 32 K:
//   A lane l holds W[f0 + (l % 16)][k + 8 (l / 16) .. + 8]      (one 16-B load)
//   B lane l holds x[(l % 16)][k + 8 (l / 16) .. + 8]           (zero if >= M)
//   D lane l holds acc[feature 4 (l / 16) + v][token l % 16], v = 0..3
// so a lane's four results are four consecutive features of one token: one
// 8-byte store of y.
//
// Work split (unpooler page, module description: CTA (t, s) owns features
// [16 t, 16 t + 16) and the K slice s; each warp owns consecutive K):
//   workgroup (tile, s), s < S, owns features [16 tile, 16 tile + 16);
//   its wave w owns the K range of slice (s * waves + w), kw = 32 * CHUNKS
//   consecutive K.  All of a wave's weight loads are issued first (the pages
//   load weights before their dependency wait), then its activation loads,
//   then the MFMAs, chunk i into accumulator i % ACCS.
// Reduction, in an order fixed by the launch shape (module description:
// partials summed in a fixed order, so runs are bitwise reproducible):
//   accumulators 0..ACCS-1 in order -> waves 0..waves-1 in order through LDS
//   -> with S > 1, the workgroup partials of a tile s = 0..S-1 in order, by
//   the workgroup that arrives last at the tile's counter (agent-scope
//   release/acquire; the counter is reset by that workgroup, so no memset
//   is needed between launches or graph replays).
#include "internal.h"

namespace skinny {
namespace {

// Threads per workgroup a variant is compiled for: 16 chunks of weights and
// activations need 128 VGPRs of operands, so that variant gets 8 waves.
constexpr int mfma_max_threads(int chunks) { return chunks >= 16 ? 512 : 1024; }

template <int CHUNKS, int ACCS>
__global__ __launch_bounds__(mfma_max_threads(CHUNKS)) void gemm_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
    uint16_t *__restrict__ y, float *__restrict__ partials,
    unsigned *__restrict__ counters, int M, int N, int K, int S, int tiles,
    int kw) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const int row = lane & 15;  // weight row (A) / token (B) of this lane
  const int grp = lane >> 4;  // which 8-wide K group of a 32-wide chunk

  // Workgroup -> (tile, split).  Workgroups are dispatched to the 8 XCDs
  // round-robin, so ids congruent mod 8 share an XCD (and its L2); when the
  // tile count allows, the S workgroups of a tile get ids that share one.
  int tile, s;
  const int b = blockIdx.x;
  if ((tiles & 7) == 0) {
    const int xcd = b & 7, slot = b >> 3;
    tile = (slot / S) * 8 + xcd;
    s = slot % S;
  } else {
    tile = b / S;
    s = b % S;
  }

  // K offset of this lane's 8 elements in chunk 0 of its slice.
  const int k0 = (s * waves + wave) * kw + grp * 8;
  // Byte offsets inside the 16-row weight block of this tile and inside x.
  // Lanes whose chunk lies past K, or whose token row is >= M, read past the
  // end of their buffer resource and get zeros.
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(w + (size_t)tile * kTileN * K, (unsigned)(kTileN * K * 2));
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(x, (unsigned)(M * K * 2));
  const int woff = (row * K + k0) * 2;
  const int xoff = (row * K + k0) * 2;
  const bool token = row < M;

  // Weight stream first: every W byte of the slice is read exactly once.
  u32x4 wv[CHUNKS];
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int off = k0 + i * kMfmaK < K ? woff + i * kMfmaK * 2 : kOutOfRange;
    wv[i] = __builtin_amdgcn_raw_buffer_load_b128(wres, off, 0, kCacheNT);
  }
  // Keep the compiler from sinking loads below the MFMAs: the whole slice
  // must be in flight before the first wait.
  __builtin_amdgcn_sched_barrier(0);
  // Activations: zero past row M (token padding in registers) and past K.
  u32x4 xv[CHUNKS];
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int off = k0 + i * kMfmaK < K ? xoff + i * kMfmaK * 2 : kOutOfRange;
    xv[i] = __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);

  f32x4 acc[ACCS];
#pragma unroll
  for (int a = 0; a < ACCS; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i)
    acc[i % ACCS] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, wv[i]), __builtin_bit_cast(bf16x8, xv[i]),
        acc[i % ACCS], 0, 0, 0);
  f32x4 part = acc[0];
#pragma unroll
  for (int a = 1; a < ACCS; ++a) part += acc[a];

  // Waves 0..waves-1 in order, through LDS.
  __shared__ f32x4 red[kMaxWaves][64];
  if (waves > 1) {
    red[wave][lane] = part;
    __syncthreads();
    if (wave != 0) return;
    part = red[0][lane];
    for (int v = 1; v < waves; ++v) part += red[v][lane];
  }

  if (S > 1) {
    // Workgroup partial of split s -> workspace; last arriver sums s in order.
    f32x4 *ws = reinterpret_cast<f32x4 *>(partials) + (size_t)tile * S * 64;
    if (token) ws[s * 64 + lane] = part;
    __threadfence();  // release: partial visible device-wide before the count
    unsigned prev = 0;
    if (lane == 0) prev = atomicAdd(&counters[tile], 1u);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev != (unsigned)(S - 1)) return;
    __threadfence();  // acquire: the other splits' partials
    if (token) {
      f32x4 sum = s == 0 ? part : ws[lane];
      for (int j = 1; j < S; ++j) sum += (j == s) ? part : ws[j * 64 + lane];
      part = sum;
    }
    if (lane == 0)
      __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  if (token) {
    const unsigned lo = f32_to_bf16(part[0]) | (f32_to_bf16(part[1]) << 16);
    const unsigned hi = f32_to_bf16(part[2]) | (f32_to_bf16(part[3]) << 16);
    uint2 *dst = reinterpret_cast<uint2 *>(y + (size_t)row * N + tile * kTileN + grp * 4);
    *dst = make_uint2(lo, hi);
  }
}

using MfmaKernel = void (*)(const uint16_t *, const uint16_t *, uint16_t *,
                            float *, unsigned *, int, int, int, int, int, int);

template <int C>
MfmaKernel pick_accs(int accs) {
  switch (accs) {
    case 1: return gemm_mfma_kernel<C, 1>;
    case 2: return gemm_mfma_kernel<C, 2>;
    case 4: return gemm_mfma_kernel<C, 4>;
  }
  return nullptr;
}

MfmaKernel pick(int chunks, int accs) {
  switch (chunks) {
    case 1: return pick_accs<1>(accs);
    case 2: return pick_accs<2>(accs);
    case 4: return pick_accs<4>(accs);
    case 8: return pick_accs<8>(accs);
    case 16: return pick_accs<16>(accs);
  }
  return nullptr;
}

}  // namespace

bool mfma_variant_exists(int chunks, int accs) { return pick(chunks, accs) != nullptr; }

int mfma_max_waves(int chunks) { return mfma_max_threads(chunks) / 64; }

hipError_t launch_gemm_mfma(const uint16_t *x, const uint16_t *w, uint16_t *y,
                            int M, int N, int K, const skinny_launch &l,
                            DeviceState &st, hipStream_t stream) {
  MfmaKernel k = pick(l.chunks, l.accs);
  const int tiles = N / kTileN;
  dim3 grid(tiles * l.splits), block(64 * l.waves);
  hipLaunchKernelGGL(k, grid, block, 0, stream, x, w, y, st.partials, st.counters,
                     M, N, K, l.splits, tiles, kMfmaK * l.chunks);
  return hipGetLastError();
}

}  // namespace skinny
