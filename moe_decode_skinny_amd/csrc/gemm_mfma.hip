// The MFMA path of the small-M decode GEMM  y[M, N] = x[M, K] @ W[N, K]^T
// (unpooler page, module description): BF16 operands and result, FP32 sums,
// 1 to 16 tokens.
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
// Work split (unpooler page, module description: there a thread block is a
// 16-feature tile and one of S slices of K, and its warps divide the slice
// into consecutive runs of K):
//   workgroup (group, s), s < S, owns F = rows / 16 tiles of 16 features and
//   the K slice s of length kslice = KW * kw; its waves are (tile f, quarter
//   q), q < KW, and wave (f, q) owns K [s kslice + q kw, + kw), kw = 32 CHUNKS.
//   All of a wave's weight loads are issued first (the pages load weights
//   before their dependency wait); then the workgroup reads its x slice once,
//   along K, into LDS, where the F tiles share it (activation traffic is
//   M / (16 F) of the weight traffic); then each wave runs its MFMAs, chunk i
//   into accumulator i % ACCS, with B fragments read from LDS.
// Reduction, in an order fixed by the launch shape (module description: the
// partials are added in one fixed order, so repeated runs give the same
// bits):
//   accumulators 0..ACCS-1 in order -> waves q = 0..KW-1 of a tile in order
//   through LDS -> with S = 1 the BF16 store; with S > 1 an FP32 partial per
//   split, which a second kernel (split_reduce.hip) sums s = 0..S-1 in order.
//   The kernel boundary orders the two, so no workgroup waits on another and
//   no counter or fence is needed.
#include "internal.h"

namespace skinny {
namespace {

// Threads per workgroup a variant is compiled for: 16 chunks of weights and
// activations need 128 VGPRs of operands, so that variant gets 8 waves.
constexpr int mfma_max_threads(int chunks) { return chunks >= 16 ? 512 : 1024; }

// The arguments the main loop needs come first, the workgroup's wave count
// among them (the first 14 argument dwords arrive preloaded in SGPRs;
// blockDim would be a kernel-argument fetch).
template <int CHUNKS, int ACCS>
__global__ __launch_bounds__(mfma_max_threads(CHUNKS)) void gemm_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int M, int N, int K,
    int S, int groups, int F, int kw, int waves, uint16_t *__restrict__ y,
    float *__restrict__ partials, Publish pub) {
  const int lane = threadIdx.x & 63;
  if (S == 1 && blockIdx.x == 0 && threadIdx.x == 0) publish_stage_word(pub);
  const int wave = wave_index();
  const int threads = waves * 64;
  const int KW = waves / F;
  const int f = wave / KW, q = wave - f * KW;
  const int row = lane & 15;  // weight row (A) / token (B) of this lane
  const int grp = lane >> 4;  // which 8-wide K group of a 32-wide chunk

  // Workgroup -> (group, split).  Workgroups are dispatched to the 8 XCDs
  // round-robin, so ids congruent mod 8 share an XCD and its L2; when the
  // group count allows, the S workgroups of a group (which read the same
  // weight rows' neighbourhood and write one partial block) share one.
  int group, s;
  const int b = blockIdx.x;
  if ((groups & 7) == 0) {
    const int xcd = b & 7, slot = b >> 3;
    group = (slot / S) * 8 + xcd;
    s = slot % S;
  } else {
    group = b / S;
    s = b % S;
  }
  const int tile = group * F + f;

  // This workgroup's K range is [kbase, kbase + kslice).  Reads past K, or
  // past row M of x, fall outside their buffer resource and return zeros.
  const int kslice = KW * kw;
  const int kbase = s * kslice;
  const int k0 = kbase + q * kw + grp * 8;
  const __amdgpu_buffer_rsrc_t wres =
      buffer_rsrc(w + (size_t)tile * kTileN * K, (unsigned)(kTileN * K * 2));
  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(x, (unsigned)(M * K * 2));
  const int woff = (row * K + k0) * 2;

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

  // Activations: the workgroup's x[0..M)[kbase .. kbase + kslice) is read
  // once, with 16-byte loads running along K (a wave-wide load covers 1 KiB
  // of one token row), into LDS rows padded by 16 bytes so that the B-operand
  // reads below (16 tokens at one K offset) hit 16 different bank groups.
  // Segment j of the slice is token j / (kslice / 8), K offset 8 (j % ..);
  // a thread takes segments tid, tid + threads, ...: at most CHUNKS of them.
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t *xs = lds;
  const int xstride = kslice + 8;
  const int seg_row = kslice / 8;
  const int segs = M * seg_row;
  const int iters = (segs + threads - 1) / threads;
  u32x4 xv[CHUNKS];
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    if (i < iters) {
      const int j = threadIdx.x + i * threads;
      const int t = j / seg_row, k = kbase + (j - t * seg_row) * 8;
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(
          xres, (j < segs && k < K) ? (t * K + k) * 2 : kOutOfRange, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    if (i < iters) {
      const int j = threadIdx.x + i * threads;
      const int t = j / seg_row, c = j - t * seg_row;
      if (j < segs) *reinterpret_cast<u32x4 *>(xs + t * xstride + c * 8) = xv[i];
    }
  }
  __syncthreads();

  const bool token = row < M;
  const uint16_t *xsrow = xs + row * xstride + q * kw + grp * 8;
  f32x4 acc[ACCS];
#pragma unroll
  for (int a = 0; a < ACCS; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const u32x4 bv = token ? *reinterpret_cast<const u32x4 *>(xsrow + i * kMfmaK)
                           : u32x4{0, 0, 0, 0};
    acc[i % ACCS] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, wv[i]), __builtin_bit_cast(bf16x8, bv), acc[i % ACCS], 0, 0, 0);
  }
  f32x4 part = acc[0];
#pragma unroll
  for (int a = 1; a < ACCS; ++a) part += acc[a];

  // Waves q = 0..KW-1 of each tile in order, through LDS (the x slice is no
  // longer needed: the same LDS holds one 1 KiB partial per wave).
  if (KW > 1) {
    f32x4 *red = reinterpret_cast<f32x4 *>(lds);
    __syncthreads();
    red[wave * 64 + lane] = part;
    __syncthreads();
    if (q != 0) return;
    part = red[(f * KW) * 64 + lane];
    for (int v = 1; v < KW; ++v) part += red[(f * KW + v) * 64 + lane];
  }

  if (!token) return;
  const int col = tile * kTileN + grp * 4;
  if (S == 1) {
    const unsigned lo = f32_to_bf16(part[0]) | (f32_to_bf16(part[1]) << 16);
    const unsigned hi = f32_to_bf16(part[2]) | (f32_to_bf16(part[3]) << 16);
    *reinterpret_cast<uint2 *>(y + (size_t)row * N + col) = make_uint2(lo, hi);
    if (uint16_t *slot = publish_slot(pub, N))
      *reinterpret_cast<uint2 *>(slot + (size_t)row * N + col) =
          make_uint2(publish_pair(lo), publish_pair(hi));
  } else {
    // FP32 partial of split s: partials[s][token][feature]
    *reinterpret_cast<f32x4 *>(partials + ((size_t)s * M + row) * N + col) = part;
  }
}

using MfmaKernel = void (*)(const uint16_t *, const uint16_t *, int, int, int, int, int, int,
                            int, int, uint16_t *, float *, Publish);

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

// Allow every variant the largest dynamic LDS a launch may ask for.  Called
// once per device from skinny_init, outside any graph capture.
hipError_t mfma_prepare() {
  static const int kChunks[] = {1, 2, 4, 8, 16}, kAccs[] = {1, 2, 4};
  for (int c : kChunks)
    for (int a : kAccs) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(pick(c, a)),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)kMaxDynamicLds);
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

size_t mfma_lds_bytes(int M, const skinny_launch &l) {
  const int F = l.rows / kTileN, KW = l.waves / F;
  const size_t xbytes = (size_t)M * (KW * kMfmaK * l.chunks + 8) * sizeof(uint16_t);
  const size_t rbytes = (size_t)l.waves * 64 * sizeof(f32x4);
  return xbytes > rbytes ? xbytes : rbytes;
}

hipError_t launch_gemm_mfma(const uint16_t *x, const uint16_t *w, uint16_t *y,
                            int M, int N, int K, const skinny_launch &l,
                            const Workspace &ws, const Publish &pub, hipStream_t stream) {
  float *partials = ws.partials;
  MfmaKernel k = pick(l.chunks, l.accs);
  const int F = l.rows / kTileN;
  const int groups = N / l.rows;
  dim3 grid(groups * l.splits), block(64 * l.waves);
  hipLaunchKernelGGL(k, grid, block, mfma_lds_bytes(M, l), stream, x, w, M, N, K, l.splits,
                     groups, F, kMfmaK * l.chunks, l.waves, y, partials, pub);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || l.splits == 1) return e;
  return launch_split_reduce(partials, y, M, N, l.splits, pub, stream);
}

}  // namespace skinny
