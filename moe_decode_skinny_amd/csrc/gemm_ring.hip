// The layer-ring launch of the DOT2 GEMM: `count` independent small-M GEMMs
// y_i[M, N] = x_i[M, K] @ W_i[N, K]^T of one shape in one persistent launch,
// each weight matrix streamed while the previous GEMM is finished.
//
// The unpooler page's module description loads the weights before the
// dependency wait and the activations after it, so that one layer's weight
// stream overlaps the end of the previous kernel.  Within one launch the same
// ordering becomes a software pipeline per workgroup: the (item, block)
// tiles are taken in item order, j = blockIdx.x + n * gridDim.x, and while
// tile j is multiplied, reduced and stored, the weight loads of tile
// j + gridDim.x are already in flight.  Each tile's activations are loaded
// only when the tile starts, after the weights of the tile before it.
//
// Per tile the arithmetic is that of the single-call DOT2 kernel with
// splits = 1 at the same (rows, chunks, waves): the same lane products, the
// same wave reduce-scatter and the same wave order through LDS, so every
// item's y is bitwise identical to skinny_gemm_bf16_launch at that shape.
#include "dot2_device.h"

namespace skinny {
namespace {

using namespace dot2;

// Issue the loads of ROWS weight rows of one tile (or of nothing: bytes = 0
// turns every load into a zero read that touches no memory).
template <int ROWS, int CHUNKS>
__device__ __forceinline__ void load_weights(u32x4 (&wv)[ROWS][CHUNKS], const uint16_t *w,
                                             unsigned bytes, int K, int k0) {
  const __amdgpu_buffer_rsrc_t res = buffer_rsrc(w, bytes);
#pragma unroll
  for (int c = 0; c < CHUNKS; ++c) {
    const bool in = k0 + c * kDot2K < K;
#pragma unroll
    for (int r = 0; r < ROWS; ++r)
      wv[r][c] = __builtin_amdgcn_raw_buffer_load_b128(
          res, in ? (r * K + k0 + c * kDot2K) * 2 : kOutOfRange, 0, kCacheNT);
  }
}

struct RingShape {
  int count, M, N, K, groups, total, kw;
};

// One tile: activations of tile j, then the weights of tile j + G into
// `next`, then the products with `cur`, the reductions and the store.
// Returns true when tile j + G does not exist.  P selects the LDS buffer.
template <int ROWS, int CHUNKS, int MT, int P>
__device__ __forceinline__ bool ring_tile(const RingItems &items, const RingShape &sh, int j,
                                          u32x4 (&cur)[ROWS][CHUNKS],
                                          u32x4 (&next)[ROWS][CHUNKS],
                                          float (&red)[2][kDot2MaxThreads / 64][ROWS * MT],
                                          int lane, int wave, int waves, int k0) {
  const int item = j / sh.groups;
  const int f0 = (j - item * sh.groups) * ROWS;
  const int K = sh.K;

  const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(items.x[item], (unsigned)(sh.M * K * 2));
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
  const int jn = j + (int)gridDim.x;
  const bool more = jn < sh.total;
  {
    const int ni = more ? jn / sh.groups : item;
    const int nf0 = more ? (jn - ni * sh.groups) * ROWS : 0;
    load_weights<ROWS, CHUNKS>(next, items.w[ni] + (size_t)nf0 * K,
                               more ? (unsigned)(ROWS * K * 2) : 0u, K, k0);
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
      for (int t = 0; t < MT; ++t) acc[r][t] = dot8(cur[r][c], xv[t][c], acc[r][t]);

  constexpr int kOut = ROWS * MT;
  constexpr int kShift = 6 - log2i(kOut);
  float v[kOut];
#pragma unroll
  for (int r = 0; r < ROWS; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) v[r * MT + t] = acc[r][t];
  wave_reduce_scatter<kOut>(v, lane);

  // Buffer P of tile n is rewritten at tile n + 2, after the barrier of
  // tile n + 1, which wave 0 reaches only once it has read tile n's sums.
  if ((lane & ((1 << kShift) - 1)) == 0) red[P][wave][lane >> kShift] = v[0];
  __syncthreads();
  if (wave == 0 && lane < kOut) {
    const int r = lane / MT, t = lane % MT;
    float part = red[P][0][lane];
    for (int v2 = 1; v2 < waves; ++v2) part += red[P][v2][lane];
    if (t < sh.M) items.y[item][(size_t)t * sh.N + f0 + r] = (uint16_t)f32_to_bf16(part);
  }
  return !more;
}

template <int ROWS, int CHUNKS, int MT>
__global__ __launch_bounds__(kDot2MaxThreads) void gemm_dot2_ring_kernel(
    RingItems items, int count, int M, int N, int K, int groups, int kw) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int waves = blockDim.x >> 6;
  const RingShape sh{count, M, N, K, groups, count * groups, kw};
  const int k0 = wave * kw + lane * 8;
  __shared__ float red[2][kDot2MaxThreads / 64][ROWS * MT];

  // gridDim.x <= count * groups, so every workgroup has a first tile.
  int j = blockIdx.x;
  u32x4 wa[ROWS][CHUNKS], wb[ROWS][CHUNKS];
  {
    const int item = j / groups;
    const int f0 = (j - item * groups) * ROWS;
    load_weights<ROWS, CHUNKS>(wa, items.w[item] + (size_t)f0 * K, (unsigned)(ROWS * K * 2),
                               K, k0);
  }
  for (;;) {
    if (ring_tile<ROWS, CHUNKS, MT, 0>(items, sh, j, wa, wb, red, lane, wave, waves, k0)) break;
    j += gridDim.x;
    if (ring_tile<ROWS, CHUNKS, MT, 1>(items, sh, j, wb, wa, red, lane, wave, waves, k0)) break;
    j += gridDim.x;
  }
}

using RingKernel = void (*)(RingItems, int, int, int, int, int, int);

// Register budget per lane: two weight buffers 8 * ROWS * CHUNKS,
// activations 4 * MT * CHUNKS, sums ROWS * MT.
constexpr bool ring_fits(int rows, int chunks, int mt) {
  return 8 * rows * chunks + 4 * mt * chunks + rows * mt <= 160;
}

template <int R, int C, int T>
constexpr RingKernel ring_variant() {
  if constexpr (ring_fits(R, C, T)) return gemm_dot2_ring_kernel<R, C, T>;
  else return nullptr;
}

template <int R, int C>
RingKernel ring_pick_mt(int mt) {
  switch (mt) {
    case 1: return ring_variant<R, C, 1>();
    case 2: return ring_variant<R, C, 2>();
    case 4: return ring_variant<R, C, 4>();
    case 8: return ring_variant<R, C, 8>();
    case 16: return ring_variant<R, C, 16>();
  }
  return nullptr;
}

template <int R>
RingKernel ring_pick_chunks(int chunks, int mt) {
  switch (chunks) {
    case 1: return ring_pick_mt<R, 1>(mt);
    case 2: return ring_pick_mt<R, 2>(mt);
    case 4: return ring_pick_mt<R, 4>(mt);
  }
  return nullptr;
}

RingKernel ring_pick(int rows, int chunks, int mt) {
  switch (rows) {
    case 2: return ring_pick_chunks<2>(chunks, mt);
    case 4: return ring_pick_chunks<4>(chunks, mt);
    case 8: return ring_pick_chunks<8>(chunks, mt);
  }
  return nullptr;
}

}  // namespace

bool ring_variant_exists(int rows, int chunks, int mt) {
  return ring_pick(rows, chunks, mt) != nullptr;
}

hipError_t launch_gemm_ring(const RingItems &items, int count, int M, int N, int K,
                            const skinny_launch &l, int workgroups, hipStream_t stream) {
  RingKernel k = ring_pick(l.rows, l.chunks, dot2_token_tile(M));
  const int groups = N / l.rows;
  hipLaunchKernelGGL(k, dim3(workgroups), dim3(64 * l.waves), 0, stream, items, count, M, N,
                     K, groups, kDot2K * l.chunks);
  return hipGetLastError();
}

}  // namespace skinny
