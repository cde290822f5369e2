// The layer-ring launch: `count` independent small-M GEMMs
// y_i[M, N] = x_i[M, K] @ W_i[N, K]^T of one shape in one persistent launch,
// each weight matrix streamed while the previous GEMM is finished.  Three
// kernel families: DOT2 (VALU dot products, lanes along K), MFMA 16x16x32
// and the 16-block MFMA 4x4x4 (lanes along K, products on the matrix cores).
//
// On the unpooler page (module description) a kernel issues its weight loads
// ahead of the wait on the previous kernel and reads activations only after
// it, so one layer's weight stream overlaps the tail of the layer before.  Within one launch the same
// ordering becomes a software pipeline per workgroup: while one tile (item,
// output block) is multiplied, reduced and stored, the weight loads of the
// workgroup's next tile are already in flight.  Activations are loaded when a
// workgroup starts on an item, after the weights of the tile before.
//
// Tile order.  The count * groups tiles (groups = N / rows output blocks per
// item) are cut into segments of `seg` consecutive blocks of one item;
// workgroup b takes segment slots b, b + G, b + 2 G, ... (G workgroups) and
// the blocks of each segment in order.  A wave's activations depend only on
// the item and its K range, so they stay in registers for the whole segment:
// the activation traffic is that of one tile per segment.  Slots map to
// segments item-major, or (the XCD-local order) so that, when G is a
// multiple of 8, every segment of one item runs on one XCD (workgroups are dealt to the eight XCDs round-robin, so slot t
// runs on XCD t mod 8): slot t < local belongs to item (t mod 8) + 8 q, where
// q = (t div 8) div spi, for the first 8 (count div 8) items; the remaining
// items follow in item-major order.  Each item's activations then reach one
// XCD's L2 instead of all eight.  Any slot order computes the same tiles.
//
// Per tile the arithmetic is that of the single-call kernel of the same
// family with splits = 1 at the same (rows, chunks, waves, accs): the same
// products in the same order, the same cross-lane and cross-wave sums, so
// every item's y is bitwise identical to skinny_gemm_bf16_launch at that
// shape.  The MFMA ring differs from the single-call MFMA kernel only in
// where its B fragments come from: each wave loads them from global memory
// (L2) instead of a workgroup copy in LDS, so the LDS capacity does not limit
// K.
#include "blocks_device.h"
#include "dot2_device.h"
#include "internal.h"

namespace skinny {
namespace {

using namespace dot2;

// A workgroup's place in its tile walk and the tile it names.
struct RingWalk {
  int groups, seg, spi, segs;  // blocks per item, blocks per segment,
                               // segments per item, segments in all
  int local;                   // slots dealt XCD by XCD (0: item-major only)
  // Item and segment-in-item of slot s.
  __device__ void place(int s, int &item, int &j) const {
    if (s < local) {
      const int r = s >> 3, q = r / spi;
      item = (s & 7) + 8 * q;
      j = r - q * spi;
    } else {
      const int t = s - local, q = t / spi;
      item = local / spi + q;
      j = t - q * spi;
    }
  }
  __device__ int item(int s) const {
    int i, j;
    place(s, i, j);
    return i;
  }
  __device__ int block(int s, int sub) const {
    int i, j;
    place(s, i, j);
    return j * seg + sub;
  }
  // The tile after (s, sub) for this workgroup; false past the last one.
  __device__ bool advance(int &s, int &sub) const {
    if (++sub == seg) {
      sub = 0;
      s += (int)gridDim.x;
    }
    return s < segs;
  }
};

// The ring kernels' arguments: the first item's weights, the sizes, the wave
// count and the walk come first, the item table last.  The first 14
// argument dwords arrive preloaded in SGPRs, so a workgroup whose first tile
// belongs to item 0 (every tile of a single GEMM run as a walk) starts its
// weight stream without a kernel-argument fetch; the table is read as the
// walk goes on.
__device__ __forceinline__ const uint16_t *first_weights(const RingItems &items,
                                                         const uint16_t *w_first, int item) {
  return item == 0 ? w_first : items.w[item];
}

// ------------------------------------------------------------------ DOT2 ring
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

struct Dot2Args {
  int M, N, K;
};

// One tile (s, sub): activations if the segment starts here, then the
// weights of the next tile into `next`, then the products with `cur`, the
// reductions and the store.  Returns false after the workgroup's last tile.
// P selects the LDS buffer.
template <int ROWS, int CHUNKS, int MT, int WAVES, int P>
__device__ __forceinline__ bool dot2_ring_tile(const RingItems &items, const Dot2Args &a,
                                               const RingWalk &walk, int &s, int &sub,
                                               u32x4 (&cur)[ROWS][CHUNKS],
                                               u32x4 (&next)[ROWS][CHUNKS],
                                               u32x4 (&xv)[MT][CHUNKS],
                                               float (&red)[2][WAVES][ROWS * MT],
                                               int lane, int wave, int waves, int k0) {
  const int K = a.K;
  const int item = walk.item(s);
  const int f0 = walk.block(s, sub) * ROWS;

  if (sub == 0) {
    const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(items.x[item], (unsigned)(a.M * K * 2));
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) {
      const bool in = k0 + c * kDot2K < K;
#pragma unroll
      for (int t = 0; t < MT; ++t)
        xv[t][c] = __builtin_amdgcn_raw_buffer_load_b128(
            xres, in ? (t * K + k0 + c * kDot2K) * 2 : kOutOfRange, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  int ns = s, nsub = sub;
  const bool more = walk.advance(ns, nsub);
  {
    // Past the last tile, name the current one again (with no bytes): the
    // index arithmetic stays branch-free.
    const int cs = more ? ns : s, csub = more ? nsub : sub;
    load_weights<ROWS, CHUNKS>(next, items.w[walk.item(cs)] + (size_t)walk.block(cs, csub) * ROWS * K,
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
    const float part =
        sum_waves_in_order<WAVES, float>(waves, [&](int v2) { return red[P][v2][lane]; });
    if (t < a.M) items.y[item][(size_t)t * a.N + f0 + r] = (uint16_t)f32_to_bf16(part);
  }
  s = ns;
  sub = nsub;
  return more;
}

// THREADS: the launch bound, 512, or 1024 for the variants whose registers
// fit 16 waves (long K at one chunk per wave).
template <int ROWS, int CHUNKS, int MT, int THREADS>
__global__ __launch_bounds__(THREADS) void gemm_dot2_ring_kernel(
    const uint16_t *w_first, int M, int N, int K, int kw, int waves, int groups, int seg,
    int spi, int segs, int local, RingItems items) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const RingWalk walk{groups, seg, spi, segs, local};
  const Dot2Args a{M, N, K};
  const int k0 = wave * kw + lane * 8;
  __shared__ float red[2][THREADS / 64][ROWS * MT];

  // gridDim.x <= walk.segs, so every workgroup has a first tile.
  int s = blockIdx.x, sub = 0;
  u32x4 wa[ROWS][CHUNKS], wb[ROWS][CHUNKS], xv[MT][CHUNKS];
  load_weights<ROWS, CHUNKS>(
      wa, first_weights(items, w_first, walk.item(s)) + (size_t)walk.block(s, 0) * ROWS * K,
      (unsigned)(ROWS * K * 2), K, k0);
  for (;;) {
    if (!dot2_ring_tile<ROWS, CHUNKS, MT, THREADS / 64, 0>(items, a, walk, s, sub, wa, wb, xv,
                                                            red, lane, wave, waves, k0))
      break;
    if (!dot2_ring_tile<ROWS, CHUNKS, MT, THREADS / 64, 1>(items, a, walk, s, sub, wb, wa, xv,
                                                            red, lane, wave, waves, k0))
      break;
  }
}

using Dot2RingKernel = void (*)(const uint16_t *, int, int, int, int, int, int, int, int, int,
                                int, RingItems);

// Register budget per lane: two weight buffers 8 * ROWS * CHUNKS,
// activations 4 * MT * CHUNKS, sums ROWS * MT: at most 160 for 8 waves, 112
// for the 16-wave form (128 registers a lane, less the addresses).
constexpr int dot2_ring_regs(int rows, int chunks, int mt) {
  return 8 * rows * chunks + 4 * mt * chunks + rows * mt;
}

template <int R, int C, int T, int THREADS>
constexpr Dot2RingKernel dot2_ring_variant() {
  if constexpr (dot2_ring_regs(R, C, T) <= (THREADS > 512 ? 112 : 160))
    return gemm_dot2_ring_kernel<R, C, T, THREADS>;
  else
    return nullptr;
}

template <int R, int C, int THREADS>
Dot2RingKernel dot2_ring_pick_mt(int mt) {
  switch (mt) {
    case 1: return dot2_ring_variant<R, C, 1, THREADS>();
    case 2: return dot2_ring_variant<R, C, 2, THREADS>();
    case 4: return dot2_ring_variant<R, C, 4, THREADS>();
    case 8: return dot2_ring_variant<R, C, 8, THREADS>();
    case 16: return dot2_ring_variant<R, C, 16, THREADS>();
  }
  return nullptr;
}

template <int R, int THREADS>
Dot2RingKernel dot2_ring_pick_chunks(int chunks, int mt) {
  switch (chunks) {
    case 1: return dot2_ring_pick_mt<R, 1, THREADS>(mt);
    case 2: return dot2_ring_pick_mt<R, 2, THREADS>(mt);
    case 4: return dot2_ring_pick_mt<R, 4, THREADS>(mt);
  }
  return nullptr;
}

template <int THREADS>
Dot2RingKernel dot2_ring_pick_rows(int rows, int chunks, int mt) {
  switch (rows) {
    case 2: return dot2_ring_pick_chunks<2, THREADS>(chunks, mt);
    case 4: return dot2_ring_pick_chunks<4, THREADS>(chunks, mt);
    case 8: return dot2_ring_pick_chunks<8, THREADS>(chunks, mt);
  }
  return nullptr;
}

// The variant for a launch of `waves` waves: the 8-wave form up to 8 waves,
// the 16-wave form beyond.
Dot2RingKernel dot2_ring_pick(int rows, int chunks, int mt, int waves) {
  if (waves <= kDot2MaxThreads / 64) return dot2_ring_pick_rows<kDot2MaxThreads>(rows, chunks, mt);
  if (waves <= 16) return dot2_ring_pick_rows<1024>(rows, chunks, mt);
  return nullptr;
}

// --------------------------------------------------------- 16-block MFMA ring
// Per tile the arithmetic of the single-call kernel (blocks_device.h) at
// splits = 1: wave w owns K [w kw, (w + 1) kw), kw = 128 CHUNKS, of the
// tile's 4 R4 rows; the pipeline is the DOT2 ring's.
template <int R4, int CHUNKS, int Q, int WAVES, int P>
__device__ __forceinline__ bool blocks_ring_tile(const RingItems &items, const Dot2Args &a,
                                                 const RingWalk &walk, int &s, int &sub,
                                                 u32x4 (&cur)[R4][CHUNKS],
                                                 u32x4 (&next)[R4][CHUNKS],
                                                 u32x4 (&xv)[Q][CHUNKS],
                                                 float (&red)[2][WAVES][blocks::kOutputs<R4, Q>],
                                                 int lane, int wave, int waves, int k0) {
  constexpr int ROWS = 4 * R4;
  const int K = a.K;
  const int item = walk.item(s);
  const int f0 = walk.block(s, sub) * ROWS;

  if (sub == 0) {
    // The activation offsets are recomputed here (a few adds once per
    // segment) rather than held in registers across the tile loop.
    int kx = k0;
    asm volatile("" : "+v"(kx));
    blocks::load_sets<Q, CHUNKS, 0>(xv, buffer_rsrc(items.x[item], (unsigned)(a.M * K * 2)), K,
                                    kx);
  }
  __builtin_amdgcn_sched_barrier(0);
  int ns = s, nsub = sub;
  const bool more = walk.advance(ns, nsub);
  {
    const int cs = more ? ns : s, csub = more ? nsub : sub;
    blocks::load_sets<R4, CHUNKS, kCacheNT>(
        next,
        buffer_rsrc(items.w[walk.item(cs)] + (size_t)walk.block(cs, csub) * ROWS * K,
                    more ? (unsigned)(ROWS * K * 2) : 0u),
        K, k0);
  }
  __builtin_amdgcn_sched_barrier(0);

  // Into the MFMA layout: the segment's activations once, this tile's weights.
  if (sub == 0) blocks::transpose_sets<Q, CHUNKS>(xv, lane);
  blocks::transpose_sets<R4, CHUNKS>(cur, lane);
  f32x4 acc[Q][R4];
  blocks::products<R4, CHUNKS, Q>(cur, xv, acc);
  // Buffer P: as in the DOT2 ring.
  blocks::reduce_to_lds<R4, Q>(acc, red[P][wave], lane);
  __syncthreads();
  if (wave == 0) {
    constexpr int kOut = blocks::kOutputs<R4, Q>;
#pragma unroll
    for (int o0 = 0; o0 < kOut; o0 += 64) {
      const int o = o0 + lane;
      if (o < kOut) {
        const float part =
            sum_in_order<WAVES, float>(waves, [&](int v2) { return red[P][v2][o]; });
        const int t = blocks::output_token(o, R4), r = blocks::output_row(o, R4);
        if (t < a.M) items.y[item][(size_t)t * a.N + f0 + r] = (uint16_t)f32_to_bf16(part);
      }
    }
  }
  s = ns;
  sub = nsub;
  return more;
}

template <int R4, int CHUNKS, int Q, int THREADS>
__global__ __launch_bounds__(THREADS) void gemm_blocks_ring_kernel(
    const uint16_t *w_first, int M, int N, int K, int kw, int waves, int groups, int seg,
    int spi, int segs, int local, RingItems items) {
  constexpr int ROWS = 4 * R4;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const RingWalk walk{groups, seg, spi, segs, local};
  const Dot2Args a{M, N, K};
  const int k0 = wave * kw + lane * 8;
  __shared__ float red[2][THREADS / 64][blocks::kOutputs<R4, Q>];

  // gridDim.x <= walk.segs, so every workgroup has a first tile.
  int s = blockIdx.x, sub = 0;
  u32x4 wa[R4][CHUNKS], wb[R4][CHUNKS], xv[Q][CHUNKS];
  blocks::load_sets<R4, CHUNKS, kCacheNT>(
      wa, buffer_rsrc(first_weights(items, w_first, walk.item(s)) +
                          (size_t)walk.block(s, 0) * ROWS * K,
                      (unsigned)(ROWS * K * 2)),
      K, k0);
  for (;;) {
    if (!blocks_ring_tile<R4, CHUNKS, Q, THREADS / 64, 0>(items, a, walk, s, sub, wa, wb, xv,
                                                          red, lane, wave, waves, k0))
      break;
    if (!blocks_ring_tile<R4, CHUNKS, Q, THREADS / 64, 1>(items, a, walk, s, sub, wb, wa, xv,
                                                          red, lane, wave, waves, k0))
      break;
  }
}

// Register budget per lane: two weight buffers 8 * R4 * CHUNKS, activations
// 4 * Q * CHUNKS, sums 4 * Q * R4: at most 112 for 16 waves (128 registers a
// lane), 224 for 8 waves (256 a lane; the largest forms compile to 230-238
// registers without spilling).
constexpr int blocks_ring_regs(int r4, int chunks, int q) {
  return 8 * r4 * chunks + 4 * q * chunks + 4 * q * r4;
}

template <int R4, int C, int Q, int THREADS>
constexpr Dot2RingKernel blocks_ring_variant() {
  if constexpr (blocks_ring_regs(R4, C, Q) <= (THREADS > 512 ? 112 : 224))
    return gemm_blocks_ring_kernel<R4, C, Q, THREADS>;
  else
    return nullptr;
}

template <int R4, int C, int THREADS>
Dot2RingKernel blocks_ring_pick_q(int q) {
  switch (q) {
    case 1: return blocks_ring_variant<R4, C, 1, THREADS>();
    case 2: return blocks_ring_variant<R4, C, 2, THREADS>();
    case 4: return blocks_ring_variant<R4, C, 4, THREADS>();
  }
  return nullptr;
}

template <int R4, int THREADS>
Dot2RingKernel blocks_ring_pick_chunks(int chunks, int q) {
  switch (chunks) {
    case 4: return blocks_ring_pick_q<R4, 4, THREADS>(q);
    case 8: return blocks_ring_pick_q<R4, 8, THREADS>(q);
  }
  return nullptr;
}

template <int THREADS>
Dot2RingKernel blocks_ring_pick_rows(int rows, int chunks, int q) {
  switch (rows) {
    case 4: return blocks_ring_pick_chunks<1, THREADS>(chunks, q);
    case 8: return blocks_ring_pick_chunks<2, THREADS>(chunks, q);
  }
  return nullptr;
}

Dot2RingKernel blocks_ring_pick(int rows, int chunks, int q, int waves) {
  if (waves >= 1 && waves <= 8) return blocks_ring_pick_rows<512>(rows, chunks, q);
  if (waves <= 16) return blocks_ring_pick_rows<1024>(rows, chunks, q);
  return nullptr;
}

// ------------------------------------------------------------------ MFMA ring
// A block is F MFMA tiles of 16 features; waves (f, q), q < KW, and wave
// (f, q) owns K [q kw, (q + 1) kw), kw = 32 CHUNKS, of tile block * F + f.
// Lane layout of v_mfma_f32_16x16x32_bf16 as in the single-call kernel:
// A lane l = W[row l % 16][k + 8 (l / 16) ..], B lane l = x[token l % 16][same
// k], D lane l = features 4 (l / 16) + 0..3 of token l % 16.
//
// Loading A fragments straight from memory makes every load instruction touch
// 16 rows (64 bytes of each).  The staged form (SKINNY_PATH_MFMA_LDS) loads
// the wave's 16 x kw weight slice row by row instead (one instruction covers
// 1 KiB of whole-row pieces), writes it to the wave's own padded LDS region
// and reads the A fragments back from there.  The MFMA operands, and so the
// results, are the same.
constexpr int mfma_ring_threads(int chunks) { return chunks >= 16 ? 512 : 1024; }

template <int CHUNKS>
__device__ __forceinline__ void load_tile_weights(u32x4 (&wv)[CHUNKS], const uint16_t *w,
                                                  unsigned bytes, int K, int k0, int row) {
  const __amdgpu_buffer_rsrc_t res = buffer_rsrc(w, bytes);
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i)
    wv[i] = __builtin_amdgcn_raw_buffer_load_b128(
        res, k0 + i * kMfmaK < K ? (row * K + k0 + i * kMfmaK) * 2 : kOutOfRange, 0, kCacheNT);
}

// The staged layout: the wave's slice is 16 rows x 4 CHUNKS pieces of 16
// bytes; load i, lane l takes piece e = 64 i + l in row-major order.  In LDS
// a row is 4 CHUNKS + 1 pieces long: the pad piece spreads the 16 rows read
// by one fragment load over different banks, and the fragment offsets of the
// chunks stay constants of the instruction (a swizzled layout without the pad
// measured slower).
template <int CHUNKS>
struct Staging {
  static constexpr int kRow = 4 * CHUNKS + 1;    // LDS row stride in pieces
  static constexpr int kLog = log2i(4 * CHUNKS);  // pieces per row, log2
  static constexpr int kPieces = 16 * kRow;      // LDS pieces per wave
  __device__ static int slot(int r, int p) { return r * kRow + p; }
};

template <int CHUNKS>
__device__ __forceinline__ void load_tile_rows(u32x4 (&wv)[CHUNKS], const uint16_t *w,
                                               unsigned bytes, int K, int kq, int lane) {
  using St = Staging<CHUNKS>;
  const __amdgpu_buffer_rsrc_t res = buffer_rsrc(w, bytes);
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i) {
    const int e = i * 64 + lane;
    const int k = kq + (e & (4 * CHUNKS - 1)) * 8;
    wv[i] = __builtin_amdgcn_raw_buffer_load_b128(
        res, k < K ? ((e >> St::kLog) * K + k) * 2 : kOutOfRange, 0, kCacheNT);
  }
}

// Orders one wave's LDS writes before its reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct MfmaArgs {
  int M, N, K, F, KW, waves;
};

template <int CHUNKS, int ACCS, bool STAGED, int P>
__device__ __forceinline__ bool mfma_ring_tile(const RingItems &items, const MfmaArgs &a,
                                               const RingWalk &walk, int &s, int &sub,
                                               u32x4 (&cur)[CHUNKS], u32x4 (&next)[CHUNKS],
                                               u32x4 (&xv)[CHUNKS], u32x4 *stage, f32x4 *red,
                                               int lane, int wave, int f, int q, int kq) {
  const int row = lane & 15, grp = lane >> 4;
  const int K = a.K;
  const int k0 = kq + grp * 8;
  const int item = walk.item(s);
  const int tile = walk.block(s, sub) * a.F + f;

  // B fragments x[row][k0 + 32 i ..] when the segment starts; rows >= M and
  // K past the end read zeros.
  if (sub == 0) {
    const __amdgpu_buffer_rsrc_t xres = buffer_rsrc(items.x[item], (unsigned)(a.M * K * 2));
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i)
      xv[i] = __builtin_amdgcn_raw_buffer_load_b128(
          xres, k0 + i * kMfmaK < K ? (row * K + k0 + i * kMfmaK) * 2 : kOutOfRange, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  int ns = s, nsub = sub;
  const bool more = walk.advance(ns, nsub);
  {
    const int cs = more ? ns : s, csub = more ? nsub : sub;  // as in the DOT2 ring
    const uint16_t *wn = items.w[walk.item(cs)] +
                         (size_t)(walk.block(cs, csub) * a.F + f) * kTileN * K;
    const unsigned bytes = more ? (unsigned)(kTileN * K * 2) : 0u;
    if constexpr (STAGED)
      load_tile_rows<CHUNKS>(next, wn, bytes, K, kq, lane);
    else
      load_tile_weights<CHUNKS>(next, wn, bytes, K, k0, row);
  }
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (STAGED) {
    using St = Staging<CHUNKS>;
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int e = i * 64 + lane;
      stage[St::slot(e >> St::kLog, e & (4 * CHUNKS - 1))] = cur[i];
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) cur[i] = stage[St::slot(row, 4 * i + grp)];
  }

  f32x4 acc[ACCS];
#pragma unroll
  for (int c = 0; c < ACCS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < CHUNKS; ++i)
    acc[i % ACCS] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, cur[i]), __builtin_bit_cast(bf16x8, xv[i]), acc[i % ACCS], 0,
        0, 0);
  f32x4 part = acc[0];
#pragma unroll
  for (int c = 1; c < ACCS; ++c) part += acc[c];

  // Waves q = 0..KW-1 of each tile in order through LDS buffer P (rewritten
  // two tiles later, after a barrier that follows every read of it).
  if (a.KW > 1) {
    f32x4 *buf = red + P * a.waves * 64;
    buf[wave * 64 + lane] = part;
    __syncthreads();
    if (q == 0) {
      part = buf[f * a.KW * 64 + lane];
      for (int v = 1; v < a.KW; ++v) part += buf[(f * a.KW + v) * 64 + lane];
    }
  }
  if (q == 0 && row < a.M) {
    const int col = tile * kTileN + grp * 4;
    const unsigned lo = f32_to_bf16(part[0]) | (f32_to_bf16(part[1]) << 16);
    const unsigned hi = f32_to_bf16(part[2]) | (f32_to_bf16(part[3]) << 16);
    *reinterpret_cast<uint2 *>(items.y[item] + (size_t)row * a.N + col) = make_uint2(lo, hi);
  }
  s = ns;
  sub = nsub;
  return more;
}

// Dynamic LDS: the staged form's per-wave regions, then the two reduction
// buffers of waves x 64 lanes x 16 bytes.
template <int CHUNKS, int ACCS, bool STAGED>
__global__ __launch_bounds__(mfma_ring_threads(CHUNKS)) void gemm_mfma_ring_kernel(
    const uint16_t *w_first, int M, int N, int K, int kw, int waves, int F, int groups,
    int seg, int spi, int segs, int local, RingItems items) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const RingWalk walk{groups, seg, spi, segs, local};
  const int KW = waves / F;
  const int f = wave / KW, q = wave - f * KW;
  const MfmaArgs a{M, N, K, F, KW, waves};
  const int kq = q * kw;
  extern __shared__ __align__(16) u32x4 ring_lds[];
  constexpr int kStage = STAGED ? Staging<CHUNKS>::kPieces : 0;
  u32x4 *stage = ring_lds + wave * kStage;
  f32x4 *red = reinterpret_cast<f32x4 *>(ring_lds + waves * kStage);

  int s = blockIdx.x, sub = 0;  // gridDim.x <= walk.segs
  u32x4 wa[CHUNKS], wb[CHUNKS], xv[CHUNKS];
  {
    const uint16_t *w0 = first_weights(items, w_first, walk.item(s)) +
                         (size_t)(walk.block(s, 0) * F + f) * kTileN * K;
    if constexpr (STAGED)
      load_tile_rows<CHUNKS>(wa, w0, (unsigned)(kTileN * K * 2), K, kq, lane);
    else
      load_tile_weights<CHUNKS>(wa, w0, (unsigned)(kTileN * K * 2), K, kq + (lane >> 4) * 8,
                                lane & 15);
  }
  for (;;) {
    if (!mfma_ring_tile<CHUNKS, ACCS, STAGED, 0>(items, a, walk, s, sub, wa, wb, xv, stage, red,
                                                  lane, wave, f, q, kq))
      break;
    if (!mfma_ring_tile<CHUNKS, ACCS, STAGED, 1>(items, a, walk, s, sub, wb, wa, xv, stage, red,
                                                  lane, wave, f, q, kq))
      break;
  }
}

using MfmaRingKernel = void (*)(const uint16_t *, int, int, int, int, int, int, int, int, int,
                                int, int, RingItems);

template <int C, bool STAGED>
MfmaRingKernel mfma_ring_pick_accs(int accs) {
  switch (accs) {
    case 1: return gemm_mfma_ring_kernel<C, 1, STAGED>;
    case 2: return gemm_mfma_ring_kernel<C, 2, STAGED>;
  }
  return nullptr;
}

MfmaRingKernel mfma_ring_pick(int chunks, int accs, bool staged) {
  if (staged) {
    switch (chunks) {
      case 2: return mfma_ring_pick_accs<2, true>(accs);
      case 4: return mfma_ring_pick_accs<4, true>(accs);
      case 8: return mfma_ring_pick_accs<8, true>(accs);
      case 16: return mfma_ring_pick_accs<16, true>(accs);
    }
    return nullptr;
  }
  switch (chunks) {
    case 1: return mfma_ring_pick_accs<1, false>(accs);
    case 2: return mfma_ring_pick_accs<2, false>(accs);
    case 4: return mfma_ring_pick_accs<4, false>(accs);
    case 8: return mfma_ring_pick_accs<8, false>(accs);
    case 16: return mfma_ring_pick_accs<16, false>(accs);
  }
  return nullptr;
}

size_t stage_pieces(int chunks) {
  switch (chunks) {
    case 2: return Staging<2>::kPieces;
    case 4: return Staging<4>::kPieces;
    case 8: return Staging<8>::kPieces;
    case 16: return Staging<16>::kPieces;
  }
  return 0;
}

}  // namespace

bool ring_variant_exists(int rows, int chunks, int mt, int waves) {
  return dot2_ring_pick(rows, chunks, mt, waves) != nullptr;
}

bool blocks_ring_variant_exists(int rows, int chunks, int q, int waves) {
  return blocks_ring_pick(rows, chunks, q, waves) != nullptr;
}

bool mfma_ring_variant_exists(int chunks, int accs, bool staged) {
  return mfma_ring_pick(chunks, accs, staged) != nullptr;
}

int mfma_ring_max_waves(int chunks) { return mfma_ring_threads(chunks) / 64; }

size_t mfma_ring_lds_bytes(const skinny_launch &l) {
  const size_t stage = l.path == SKINNY_PATH_MFMA_LDS ? stage_pieces(l.chunks) : 0;
  return (size_t)l.waves * (stage + 2 * 64) * sizeof(u32x4);
}

hipError_t ring_prepare() {
  static const int kChunks[] = {1, 2, 4, 8, 16}, kAccs[] = {1, 2};
  for (int staged = 0; staged < 2; ++staged)
    for (int c : kChunks)
      for (int a : kAccs) {
        MfmaRingKernel k = mfma_ring_pick(c, a, staged != 0);
        if (!k) continue;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)kMaxDynamicLds);
        if (e != hipSuccess) return e;
      }
  return hipSuccess;
}

hipError_t launch_gemm_ring(const RingItems &items, int count, int M, int N, int K,
                            const skinny_ring_launch &r, hipStream_t stream) {
  const skinny_launch &l = r.gemm;
  const int groups = N / l.rows;
  const int spi = groups / r.segment;
  // XCD-local slots only when the workgroups divide evenly over the 8 XCDs.
  const int local =
      r.order == SKINNY_RING_XCD_LOCAL && r.workgroups % 8 == 0 ? (count / 8) * 8 * spi : 0;
  const int segs = count * spi;
  if (l.path == SKINNY_PATH_MFMA || l.path == SKINNY_PATH_MFMA_LDS) {
    hipLaunchKernelGGL(mfma_ring_pick(l.chunks, l.accs, l.path == SKINNY_PATH_MFMA_LDS),
                       dim3(r.workgroups), dim3(64 * l.waves), mfma_ring_lds_bytes(l), stream,
                       items.w[0], M, N, K, kMfmaK * l.chunks, l.waves, l.rows / kTileN, groups,
                       r.segment, spi, segs, local, items);
  } else if (l.path == SKINNY_PATH_MFMA_4X4) {
    hipLaunchKernelGGL(blocks_ring_pick(l.rows, l.chunks, blocks_token_sets(M), l.waves),
                       dim3(r.workgroups), dim3(64 * l.waves), 0, stream, items.w[0], M, N, K,
                       kBlockK * l.chunks, l.waves, groups, r.segment, spi, segs, local, items);
  } else {
    hipLaunchKernelGGL(dot2_ring_pick(l.rows, l.chunks, dot2_token_tile(M), l.waves),
                       dim3(r.workgroups), dim3(64 * l.waves), 0, stream, items.w[0], M, N, K,
                       kDot2K * l.chunks, l.waves, groups, r.segment, spi, segs, local, items);
  }
  return hipGetLastError();
}

}  // namespace skinny
