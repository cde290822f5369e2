// The 16-block MFMA path of the small-M decode GEMM y[M, N] = x[M, K] @ W[N, K]^T
// (unpooler page, module description): lanes run along K as in the DOT2
// path, the products go to the matrix cores (v_mfma_f32_4x4x4_16b_bf16; the
// lane layout and the order of the sums are in blocks_device.h).
//   wave w of workgroup (group, h, s) owns K range (s * waves + w) * kw,
//   kw = 128 * CHUNKS (CHUNKS 4 or 8: whole 512-K load groups), of the
//   workgroup's 4 * R4 weight rows, and tokens 4 Q h .. 4 Q h + 4 Q - 1 (Q
//   sets of 4; with H = 1 token group, all M tokens); the activations are
//   loaded first, then the weights, and both are transposed into the MFMA
//   layout inside each 4-lane group, activations first.
// Token groups (H > 1) split the activations instead of K: each workgroup
// pulls 1 / H of them through its compute unit and all of its rows'
// weights, which the H workgroups of a row group (dealt to one XCD) share
// through that XCD's L2, so HBM still streams W once.  No partials and no
// hand-off: a token's sums are the same instructions in the same order as
// with H = 1, so the bits are too.
// Load order: the pages load weights ahead of the activations so that the
// weight stream can start before the previous kernel ends.  Inside one
// launch on gfx950 the activations (L2 hits after the first compute unit of
// an XCD fetched them) are issued first instead: vector loads complete in
// issue order, so their transposes, four VALU instructions per loaded dword
// and most of a wave's VALU work at 9..16 tokens, then run while the weights
// are still streaming from HBM instead of after them.  The arithmetic and
// its order are the same either way.
// Reduction in an order fixed by the launch shape (module description): the
// 16 blocks across lanes, waves 0..waves-1 in order through LDS, and with
// S > 1 an FP32 partial per split, the splits summed s = 0..S-1 in order by
// the last of an output block's S workgroups to finish (see block_handoff),
// or, for launches with more output blocks than the hand-off counters
// cover, by the split_reduce kernel; both give the same bits.
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

// One wave's K slice of split s: wave v of the workgroup covers K from
// (s * waves + v) * kw.  Loads (activations first), transposes and products,
// then the 16-block sum into red[v] (kOutputs values).
template <int R4, int CHUNKS, int Q>
__device__ __forceinline__ void wave_slice(const uint16_t *__restrict__ x,
                                           const uint16_t *__restrict__ w, int M, int K, int f0,
                                           int s, int v, int waves, int kw, int lane,
                                           float *red) {
  constexpr int ROWS = 4 * R4;
  const int k0 = (s * waves + v) * kw + lane * 8;
  u32x4 wv[R4][CHUNKS], xv[Q][CHUNKS];
  load_sets<Q, CHUNKS, 0>(xv, buffer_rsrc(x, (unsigned)(M * K * 2)), K, k0);
  __builtin_amdgcn_sched_barrier(0);
  load_sets<R4, CHUNKS, kCacheNT>(wv, buffer_rsrc(w + (size_t)f0 * K, (unsigned)(ROWS * K * 2)),
                                  K, k0);
  __builtin_amdgcn_sched_barrier(0);
  transpose_sets<Q, CHUNKS>(xv, lane);
  __builtin_amdgcn_sched_barrier(0);
  transpose_sets<R4, CHUNKS>(wv, lane);
  f32x4 acc[Q][R4];
  products<R4, CHUNKS, Q>(wv, xv, acc);
  reduce_to_lds<R4, Q>(acc, red, lane);
}

// Output o = i * 64 + lane (i < kPer) summed over the waves' slices in wave
// order (waves <= kWaves).
template <int kOut, int kPer, int kWaves>
__device__ __forceinline__ void sum_waves(float (*red)[kOut], int waves, int lane, float *part) {
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int o = i * 64 + lane, oc = o < kOut ? o : 0;
    const float p = sum_in_order<kWaves, float>(waves, [&](int v) { return red[v][oc]; });
    part[i] = o < kOut ? p : 0.f;
  }
}

// Splits 0..S-1 summed in order (S = 2, 4, 8 or 16), with the S terms
// loaded before the first add and no load past S.
template <typename Term>
__device__ __forceinline__ float sum_splits(int S, Term term) {
  switch (S) {
    case 2: return sum_in_order<2, float>(2, term);
    case 4: return sum_in_order<4, float>(4, term);
    case 8: return sum_in_order<8, float>(8, term);
    default: return sum_in_order<16, float>(16, term);
  }
}

// The split hand-off of one output block (S > 1), in wave 0 of each of its S
// workgroups: store this split's partial, then mark the arrival in the
// block's counter word (bit s, and bit 16 + XCD id), one atomic OR whose
// returned value tells the last arriver.  Returns true in the last one.
// The S workgroups of a block are dealt to one XCD (ids congruent mod 8, see
// the kernel), so partials pass through that XCD's L2: plain stores waited
// for before the atomic, and in the last arriver plain loads.  Those loads
// cannot meet a stale line in this CU's L1: a block's slot is read once per
// launch, by its last arriver, after every store to it; slots of different
// blocks share no cache line (S * kOut floats with S even and kOut a
// multiple of 16); and the compute units' L1 caches are invalidated when a
// launch starts.  (The L1 invalidate below matters only in thread-group-split
// mode; outside it, measured with polling loads, it does not drop lines.)
// *mixed is set when the arrivals came from more than one XCD, whose L2s do
// not see each other's stores; the caller then recomputes the other splits
// instead of reading them.  The counter word is reset by the last arriver,
// so it is zero again for the next call (no memset).
template <int kPer>
__device__ __forceinline__ bool block_handoff(float *__restrict__ slots,
                                              unsigned *__restrict__ counter, int S, int s,
                                              int kOut, int lane, const float *part,
                                              bool *mixed) {
  const __amdgpu_buffer_rsrc_t res = buffer_rsrc(slots, (unsigned)(S * kOut * 4));
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int o = i * 64 + lane;
    if (o < kOut)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(part[i]), res, (s * kOut + o) * 4, 0,
                                            0);
  }
  // every lane's stores have reached L2 before the arrival is marked
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  const unsigned xcc = __builtin_amdgcn_s_getreg(kHwRegXccId) & 7u;
  const unsigned mine = (1u << s) | (1u << (16 + xcc));
  unsigned old = 0;
  if (lane == 0)
    old = __hip_atomic_fetch_or(counter, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned all = (unsigned)__builtin_amdgcn_readfirstlane((int)old) | mine;
  if ((all & 0xFFFFu) != (1u << S) - 1u) return false;
  *mixed = __builtin_popcount(all >> 16) != 1;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  asm volatile("buffer_inv sc0" ::: "memory");  // see above: thread-group-split mode
  if (lane == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// mode: bit 0 the splits are summed in the kernel (counters and partial
// slots valid), bit 1 that hand-off always recomputes (test hook).  The
// arguments the main loop needs come first and include the wave count, so
// the start reads no implicit argument (blockDim).  Unlike the other GEMM
// kernels this one is built without argument preloading: its 16-token
// launch measured slower with it.
constexpr int kModeHandoff = 1, kModeRecompute = 2;

template <int R4, int CHUNKS, int Q, int THREADS>
__global__ __launch_bounds__(THREADS) void gemm_blocks_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w, int M, int N, int K,
    int S, int H, int groups, int kw, int waves, int mode, uint16_t *__restrict__ y,
    float *__restrict__ partials, unsigned *__restrict__ counters, Publish pub) {
  constexpr int kOut = kOutputs<R4, Q>, kPer = (kOut + 63) / 64;
  const int lane = threadIdx.x & 63;
  if ((S == 1 || (mode & kModeHandoff)) && blockIdx.x == 0 && threadIdx.x == 0)
    publish_stage_word(pub);
  const int wave = wave_index();

  // Workgroup -> (row group, token group h, split s): workgroups are dealt
  // to the XCDs round-robin (ids congruent mod 8 share an XCD, also when the
  // part has fewer XCDs), so with a row-group count divisible by 8 the H * S
  // workgroups of a row group share an XCD and its L2.
  const int per = H * S;
  int group, j;
  const int b = blockIdx.x;
  if ((groups & 7) == 0) {
    const int xcd = b & 7, slot = b >> 3;
    group = (slot / per) * 8 + xcd;
    j = slot % per;
  } else {
    group = b / per;
    j = b % per;
  }
  const int h = j / S, s = j % S;
  const int f0 = group * 4 * R4;
  const int t0 = 4 * Q * h;           // first token of this workgroup
  const int Mh = min(4 * Q, M - t0);  // its token count, >= 1
  const uint16_t *xh = x + (size_t)t0 * K;
  const int ob = group * H + h;       // output block (row group, token group)

  __shared__ float red[THREADS / 64][kOut];
  wave_slice<R4, CHUNKS, Q>(xh, w, Mh, K, f0, s, wave, waves, kw, lane, red[wave]);
  __syncthreads();
  if (wave != 0) return;
  float part[kPer];
  sum_waves<kOut, kPer, THREADS / 64>(red, waves, lane, part);

  if (S > 1 && !(mode & kModeHandoff)) {  // FP32 partial of split s for split_reduce: [s][token][feature]
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int o = i * 64 + lane;
      if (o >= kOut) break;
      const int t = output_token(o, R4), r = output_row(o, R4);
      if (t < Mh) partials[((size_t)s * M + t0 + t) * N + f0 + r] = part[i];
    }
    return;
  }
  if (S > 1) {
    bool mixed = false;
    if (!block_handoff<kPer>(partials + (size_t)ob * S * kOut,
                             counters + (size_t)ob * kCounterStride, S, s, kOut, lane, part,
                             &mixed))
      return;
    float sum[kPer];
    if (!mixed && !(mode & kModeRecompute)) {
      const __amdgpu_buffer_rsrc_t res =
          buffer_rsrc(partials + (size_t)ob * S * kOut, (unsigned)(S * kOut * 4));
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int oc = i * 64 + lane < kOut ? i * 64 + lane : 0;
        sum[i] = sum_splits(S, [&](int s2) {
          // the other splits' partials (sc0 policy; no stale L1 line, see
          // block_handoff)
          return s2 == s ? part[i]
                         : __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                               res, (s2 * kOut + oc) * 4, 0, 1));
        });
      }
    } else {
      // Splits on several XCDs: this wave recomputes every other split's
      // wave slices itself (the other waves have left; their LDS rows are
      // free), with the instructions the other workgroups ran, and sums
      // them in the same orders: the same bits.
      for (int s2 = 0; s2 < S; ++s2) {
        float p2[kPer];
        if (s2 == s) {
#pragma unroll
          for (int i = 0; i < kPer; ++i) p2[i] = part[i];
        } else {
          for (int v = 0; v < waves; ++v)
            wave_slice<R4, CHUNKS, Q>(xh, w, Mh, K, f0, s2, v, waves, kw, lane, red[v]);
          sum_waves<kOut, kPer, THREADS / 64>(red, waves, lane, p2);
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) sum[i] = s2 == 0 ? p2[i] : sum[i] + p2[i];
      }
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) part[i] = sum[i];
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int o = i * 64 + lane;
    if (o >= kOut) break;
    const int t = output_token(o, R4), r = output_row(o, R4);
    if (t >= Mh) continue;
    const unsigned bits = f32_to_bf16(part[i]);
    if (S == 1)
      store_out_device(y + (size_t)(t0 + t) * N + f0 + r, bits);
    else
      y[(size_t)(t0 + t) * N + f0 + r] = (uint16_t)bits;
    if (uint16_t *slot = publish_slot(pub, N))
      slot[(size_t)(t0 + t) * N + f0 + r] = (uint16_t)publish_bits(bits);
  }
}

using BlocksKernel = void (*)(const uint16_t *, const uint16_t *, int, int, int, int, int, int,
                              int, int, int, uint16_t *, float *, unsigned *, Publish);

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

int blocks_group_token_sets(int M, int H) {
  if (H != 1 && H != 2 && H != 4) return 0;
  const int q = blocks_token_sets((M + H - 1) / H);
  return q && (M + 4 * q - 1) / (4 * q) == H ? q : 0;
}

bool blocks_variant_exists(int rows, int chunks, int q, int waves) {
  return waves >= 1 && waves <= kBlocksMaxWaves && pick(rows, chunks, q, waves) != nullptr;
}

hipError_t launch_gemm_blocks(const uint16_t *x, const uint16_t *w, uint16_t *y, int M,
                              int N, int K, const skinny_launch &l, const Workspace &ws,
                              const Publish &pub, hipStream_t stream) {
  const int H = l.accs;  // token groups
  const int q = blocks_group_token_sets(M, H);
  BlocksKernel k = pick(l.rows, l.chunks, q, l.waves);
  const int groups = N / l.rows;
  const long blocks = (long)groups * H;
  // the in-kernel hand-off when the counters cover the output blocks and
  // the partial slots fit; otherwise the two-kernel split (same sums, same
  // order)
  const bool handoff = l.splits > 1 && ws.counters && blocks <= kMaxHandoffGroups &&
                       (size_t)blocks * l.splits * 16 * q * (l.rows / 4) <= ws.partial_floats;
  dim3 grid(groups * H * l.splits), block(64 * l.waves);
  const int mode = (handoff ? kModeHandoff : 0) | (ws.force_recompute ? kModeRecompute : 0);
  hipLaunchKernelGGL(k, grid, block, 0, stream, x, w, M, N, K, l.splits, H, groups,
                     kBlockK * l.chunks, l.waves, mode, y, ws.partials,
                     handoff ? ws.counters : nullptr, pub);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || l.splits == 1 || handoff) return e;
  return launch_split_reduce(ws.partials, y, M, N, l.splits, pub, stream);
}

}  // namespace skinny
