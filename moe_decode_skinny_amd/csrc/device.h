// What the kernels depend on, shared by the libskinny translation units: the
// limits, the structs passed to kernels by value and the device helpers.
// Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "skinny.h"

namespace skinny {

// ---------------------------------------------------------------- limits
constexpr int kMaxM = 16;          // tokens (unpooler page: 1 <= M <= 16)
constexpr int kTileN = 16;         // features per MFMA tile (grid N / 16)
constexpr int kMfmaK = 32;         // K per v_mfma_f32_16x16x32_bf16
constexpr int kDot2K = 512;        // K per DOT2 chunk: 64 lanes x 8 bf16
constexpr int kBlockK = 128;       // K per 16-block MFMA chunk: 16 blocks x 8 bf16
constexpr int kGroupK = 4 * kBlockK;  // K per 16-block load group (4 chunks, 1 KiB a row)
constexpr int kBlocksMaxWaves = 16;
constexpr int kMaxMfmaChunks = 16;
constexpr int kMaxDot2Chunks = 4;
constexpr int kMaxSplits = 16;
// Split-K workspace owned by the library (per device, from skinny_init):
// FP32 partials [split][token][feature], S * M * N floats at most.
constexpr size_t kWorkspaceFloats = size_t(2) << 20;  // 8 MiB
// The same partials for skinny_gemm_bf16_noalloc, in a static device array of
// the library (no allocation): S * M * N floats at most.
constexpr size_t kScratchFloats = size_t(1) << 18;  // 1 MiB
// Counter words of the 16-block path's in-kernel split hand-off, one per
// output group, each on its own 256-byte stretch (arrivals of different
// groups then do not contend for one cache line); zero between calls.
constexpr int kMaxHandoffGroups = 2048;
constexpr int kCounterStride = 64;  // words
constexpr size_t kCounterWords = (size_t)kMaxHandoffGroups * kCounterStride;  // 512 KiB

// Where a GEMM call's split-K scratch lives (the skinny_init workspace, or
// the static scratch array of skinny_gemm_bf16_noalloc).
struct Workspace {
  float *partials = nullptr;     // FP32 partials
  size_t partial_floats = 0;     // their capacity
  unsigned *counters = nullptr;  // kCounterWords hand-off counters, zero between calls
  bool force_recompute = false;  // test hook: the hand-off always recomputes the splits
};

constexpr size_t kMaxDynamicLds = 160 * 1024;  // all of a gfx950 CU's LDS

// The dual norm's per-slice sums of squares (binary64), M * slices of them,
// in a buffer of its own (per device, from skinny_init).
constexpr size_t kNormPartials = 65536;
constexpr int kDualSlice = 1024;  // columns per workgroup of the two-kernel dual norm

// The zero-copy publish of a GEMM call (unpooler page, module description,
// zero-copy epilogue): y also goes into this rank's slot of a mailbox
// [3 stages][tp][capacity][N] at the stage read on the device when the
// kernel runs, with -0.0 (the mailbox's "not yet written" sentinel) stored
// as +0.0.  data == nullptr: no publish.
struct Publish {
  uint16_t *data = nullptr;
  const int *stage_src = nullptr;  // stage_state[0], or the ticket word
  int *stage_word = nullptr;       // stage_state[1]; nullptr with a ticket
  int shift = 0;                   // 16 with a ticket (stage << 16)
  int tp = 0, rank = 0, capacity = 0;
};

// The layer ring: up to kMaxRingItems independent GEMMs of one shape.
constexpr int kMaxRingItems = 64;
struct RingItems {
  const uint16_t *x[kMaxRingItems];
  const uint16_t *w[kMaxRingItems];
  uint16_t *y[kMaxRingItems];
};
}  // namespace skinny

// ------------------------------------------------------------ device helpers
#if defined(__HIPCC__)
namespace skinny {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The in-order sum term(0) + term(1) + ... + term(n - 1) of 1 <= n <= N
// terms, n known only at run time (a wave or split count).  A plain loop
// with a run-time bound waits for each term's load before it issues the
// next; here every load is issued first and the adds follow in index
// order, so the result is the plain loop's and the loads cost one round
// trip instead of n.  term(i) is evaluated for every i < N, with no
// branch: the caller makes that safe (a row of a static LDS array, a buffer
// load, which returns zero past its range); terms from n on are not added.
template <int N, typename T, typename Term>
__device__ __forceinline__ T sum_in_order(int n, Term term) {
  T v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = term(i);
  T sum = v[0];
#pragma unroll
  for (int i = 1; i < N; ++i) sum = i < n ? sum + v[i] : sum;
  return sum;
}

// sum_in_order over the rows of a workgroup's waves (1 <= waves <= MAXW):
// reads the next power of two >= waves rows, not MAXW, so a one-wave launch
// reads one.
template <int MAXW, typename T, typename Term>
__device__ __forceinline__ T sum_waves_in_order(int waves, Term term) {
  static_assert(MAXW == 8 || MAXW == 16, "8 or 16 waves at most");
  if (waves == 1) return term(0);
  if (waves <= 2) return sum_in_order<2, T>(waves, term);
  if (waves <= 4) return sum_in_order<4, T>(waves, term);
  if (MAXW == 8 || waves <= 8) return sum_in_order<8, T>(waves, term);
  return sum_in_order<MAXW, T>(waves, term);
}

// FP32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ unsigned f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// The wave's index in its workgroup as a wave-uniform (scalar) value.  The
// compiler cannot prove threadIdx.x >> 6 uniform, and a buffer resource
// derived from a value it takes as divergent is rebuilt lane by lane in a
// loop around every load.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ float bf16_lo(unsigned u) { return __uint_as_float(u << 16); }

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zeros instead of touching memory, which gives token padding and
// ragged-K tails without branches.  bytes must be < 2^31.
constexpr unsigned kBufferFlags = 0x00020000u;  // gfx9 dword3: 32-bit data format
constexpr int kOutOfRange = 0x7FFFF000;         // an offset past any resource used here
constexpr int kCacheNT = 2;                     // nontemporal (streaming) load policy
// s_getreg operand of the XCC_ID hardware register, bits 3..0 (the XCD a
// wave runs on).
constexpr int kHwRegXccId = 20 | (0 << 6) | ((4 - 1) << 11);

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           (int)kBufferFlags);
}
__device__ __forceinline__ float bf16_hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }

// An output store with the device-scope cache policy (a relaxed agent-scope
// atomic store: the store's sc1 bit).  Used only where it measured faster:
// the 16-block kernel at one split and the split reduce, 1-2.5% per call.
// With the same store, DOT2 at 1-2 tokens and the layer ring were 3.5-13%
// slower and the 16-block kernel's in-kernel split 1-3% slower, so those
// keep plain stores.
__device__ __forceinline__ void store_out_device(uint16_t *p, unsigned bits) {
  __hip_atomic_store(p, (uint16_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Four outputs, p 8-byte aligned: lo holds the first two.
__device__ __forceinline__ void store_out_device(uint16_t *p, unsigned lo, unsigned hi) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), ((uint64_t)hi << 32) | lo, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------- zero-copy publish helpers
// The publish stage of this call: the stage word's value, or the upper half
// of the ticket; anything outside 0..2 (negative values included) means no
// publish.
__device__ __forceinline__ unsigned publish_stage(const Publish &p) {
  return (unsigned)*p.stage_src >> p.shift;
}

// The slot [capacity][N] this call publishes into, or nullptr.
__device__ __forceinline__ uint16_t *publish_slot(const Publish &p, int N) {
  if (!p.data) return nullptr;
  const unsigned stage = publish_stage(p);
  if (stage > 2) return nullptr;
  return p.data + ((size_t)stage * p.tp + p.rank) * (size_t)p.capacity * N;
}

// Sets the active-stage word (one thread of the writing kernel calls it).
__device__ __forceinline__ void publish_stage_word(const Publish &p) {
  if (!p.data || !p.stage_word) return;
  const unsigned stage = publish_stage(p);
  if (stage <= 2) *p.stage_word = (int)stage;
}

// bf16 bits as published: -0.0 (0x8000) becomes +0.0; one value, or two
// packed in 32 bits.
__device__ __forceinline__ unsigned publish_bits(unsigned b) { return b == 0x8000u ? 0u : b; }
__device__ __forceinline__ unsigned publish_pair(unsigned v) {
  return publish_bits(v & 0xffffu) | (publish_bits(v >> 16) << 16);
}

}  // namespace skinny
#endif
