// Host-side declarations shared by the libskinny translation units: the
// per-device state, the kernel launchers and the variant queries used by
// validation.  What the kernels themselves depend on (limits, kernel
// argument structs, device helpers) is in device.h.  Not installed.
#pragma once

#include <atomic>

#include "device.h"

namespace skinny {

struct DeviceState {
  // Set (release) by skinny_init once the buffers below exist; compute calls
  // on other threads read it (acquire) without taking the init lock.
  std::atomic<bool> ready{false};
  float *partials = nullptr;         // kWorkspaceFloats
  unsigned *counters = nullptr;      // kCounterWords, zeroed by skinny_init
  double *norm_partials = nullptr;   // kNormPartials
  // This device's address of the library's static scratch array
  // (skinny_gemm_bf16_noalloc: kScratchFloats partials, then kCounterWords
  // counters), from hipGetSymbolAddress.
  float *scratch = nullptr;
  // Test hook, from the environment at skinny_init
  // (SKINNY_FORCE_SPLIT_RECOMPUTE=1): the 16-block split hand-off takes its
  // cross-XCD path (recompute every split) on every call.
  bool force_recompute = false;
};

// The state of the current HIP device, or nullptr (and a reason) if the
// device has not been initialised.
DeviceState *current_state(int *status);


// ------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already valid.
// `ws`: the split-K scratch, used when l.splits > 1.
hipError_t launch_gemm_mfma(const uint16_t *x, const uint16_t *w, uint16_t *y,
                            int M, int N, int K, const skinny_launch &l,
                            const Workspace &ws, const Publish &pub, hipStream_t stream);
hipError_t launch_gemm_dot2(const uint16_t *x, const uint16_t *w, uint16_t *y,
                            int M, int N, int K, const skinny_launch &l,
                            const Workspace &ws, const Publish &pub, hipStream_t stream);
hipError_t launch_gemm_blocks(const uint16_t *x, const uint16_t *w, uint16_t *y,
                              int M, int N, int K, const skinny_launch &l,
                              const Workspace &ws, const Publish &pub, hipStream_t stream);
hipError_t launch_gemm_ring(const RingItems &items, int count, int M, int N, int K,
                            const skinny_ring_launch &r, hipStream_t stream);
hipError_t launch_split_reduce(const float *partials, uint16_t *y, int M, int N, int S,
                               const Publish &pub, hipStream_t stream);
hipError_t launch_dual_norm(const uint16_t *partial, float *residual, const uint16_t *post_w,
                            float post_gc, float post_eps, const uint16_t *alpha,
                            float alpha_scalar, const uint16_t *beta, const uint16_t *next_w,
                            float pre_gc, float pre_eps, uint16_t *out, int M, int H,
                            DeviceState &st, hipStream_t stream);
hipError_t launch_rmsnorm(const uint16_t *r, const uint16_t *w, float gain_center,
                          float eps, const float *global_scale, uint8_t *a,
                          uint8_t *a_sf, uint16_t *y, int M, int P, bool quant,
                          hipStream_t stream);

// Instantiation tables (which template variants exist), used by validation.
bool mfma_variant_exists(int chunks, int accs);
int mfma_max_waves(int chunks);  // waves per MFMA workgroup (launch bound)
size_t mfma_lds_bytes(int M, const skinny_launch &l);  // dynamic LDS of a launch
hipError_t mfma_prepare();  // per-device kernel attributes (skinny_init)
bool dot2_variant_exists(int rows, int chunks, int mt, int waves);
int dot2_token_tile(int M);  // smallest compiled token count >= M, 0 if none
int dot2_max_waves();        // waves per DOT2 workgroup (the 16-wave form's bound)
int blocks_token_sets(int M);  // 4-token sets of the 16-block MFMA path (1, 2, 4), 0 if none
// 4-token sets per workgroup of a 16-block launch with H token groups (1, 2
// or 4); 0 unless every group gets at least one of the M tokens
int blocks_group_token_sets(int M, int H);
bool blocks_variant_exists(int rows, int chunks, int q, int waves);
bool ring_variant_exists(int rows, int chunks, int mt, int waves);  // DOT2 ring (<= 16 waves)
bool blocks_ring_variant_exists(int rows, int chunks, int q, int waves);  // MFMA 4x4 ring
bool mfma_ring_variant_exists(int chunks, int accs, bool staged);  // MFMA ring
int mfma_ring_max_waves(int chunks);
size_t mfma_ring_lds_bytes(const skinny_launch &l);  // dynamic LDS of an MFMA ring launch
hipError_t ring_prepare();  // per-device kernel attributes (skinny_init)

}  // namespace skinny

