// RMSNorm with gain center and the block-16 NVFP4 expert input
// (pooler_gather page, module description and compile_norm_quant):
//   yn = bf16( r * rsqrt(mean(r^2) + eps) * (w + gain_center) )
//   a, a_sf = nvfp4(yn, global_scale, block 16)
// with the conversions of cvt_e2m1x8_f32 / cvt_f32_to_e4m3 (round to nearest
// even, saturate to the largest finite value) and the output scale of
// nvfp4_compute_output_scale (the reciprocal of dec(sf) / global_scale, zero
// when dec(sf) is zero).
//
// gfx950 design: one workgroup of 256 threads per row; thread t owns whole
// 16-column blocks (t, t + 256, ...), so a block's amax, scale and codes stay
// in one thread and its 8 code bytes leave as one 8-byte store.
// Arithmetic is binary64 (gfx950 has full-rate FP64 vector units and the
// kernel is latency-bound, so this costs nothing measurable): the sum of
// squares, the reciprocal root, the product r * inv * (w + gain_center), the
// block scale global_scale * amax / 6, the output scale and the scaled values
// are all exact or rounded once in binary64, and every narrowing (to
// bfloat16, e4m3fn, e2m1) is a single round-to-nearest-even from binary64.
// The sum of squares is reduced in a fixed order: per thread in column order,
// a lane butterfly inside each wave, then the four wave sums in wave order.
// The e4m3 and e2m1 encoders are written out in integer/compare form (no
// vendor conversion instruction), so rounding and saturation are exactly the
// round-to-nearest-even + satfinite the pages specify.
// Readings (the norm/quant kernel body is not printed): the block scale is
// e4m3(global_scale * amax / 6); the output scale is global_scale / dec(sf);
// a negative value that rounds to zero keeps its sign.
#include "norm_device.h"
#include "internal.h"

namespace skinny {
namespace {

using namespace norm;

// |v| -> e4m3fn code, round to nearest even, saturating at 448 (0x7E).
__device__ __forceinline__ unsigned e4m3_rn_satfinite(double v) {
  const double a = fabs(v);
  if (a != a) return 0x7Fu;
  if (a >= 448.0) return 0x7Eu;
  if (a < 0x1p-6) return (unsigned)rint(a * 512.0);   // step 2^-9; 8 -> 0x08
  unsigned long long b = (unsigned long long)__double_as_longlong(a);
  b += 0xffffffffffffull + ((b >> 49) & 1ull);        // keep 3 mantissa bits
  const unsigned exp = (unsigned)(b >> 52) - 1023u + 7u;  // 1..15
  return (exp << 3) | (unsigned)((b >> 49) & 7ull);
}

// e4m3fn code (finite, non-negative) -> its value.
__device__ __forceinline__ double e4m3_value(unsigned c) {
  const unsigned exp = (c >> 3) & 15u, man = c & 7u;
  if (exp == 0) return (double)man * 0x1p-9;
  return ldexp(1.0 + man * 0.125, (int)exp - 7);
}

// v -> e2m1 code: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 by index; ties to the
// even index (the comparison is >= where the upper neighbour is even);
// anything above 5 saturates to 6; the sign bit is kept.
__device__ __forceinline__ unsigned e2m1_rn_satfinite(double v) {
  const double a = fabs(v);
  const unsigned idx = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) +
                       (a > 2.5) + (a >= 3.5) + (a > 5.0);
  return (signbit(v) ? 8u : 0u) | idx;
}

template <bool QUANT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const uint16_t *__restrict__ r, const uint16_t *__restrict__ w, float gain_center,
    float eps, const float *__restrict__ global_scale, uint8_t *__restrict__ a,
    uint8_t *__restrict__ a_sf, uint16_t *__restrict__ y, int P) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int blocks = P / 16;
  const uint16_t *rrow = r + (size_t)row * P;

  // Sum of squares in a fixed order; the first block and its weights are
  // loaded before the reduction and stay in registers.
  double first[16], gfirst[16];
  double ss = 0.0;
  if (tid < blocks) {
    load16(rrow + tid * 16, first);
    load16(w + tid * 16, gfirst);
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += first[j] * first[j];
  }
  for (int blk = tid + kNormThreads; blk < blocks; blk += kNormThreads) {
    double v[16];
    load16(rrow + blk * 16, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += v[j] * v[j];
  }
  __shared__ double wave_ss[kNormThreads / 64];
  const double total = block_sum(ss, wave_ss);
  const double inv = 1.0 / sqrt(total / (double)P + (double)eps);
  const double gc = (double)gain_center;
  const double gs = QUANT ? (double)*global_scale : 0.0;

  for (int blk = tid; blk < blocks; blk += kNormThreads) {
    double v[16], g[16];
    if (blk == tid) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        v[j] = first[j];
        g[j] = gfirst[j];
      }
    } else {
      load16(rrow + blk * 16, v);
      load16(w + blk * 16, g);
    }
    unsigned yb[16];
    double amax = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      yb[j] = f64_to_bf16(v[j] * inv * (g[j] + gc));
      amax = fmax(amax, fabs((double)__uint_as_float(yb[j] << 16)));
    }
    if constexpr (QUANT) {
      const unsigned sf = e4m3_rn_satfinite(gs * amax / 6.0);
      const double dec = e4m3_value(sf);
      const double os = dec == 0.0 ? 0.0 : gs / dec;
      unsigned lo = 0, hi = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        lo |= e2m1_rn_satfinite((double)__uint_as_float(yb[j] << 16) * os) << (4 * j);
        hi |= e2m1_rn_satfinite((double)__uint_as_float(yb[j + 8] << 16) * os) << (4 * j);
      }
      *reinterpret_cast<uint2 *>(a + (size_t)row * (P / 2) + blk * 8) = make_uint2(lo, hi);
      a_sf[(size_t)row * blocks + blk] = (uint8_t)sf;
    } else {
      u32x4 o0, o1;
      o0.x = yb[0] | (yb[1] << 16);   o0.y = yb[2] | (yb[3] << 16);
      o0.z = yb[4] | (yb[5] << 16);   o0.w = yb[6] | (yb[7] << 16);
      o1.x = yb[8] | (yb[9] << 16);   o1.y = yb[10] | (yb[11] << 16);
      o1.z = yb[12] | (yb[13] << 16); o1.w = yb[14] | (yb[15] << 16);
      u32x4 *dst = reinterpret_cast<u32x4 *>(y + (size_t)row * P + blk * 16);
      dst[0] = o0;
      dst[1] = o1;
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t *r, const uint16_t *w, float gain_center,
                          float eps, const float *global_scale, uint8_t *a,
                          uint8_t *a_sf, uint16_t *y, int M, int P, bool quant,
                          hipStream_t stream) {
  dim3 grid(M), block(kNormThreads);
  if (quant)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, grid, block, 0, stream, r, w, gain_center,
                       eps, global_scale, a, a_sf, y, P);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, grid, block, 0, stream, r, w, gain_center,
                       eps, global_scale, a, a_sf, y, P);
  return hipGetLastError();
}

}  // namespace skinny
