// RMSNorm with gain center and the block-16 NVFP4 expert input
// (pooler_gather page, module description and compile_norm_quant):
//   yn = bf16( r * rsqrt(mean(r^2) + eps) * (w + gain_center) )
//   a, a_sf = nvfp4(yn, global_scale, block 16)
// with the conversions of cvt_e2m1x8_f32 / cvt_f32_to_e4m3 (round to nearest
// even, saturate to the largest finite value) and the output scale of
// nvfp4_compute_output_scale (the reciprocal of dec(sf) / global_scale, zero
// when dec(sf) is zero).
//
// gfx950 design: a row is spread over C = ceil(P / 1024) workgroups of 256
// threads.  Every workgroup of the row computes the row's sum of squares
// itself (thread t sums the 16-column blocks t, t + 256, ... in column
// order; the row is re-read from L2), so all of them reach the same bits
// without talking to each other; then workgroup c quantises blocks
// 64 c .. 64 c + 63 with four threads a block (four columns each: the block
// amax is a max over the quad, the scale is computed by all four alike, and
// each thread stores its four codes as two bytes).  Spreading a block's
// binary64 encoding over four threads and a row over C compute units cut the
// kernel's serial chain; the codes are the same.
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

constexpr int kQuantBlocks = kNormThreads / 4;  // 16-column blocks a workgroup quantises

// The sizes come right after the inputs: the first 14 argument dwords
// arrive preloaded in SGPRs, and the row index needs `parts` at once.
template <bool QUANT>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const uint16_t *__restrict__ r, const uint16_t *__restrict__ w, int P, int parts,
    float gain_center, float eps, const float *__restrict__ global_scale,
    uint8_t *__restrict__ a, uint8_t *__restrict__ a_sf, uint16_t *__restrict__ y) {
  const int row = blockIdx.x / parts, part = blockIdx.x - row * parts;
  const int tid = threadIdx.x;
  const int blocks = P / 16;
  const uint16_t *rrow = r + (size_t)row * P;
  // This thread's quarter (columns 4 q .. 4 q + 3) of block blk; its loads
  // are issued first, ahead of the reduction.
  const int blk = part * kQuantBlocks + (tid >> 2);
  const int q = tid & 3;
  const bool mine = blk < blocks;  // the four threads of a block agree
  uint2 rq = make_uint2(0, 0), wq = make_uint2(0, 0);
  if (mine) {
    rq = *reinterpret_cast<const uint2 *>(rrow + blk * 16 + 4 * q);
    wq = *reinterpret_cast<const uint2 *>(w + blk * 16 + 4 * q);
  }
  // The global scale too: read after the barrier it would cost one more
  // memory round trip at the end of the chain.
  const float gsf = QUANT ? *global_scale : 0.f;

  // Sum of squares of the whole row in a fixed order.
  const double ss = sum_squares<kNormThreads>(rrow, blocks, tid);
  __shared__ double wave_ss[kNormThreads / 64];
  const double total = block_sum(ss, wave_ss);
  if (!mine) return;
  const double inv = 1.0 / sqrt(total / (double)P + (double)eps);
  const double gc = (double)gain_center;

  const unsigned ru[2] = {rq.x, rq.y}, wu[2] = {wq.x, wq.y};
  unsigned yb[4];
  double amax = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const unsigned rb = (ru[j / 2] >> (16 * (j % 2))) & 0xffffu;
    const unsigned wb = (wu[j / 2] >> (16 * (j % 2))) & 0xffffu;
    yb[j] = f64_to_bf16((double)__uint_as_float(rb << 16) * inv *
                        ((double)__uint_as_float(wb << 16) + gc));
    amax = fmax(amax, fabs((double)__uint_as_float(yb[j] << 16)));
  }
  if constexpr (QUANT) {
    amax = fmax(amax, __shfl_xor(amax, 1));  // the block's amax over its quad
    amax = fmax(amax, __shfl_xor(amax, 2));
    const double gs = (double)gsf;
    const unsigned sf = e4m3_rn_satfinite(gs * amax / 6.0);
    const double dec = e4m3_value(sf);
    const double os = dec == 0.0 ? 0.0 : gs / dec;
    unsigned codes = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      codes |= e2m1_rn_satfinite((double)__uint_as_float(yb[j] << 16) * os) << (4 * j);
    // Column 4 q + j is nibble j of this thread's two bytes (even column low).
    *reinterpret_cast<uint16_t *>(a + (size_t)row * (P / 2) + blk * 8 + 2 * q) =
        (uint16_t)codes;
    if (q == 0) a_sf[(size_t)row * blocks + blk] = (uint8_t)sf;
  } else {
    *reinterpret_cast<uint2 *>(y + (size_t)row * P + blk * 16 + 4 * q) =
        make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
  }
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t *r, const uint16_t *w, float gain_center,
                          float eps, const float *global_scale, uint8_t *a,
                          uint8_t *a_sf, uint16_t *y, int M, int P, bool quant,
                          hipStream_t stream) {
  const int parts = (P / 16 + kQuantBlocks - 1) / kQuantBlocks;
  dim3 grid(parts * M), block(kNormThreads);
  if (quant)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, grid, block, 0, stream, r, w, P, parts,
                       gain_center, eps, global_scale, a, a_sf, y);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, grid, block, 0, stream, r, w, P, parts,
                       gain_center, eps, global_scale, a, a_sf, y);
  return hipGetLastError();
}

}  // namespace skinny
