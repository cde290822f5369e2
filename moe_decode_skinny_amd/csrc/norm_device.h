// Device helpers shared by the norm kernels (RMSNorm -> NVFP4 / BF16 and the
// dual norm): binary64 -> bfloat16 rounding, a 16-value bfloat16 load, and
// the fixed-order workgroup sum.
#pragma once

#include "device.h"

namespace skinny {
namespace norm {

constexpr int kNormThreads = 256;

// binary64 -> bfloat16 bits, round to nearest even (finite inputs; overflow
// gives infinity).
__device__ __forceinline__ unsigned f64_to_bf16(double v) {
  const unsigned long long u = (unsigned long long)__double_as_longlong(v);
  const unsigned sign = (unsigned)(u >> 48) & 0x8000u;
  const double a = fabs(v);
  if (a < 0x1p-126) {                       // bfloat16 subnormals: step 2^-133
    return sign | (unsigned)rint(a * 0x1p133);  // 128 -> smallest normal
  }
  unsigned long long b = u & 0x7fffffffffffffffull;
  b += 0xfffffffffffull + ((b >> 45) & 1ull);   // keep 7 of 52 mantissa bits
  const int exp = (int)(b >> 52) - 1023 + 127;
  if (exp >= 255) return sign | 0x7f80u;
  return sign | ((unsigned)exp << 7) | (unsigned)((b >> 45) & 0x7full);
}

// 16 consecutive bfloat16 values (32 bytes, 16-byte aligned) as binary64.
__device__ __forceinline__ void load16(const uint16_t *p, double (&v)[16]) {
  const u32x4 a = *reinterpret_cast<const u32x4 *>(p);
  const u32x4 b = *reinterpret_cast<const u32x4 *>(p + 8);
  const unsigned u[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    v[2 * i] = (double)bf16_lo(u[i]);
    v[2 * i + 1] = (double)bf16_hi(u[i]);
  }
}

// This thread's part of a row's sum of squares: the 16-column blocks t,
// t + THREADS, ... of `row` in column order, two blocks' loads in flight at
// a time (the order of the sum is that of the blocks either way).
template <int THREADS>
__device__ __forceinline__ double sum_squares(const uint16_t *row, int blocks, int t) {
  double ss = 0.0;
  int b = t;
  for (; b + THREADS < blocks; b += 2 * THREADS) {
    double v[16], u[16];
    load16(row + b * 16, v);
    load16(row + (b + THREADS) * 16, u);
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += v[j] * v[j];
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += u[j] * u[j];
  }
  if (b < blocks) {
    double v[16];
    load16(row + b * 16, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += v[j] * v[j];
  }
  return ss;
}

// Sum over the workgroup in a fixed order: a lane butterfly inside each wave,
// then the wave sums in wave order (every thread gets the total).  `slots`
// is LDS of THREADS / 64 doubles used only by this call.
template <int THREADS = kNormThreads>
__device__ __forceinline__ double block_sum(double v, double *slots) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if ((threadIdx.x & 63) == 0) slots[threadIdx.x >> 6] = v;
  __syncthreads();
  double total = slots[0];
#pragma unroll
  for (int i = 1; i < THREADS / 64; ++i) total += slots[i];
  return total;
}

}  // namespace norm
}  // namespace skinny
