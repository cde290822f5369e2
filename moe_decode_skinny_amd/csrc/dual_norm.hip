// The single-GPU dual norm after o_proj (oproj.batt page, AttentionBoundary):
// the o_proj output goes through post_attn_norm, a gated add into the FP32
// residual stream (in place, with the connection's alpha and beta) and
// pre_ffn_norm into the BF16 output.  The all-reduce that precedes it on
// several GPUs is the identity on one.
//
// The pages print neither the kernel nor its constants; this computes the
// reading stated with the declaration in skinny.h:
//   h_j      = bf16( p_j / sqrt(mean(p^2) + post_eps) * g_j ),
//              g_j = post_w_j + post_gain_center (1 without a post weight)
//   stream_j = f32( a_j * stream_j + beta_j * h_j ),  a_j = alpha_j or a scalar
//   out_j    = bf16( s_j / sqrt(mean(s^2) + pre_eps) * (next_w_j + pre_gain_center) )
// with s the updated stream row.
//
// gfx950 design as for the pooler norm: one 256-thread workgroup per row,
// thread t owns the 16-column blocks t, t + 256, ...; binary64 arithmetic
// (the products a * stream and beta * h are exact in binary64, their sum is
// rounded once there and then once to binary32; every bfloat16 is one
// round-to-nearest-even from binary64); both sums of squares in a fixed
// order.  A thread re-reads the stream values it wrote itself for the
// second norm.
#include "norm_device.h"

namespace skinny {
namespace {

using namespace norm;

__device__ __forceinline__ void load16_f32(const float *p, double (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p + 4 * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[4 * q + i] = (double)a[i];
  }
}

__global__ __launch_bounds__(kNormThreads) void dual_norm_kernel(
    const uint16_t *__restrict__ partial, float *__restrict__ residual,
    const uint16_t *__restrict__ post_w, float post_gc, float post_eps,
    const uint16_t *__restrict__ alpha, float alpha_scalar, const uint16_t *__restrict__ beta,
    const uint16_t *__restrict__ next_w, float pre_gc, float pre_eps,
    uint16_t *__restrict__ out, int H) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int blocks = H / 16;
  const uint16_t *prow = partial + (size_t)row * H;
  float *srow = residual + (size_t)row * H;
  uint16_t *orow = out + (size_t)row * H;
  __shared__ double slots_post[kNormThreads / 64], slots_pre[kNormThreads / 64];

  double ss = 0.0;
  for (int blk = tid; blk < blocks; blk += kNormThreads) {
    double v[16];
    load16(prow + blk * 16, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += v[j] * v[j];
  }
  const double inv = 1.0 / sqrt(block_sum(ss, slots_post) / (double)H + (double)post_eps);

  // Post norm and gated add; the new stream's sum of squares on the way.
  double ss2 = 0.0;
  for (int blk = tid; blk < blocks; blk += kNormThreads) {
    double p[16], g[16], a[16], b[16], s[16];
    load16(prow + blk * 16, p);
    if (post_w) {
      load16(post_w + blk * 16, g);
#pragma unroll
      for (int j = 0; j < 16; ++j) g[j] += (double)post_gc;
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) g[j] = 1.0;
    }
    if (alpha) {
      load16(alpha + blk * 16, a);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) a[j] = (double)alpha_scalar;
    }
    load16(beta + blk * 16, b);
    load16_f32(srow + blk * 16, s);
    f32x4 o[4];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const double h = (double)__uint_as_float(f64_to_bf16(p[j] * inv * g[j]) << 16);
      const float v = (float)(a[j] * s[j] + b[j] * h);
      o[j / 4][j % 4] = v;
      ss2 += (double)v * (double)v;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4 *>(srow + blk * 16 + 4 * q) = o[q];
  }
  const double inv2 = 1.0 / sqrt(block_sum(ss2, slots_pre) / (double)H + (double)pre_eps);

  for (int blk = tid; blk < blocks; blk += kNormThreads) {
    double s[16], w[16];
    load16_f32(srow + blk * 16, s);  // this thread's own stores above
    load16(next_w + blk * 16, w);
    unsigned yb[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) yb[j] = f64_to_bf16(s[j] * inv2 * (w[j] + (double)pre_gc));
    u32x4 o0, o1;
    o0.x = yb[0] | (yb[1] << 16);   o0.y = yb[2] | (yb[3] << 16);
    o0.z = yb[4] | (yb[5] << 16);   o0.w = yb[6] | (yb[7] << 16);
    o1.x = yb[8] | (yb[9] << 16);   o1.y = yb[10] | (yb[11] << 16);
    o1.z = yb[12] | (yb[13] << 16); o1.w = yb[14] | (yb[15] << 16);
    u32x4 *dst = reinterpret_cast<u32x4 *>(orow + blk * 16);
    dst[0] = o0;
    dst[1] = o1;
  }
}

}  // namespace

hipError_t launch_dual_norm(const uint16_t *partial, float *residual, const uint16_t *post_w,
                            float post_gc, float post_eps, const uint16_t *alpha,
                            float alpha_scalar, const uint16_t *beta, const uint16_t *next_w,
                            float pre_gc, float pre_eps, uint16_t *out, int M, int H,
                            hipStream_t stream) {
  hipLaunchKernelGGL(dual_norm_kernel, dim3(M), dim3(kNormThreads), 0, stream, partial,
                     residual, post_w, post_gc, post_eps, alpha, alpha_scalar, beta, next_w,
                     pre_gc, pre_eps, out, H);
  return hipGetLastError();
}

}  // namespace skinny
