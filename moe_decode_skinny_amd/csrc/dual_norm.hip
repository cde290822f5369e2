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
// gfx950 design as for the pooler norm: one workgroup per row (512 threads:
// one 16-column block a thread at H = 8192), thread t owning the blocks t,
// t + 512, ...; every load of a thread's first block is issued before the
// first reduction, so the kernel waits on memory once; binary64 arithmetic
// (the products a * stream and beta * h are exact in binary64, their sum is
// rounded once there and then once to binary32; every bfloat16 is one
// round-to-nearest-even from binary64); both sums of squares in a fixed
// order.  Past the first block a thread reloads, and for the second norm
// re-reads the stream values it stored itself.
#include "norm_device.h"
#include "internal.h"

namespace skinny {
namespace {

using namespace norm;

constexpr int kDualThreads = 512;  // one 16-column block a thread at H = 8192

__device__ __forceinline__ void load16_f32(const float *p, double (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p + 4 * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[4 * q + i] = (double)a[i];
  }
}

// Everything one 16-column block needs, as loaded (bf16 as doubles).
struct Block {
  double p[16], g[16], a[16], b[16], s[16], w[16];
};

__device__ __forceinline__ void load_block(Block &k, int blk, const uint16_t *prow,
                                           const float *srow, const uint16_t *post_w,
                                           float post_gc, const uint16_t *alpha,
                                           float alpha_scalar, const uint16_t *beta,
                                           const uint16_t *next_w) {
  load16(prow + blk * 16, k.p);
  load16_f32(srow + blk * 16, k.s);
  if (post_w) {
    load16(post_w + blk * 16, k.g);
#pragma unroll
    for (int j = 0; j < 16; ++j) k.g[j] += (double)post_gc;
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) k.g[j] = 1.0;
  }
  if (alpha) {
    load16(alpha + blk * 16, k.a);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) k.a[j] = (double)alpha_scalar;
  }
  load16(beta + blk * 16, k.b);
  load16(next_w + blk * 16, k.w);
}

// Post norm and gated add of one block: the new residual values (stored and
// returned in s) and their sum of squares.
__device__ __forceinline__ double gate_block(Block &k, double inv, float *dst) {
  double ss2 = 0.0;
  f32x4 o[4];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const double h = (double)__uint_as_float(f64_to_bf16(k.p[j] * inv * k.g[j]) << 16);
    const float v = (float)(k.a[j] * k.s[j] + k.b[j] * h);
    o[j / 4][j % 4] = v;
    k.s[j] = (double)v;
    ss2 += (double)v * (double)v;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<f32x4 *>(dst + 4 * q) = o[q];
  return ss2;
}

__device__ __forceinline__ void out_block(const double (&s)[16], const double (&w)[16],
                                          double inv2, float pre_gc, uint16_t *dst) {
  unsigned yb[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) yb[j] = f64_to_bf16(s[j] * inv2 * (w[j] + (double)pre_gc));
  u32x4 o0, o1;
  o0.x = yb[0] | (yb[1] << 16);   o0.y = yb[2] | (yb[3] << 16);
  o0.z = yb[4] | (yb[5] << 16);   o0.w = yb[6] | (yb[7] << 16);
  o1.x = yb[8] | (yb[9] << 16);   o1.y = yb[10] | (yb[11] << 16);
  o1.z = yb[12] | (yb[13] << 16); o1.w = yb[14] | (yb[15] << 16);
  reinterpret_cast<u32x4 *>(dst)[0] = o0;
  reinterpret_cast<u32x4 *>(dst)[1] = o1;
}

__global__ __launch_bounds__(kDualThreads) void dual_norm_kernel(
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
  __shared__ double slots_post[kDualThreads / 64], slots_pre[kDualThreads / 64];

  // The thread's first block: every load issued before the first reduction
  // (one memory latency for the whole kernel up to H = 16 * kDualThreads).
  const bool have = tid < blocks;
  Block first;
  if (have)
    load_block(first, tid, prow, srow, post_w, post_gc, alpha, alpha_scalar, beta, next_w);

  double ss = 0.0;
  if (have) {
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += first.p[j] * first.p[j];
  }
  for (int blk = tid + kDualThreads; blk < blocks; blk += kDualThreads) {
    double v[16];
    load16(prow + blk * 16, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) ss += v[j] * v[j];
  }
  const double inv =
      1.0 / sqrt(block_sum<kDualThreads>(ss, slots_post) / (double)H + (double)post_eps);

  double ss2 = 0.0;
  if (have) ss2 += gate_block(first, inv, srow + tid * 16);
  for (int blk = tid + kDualThreads; blk < blocks; blk += kDualThreads) {
    Block k;
    load_block(k, blk, prow, srow, post_w, post_gc, alpha, alpha_scalar, beta, next_w);
    ss2 += gate_block(k, inv, srow + blk * 16);
  }
  const double inv2 =
      1.0 / sqrt(block_sum<kDualThreads>(ss2, slots_pre) / (double)H + (double)pre_eps);

  if (have) out_block(first.s, first.w, inv2, pre_gc, orow + tid * 16);
  for (int blk = tid + kDualThreads; blk < blocks; blk += kDualThreads) {
    double s[16], w[16];
    load16_f32(srow + blk * 16, s);  // this thread's own stores above
    load16(next_w + blk * 16, w);
    out_block(s, w, inv2, pre_gc, orow + blk * 16);
  }
}

// ------------------------------------------------------------- two kernels
// Rows of at least 2 kDualSlice columns are spread over S = ceil(H /
// kDualSlice) workgroups of 256 threads (thread t: columns 4t .. 4t + 3 of
// its slice); one workgroup per row must pull every byte of the row through
// one CU, whose cache-miss concurrency then bounds the call.  The first
// kernel: every workgroup of a row computes the post-norm sum of squares over
// the whole partial row itself (16-column blocks t, t + 256, ... per thread,
// then the fixed-order workgroup sum: the same bits in all of them), then
// the gated add of its slice, stores the new residual values and the slice's
// sum of their squares into slice_ss[row * S + slice]; the second kernel sums
// a row's S slice sums in slice order and writes its slice of out.  The
// kernel boundary orders the two; arithmetic as in the one-kernel form.
constexpr int kSplitThreads = 256;

__device__ __forceinline__ void unpack4(uint2 u, double (&v)[4]) {
  v[0] = (double)bf16_lo(u.x);
  v[1] = (double)bf16_hi(u.x);
  v[2] = (double)bf16_lo(u.y);
  v[3] = (double)bf16_hi(u.y);
}

__global__ __launch_bounds__(kSplitThreads) void dual_gate_kernel(
    const uint16_t *__restrict__ partial, float *__restrict__ residual,
    const uint16_t *__restrict__ post_w, float post_gc, float post_eps,
    const uint16_t *__restrict__ alpha, float alpha_scalar, const uint16_t *__restrict__ beta,
    double *__restrict__ slice_ss, int H, int slices) {
  const int row = blockIdx.x / slices, sl = blockIdx.x - row * slices;
  const int tid = threadIdx.x;
  const int c0 = sl * kDualSlice + 4 * tid;
  const bool mine = c0 < H;  // H % 16 == 0: all four columns or none
  const uint16_t *prow = partial + (size_t)row * H;
  float *srow = residual + (size_t)row * H;

  // The thread's own columns first, as raw bits, all in flight during the
  // reduction (an absent post weight or alpha reads beta's bits, unused).
  uint2 pr = make_uint2(0, 0), gr = pr, ar = pr, br = pr;
  f32x4 sv = {0.f, 0.f, 0.f, 0.f};
  if (mine) {
    pr = *reinterpret_cast<const uint2 *>(prow + c0);
    sv = *reinterpret_cast<const f32x4 *>(srow + c0);
    gr = *reinterpret_cast<const uint2 *>((post_w ? post_w : beta) + c0);
    ar = *reinterpret_cast<const uint2 *>((alpha ? alpha : beta) + c0);
    br = *reinterpret_cast<const uint2 *>(beta + c0);
  }

  const double ss = sum_squares<kSplitThreads>(prow, H / 16, tid);
  __shared__ double slots[kSplitThreads / 64], slots2[kSplitThreads / 64];
  const double inv =
      1.0 / sqrt(block_sum<kSplitThreads>(ss, slots) / (double)H + (double)post_eps);

  double ss2 = 0.0;
  if (mine) {
    double p[4], g[4], a[4], b[4], s[4];
    unpack4(pr, p);
    unpack4(br, b);
    if (post_w) {
      unpack4(gr, g);
#pragma unroll
      for (int j = 0; j < 4; ++j) g[j] += (double)post_gc;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) g[j] = 1.0;
    }
    if (alpha) {
      unpack4(ar, a);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = (double)alpha_scalar;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = (double)sv[j];
    f32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double h = (double)__uint_as_float(f64_to_bf16(p[j] * inv * g[j]) << 16);
      const float v = (float)(a[j] * s[j] + b[j] * h);
      o[j] = v;
      ss2 += (double)v * (double)v;
    }
    *reinterpret_cast<f32x4 *>(srow + c0) = o;
  }
  const double slice_total = block_sum<kSplitThreads>(ss2, slots2);
  if (tid == 0) slice_ss[(size_t)row * slices + sl] = slice_total;
}

__global__ __launch_bounds__(kSplitThreads) void dual_out_kernel(
    const float *__restrict__ residual, const uint16_t *__restrict__ next_w, float pre_gc,
    float pre_eps, const double *__restrict__ slice_ss, uint16_t *__restrict__ out, int H,
    int slices) {
  const int row = blockIdx.x / slices, sl = blockIdx.x - row * slices;
  const int c0 = sl * kDualSlice + 4 * threadIdx.x;
  if (c0 >= H) return;
  // The thread's columns first, then the row's slice sums eight at a time
  // (loads in flight together), summed in slice order.
  const f32x4 sv = *reinterpret_cast<const f32x4 *>(residual + (size_t)row * H + c0);
  const uint2 wr = *reinterpret_cast<const uint2 *>(next_w + c0);
  const double *ps = slice_ss + (size_t)row * slices;
  double ss2 = 0.0;
  for (int i0 = 0; i0 < slices; i0 += 8) {
    double part[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) part[i] = i0 + i < slices ? ps[i0 + i] : 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i0 + i < slices) ss2 = i0 + i == 0 ? part[0] : ss2 + part[i];
  }
  const double inv2 = 1.0 / sqrt(ss2 / (double)H + (double)pre_eps);
  double w[4];
  unpack4(wr, w);
  unsigned yb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) yb[j] = f64_to_bf16((double)sv[j] * inv2 * (w[j] + (double)pre_gc));
  *reinterpret_cast<uint2 *>(out + (size_t)row * H + c0) =
      make_uint2(yb[0] | (yb[1] << 16), yb[2] | (yb[3] << 16));
}

}  // namespace

hipError_t launch_dual_norm(const uint16_t *partial, float *residual, const uint16_t *post_w,
                            float post_gc, float post_eps, const uint16_t *alpha,
                            float alpha_scalar, const uint16_t *beta, const uint16_t *next_w,
                            float pre_gc, float pre_eps, uint16_t *out, int M, int H,
                            DeviceState &st, hipStream_t stream) {
  const int slices = (H + kDualSlice - 1) / kDualSlice;
  if (H >= 2 * kDualSlice && (size_t)M * slices <= kNormPartials) {
    hipLaunchKernelGGL(dual_gate_kernel, dim3(M * slices), dim3(kSplitThreads), 0, stream,
                       partial, residual, post_w, post_gc, post_eps, alpha, alpha_scalar, beta,
                       st.norm_partials, H, slices);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dual_out_kernel, dim3(M * slices), dim3(kSplitThreads), 0, stream,
                       residual, next_w, pre_gc, pre_eps, st.norm_partials, out, H, slices);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dual_norm_kernel, dim3(M), dim3(kDualThreads), 0, stream, partial,
                     residual, post_w, post_gc, post_eps, alpha, alpha_scalar, beta, next_w,
                     pre_gc, pre_eps, out, H);
  return hipGetLastError();
}

}  // namespace skinny
