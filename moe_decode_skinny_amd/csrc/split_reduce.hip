// The split-K reduction of the small-M decode GEMM: y[t][n] = bf16( sum over
// s = 0..S-1, in that order, of partials[s][t][n] ).  The order is set by the
// split count alone, so a launch shape always gives the same bits (unpooler
// page, module description).
//
// It runs as the second kernel of a split launch, on the same stream, so the
// kernel boundary orders it after every partial store of the first: no
// workgroup ever waits for another.  One thread per four consecutive outputs
// of a token row: S 16-byte loads (coalesced across the row) and one 8-byte
// store (two with a zero-copy publish, whose stage word thread 0 sets).
// S is 2, 4, 8 or 16 (the split counts a launch may have).
#include "internal.h"

namespace skinny {
namespace {

constexpr int kReduceThreads = 256;

// S, the split count, is a template parameter: the S loads of a thread are
// issued together and added in order after them.
template <int S>
__global__ __launch_bounds__(kReduceThreads) void split_reduce_kernel(
    const float *__restrict__ partials, uint16_t *__restrict__ y, int M, int N, Publish pub) {
  const int i = blockIdx.x * kReduceThreads + threadIdx.x;
  if (i == 0) publish_stage_word(pub);
  const int quads = M * (N / 4);
  if (i >= quads) return;
  const int t = i / (N / 4), n = (i - t * (N / 4)) * 4;
  const size_t plane = (size_t)M * N;
  f32x4 v[S];
#pragma unroll
  for (int s = 0; s < S; ++s)
    v[s] = *reinterpret_cast<const f32x4 *>(partials + s * plane + (size_t)t * N + n);
  f32x4 sum = v[0];
#pragma unroll
  for (int s = 1; s < S; ++s) sum += v[s];
  const unsigned lo = f32_to_bf16(sum[0]) | (f32_to_bf16(sum[1]) << 16);
  const unsigned hi = f32_to_bf16(sum[2]) | (f32_to_bf16(sum[3]) << 16);
  store_out_device(y + (size_t)t * N + n, lo, hi);
  if (uint16_t *slot = publish_slot(pub, N))
    *reinterpret_cast<uint2 *>(slot + (size_t)t * N + n) =
        make_uint2(publish_pair(lo), publish_pair(hi));
}

}  // namespace

hipError_t launch_split_reduce(const float *partials, uint16_t *y, int M, int N, int S,
                               const Publish &pub, hipStream_t stream) {
  const int quads = M * (N / 4);
  dim3 grid((quads + kReduceThreads - 1) / kReduceThreads), block(kReduceThreads);
  using Kernel = void (*)(const float *, uint16_t *, int, int, Publish);
  Kernel k = S == 2 ? split_reduce_kernel<2>
           : S == 4 ? split_reduce_kernel<4>
           : S == 8 ? split_reduce_kernel<8>
           : S == 16 ? split_reduce_kernel<16>
                     : nullptr;
  if (!k) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k, grid, block, 0, stream, partials, y, M, N, pub);
  return hipGetLastError();
}

}  // namespace skinny
