// Measurement reference kernels for the small-M decode GEMM (unpooler page,
// module description: the weight stream is the call's dominant cost).  They
// compute nothing of the method: one launches an empty kernel, the other
// streams a buffer the way the GEMM kernels stream weights (16-byte loads
// with the streaming cache policy, each load instruction 1 KiB of contiguous
// memory, every load issued before the first use), so that the time of a
// single launch and of a single launch that only streams the same bytes can
// be measured beside the GEMM calls on the same device and stream.
//
// Stream layout: workgroup b of 512 threads owns bytes [b * 8192 L,
// (b + 1) * 8192 L); load i of thread t reads the 16 bytes at offset
// 8192 i + 16 t of that range.  Each thread XORs the dwords it read and
// writes 1 to sink[b] only if the result equals kCeilingPattern, which keeps
// the loads live; with any other data the sink is not written.
#include "internal.h"

namespace skinny {
namespace {

constexpr unsigned kCeilingPattern = 0x5EC0DE42u;  // the sink trigger (include/skinny.h)

__global__ void ceiling_empty_kernel() {}

template <int L>
__global__ __launch_bounds__(512) void ceiling_stream_kernel(const uint8_t *__restrict__ src,
                                                             unsigned bytes,
                                                             unsigned *__restrict__ sink) {
  const __amdgpu_buffer_rsrc_t res = buffer_rsrc(src, bytes);
  const unsigned base = blockIdx.x * (8192u * L) + threadIdx.x * 16u;
  u32x4 v[L];
#pragma unroll
  for (int i = 0; i < L; ++i)
    v[i] = __builtin_amdgcn_raw_buffer_load_b128(res, (int)(base + 8192u * i), 0, kCacheNT);
  __builtin_amdgcn_sched_barrier(0);
  unsigned x = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (x == kCeilingPattern) sink[blockIdx.x] = 1u;
}

}  // namespace

hipError_t launch_ceiling_empty(hipStream_t stream) {
  hipLaunchKernelGGL(ceiling_empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError();
}

hipError_t launch_ceiling_stream(const uint8_t *src, unsigned bytes, unsigned *sink, int L,
                                 hipStream_t stream) {
  const dim3 grid(bytes / (8192u * L)), block(512);
  switch (L) {
    case 1: hipLaunchKernelGGL(ceiling_stream_kernel<1>, grid, block, 0, stream, src, bytes, sink); break;
    case 2: hipLaunchKernelGGL(ceiling_stream_kernel<2>, grid, block, 0, stream, src, bytes, sink); break;
    case 4: hipLaunchKernelGGL(ceiling_stream_kernel<4>, grid, block, 0, stream, src, bytes, sink); break;
    case 8: hipLaunchKernelGGL(ceiling_stream_kernel<8>, grid, block, 0, stream, src, bytes, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace skinny
