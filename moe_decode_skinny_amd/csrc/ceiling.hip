// libskinny_ceiling: measurement reference kernels for the small-M decode
// GEMM's benchmark (unpooler page, module description: the weight stream is
// the call's dominant cost), built as a library of their own beside
// libskinny (include/skinny_ceiling.h).  They compute nothing of the method: one launches an empty kernel, the other
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
// The stream-and-store reference reads the same layout and then ends the way
// a GEMM workgroup does: each lane's XOR goes through LDS, wave 0 combines
// the 8 waves' words after a barrier and stores 64 words, so its result
// depends on every byte read and the launch ends with a dependent store.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "device.h"
#include "skinny_ceiling.h"

namespace skinny {
namespace {

constexpr unsigned kCeilingPattern = 0x5EC0DE42u;  // the sink trigger (include/skinny_ceiling.h)

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

template <int L>
__global__ __launch_bounds__(512) void ceiling_stream_store_kernel(
    const uint8_t *__restrict__ src, unsigned bytes, unsigned *__restrict__ out) {
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
  __shared__ unsigned words[8][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  words[wave][lane] = x;
  __syncthreads();
  if (wave != 0) return;
  unsigned r = words[0][lane];
#pragma unroll
  for (int w = 1; w < 8; ++w) r ^= words[w][lane];
  out[blockIdx.x * 64 + lane] = r;
}

thread_local char g_error[256] = "";

int fail(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return status;
}

// The current device is a gfx950 GPU (the kernels are built for it only).
int check_device() {
  int dev = -1;
  hipDeviceProp_t prop;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(SKINNY_EDEVICE, "no current HIP device");
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(SKINNY_EDEVICE, "cannot query device %d", dev);
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(SKINNY_EDEVICE, "device %d is %s; the kernels are built for gfx950", dev,
                prop.gcnArchName);
  return SKINNY_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) return fail(SKINNY_ELAUNCH, "launch failed: %s", hipGetErrorString(e));
  g_error[0] = 0;
  return SKINNY_OK;
}

}  // namespace
}  // namespace skinny

using namespace skinny;

extern "C" {

int skinny_ceiling_empty(void *stream) {
  if (int st = check_device()) return st;
  hipLaunchKernelGGL(ceiling_empty_kernel, dim3(1), dim3(64), 0,
                     static_cast<hipStream_t>(stream));
  return launched(hipGetLastError());
}

int skinny_ceiling_stream(const void *src, long long bytes, void *sink, int loads_per_lane,
                          void *stream) {
  if (!src || !sink) return fail(SKINNY_EINVAL, "null pointer");
  if ((uintptr_t)src % 16 || (uintptr_t)sink % 4)
    return fail(SKINNY_EINVAL, "src must be 16-byte and sink 4-byte aligned");
  if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8)
    return fail(SKINNY_EINVAL, "loads_per_lane=%d: needs 1, 2, 4 or 8", loads_per_lane);
  const long long unit = 8192LL * loads_per_lane;
  if (bytes <= 0 || bytes % unit || bytes > 0x7FFFF000LL)
    return fail(SKINNY_EINVAL, "bytes=%lld: needs a positive multiple of %lld below 2^31", bytes,
                unit);
  if (int st = check_device()) return st;
  const uint8_t *s = static_cast<const uint8_t *>(src);
  unsigned *k = static_cast<unsigned *>(sink);
  const unsigned n = (unsigned)bytes;
  const dim3 grid(n / (8192u * loads_per_lane)), block(512);
  hipStream_t h = static_cast<hipStream_t>(stream);
  switch (loads_per_lane) {
    case 1: hipLaunchKernelGGL(ceiling_stream_kernel<1>, grid, block, 0, h, s, n, k); break;
    case 2: hipLaunchKernelGGL(ceiling_stream_kernel<2>, grid, block, 0, h, s, n, k); break;
    case 4: hipLaunchKernelGGL(ceiling_stream_kernel<4>, grid, block, 0, h, s, n, k); break;
    default: hipLaunchKernelGGL(ceiling_stream_kernel<8>, grid, block, 0, h, s, n, k); break;
  }
  return launched(hipGetLastError());
}

int skinny_ceiling_stream_store(const void *src, long long bytes, void *out, int loads_per_lane,
                                void *stream) {
  if (!src || !out) return fail(SKINNY_EINVAL, "null pointer");
  if ((uintptr_t)src % 16 || (uintptr_t)out % 4)
    return fail(SKINNY_EINVAL, "src must be 16-byte and out 4-byte aligned");
  if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8)
    return fail(SKINNY_EINVAL, "loads_per_lane=%d: needs 1, 2, 4 or 8", loads_per_lane);
  const long long unit = 8192LL * loads_per_lane;
  if (bytes <= 0 || bytes % unit || bytes > 0x7FFFF000LL)
    return fail(SKINNY_EINVAL, "bytes=%lld: needs a positive multiple of %lld below 2^31", bytes,
                unit);
  if (int st = check_device()) return st;
  const uint8_t *s = static_cast<const uint8_t *>(src);
  unsigned *o = static_cast<unsigned *>(out);
  const unsigned n = (unsigned)bytes;
  const dim3 grid(n / (8192u * loads_per_lane)), block(512);
  hipStream_t h = static_cast<hipStream_t>(stream);
  switch (loads_per_lane) {
    case 1: hipLaunchKernelGGL(ceiling_stream_store_kernel<1>, grid, block, 0, h, s, n, o); break;
    case 2: hipLaunchKernelGGL(ceiling_stream_store_kernel<2>, grid, block, 0, h, s, n, o); break;
    case 4: hipLaunchKernelGGL(ceiling_stream_store_kernel<4>, grid, block, 0, h, s, n, o); break;
    default: hipLaunchKernelGGL(ceiling_stream_store_kernel<8>, grid, block, 0, h, s, n, o); break;
  }
  return launched(hipGetLastError());
}

const char *skinny_ceiling_last_error(void) { return g_error; }

}  // extern "C"
