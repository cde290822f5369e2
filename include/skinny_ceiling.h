/*
 * libskinny_ceiling -- measurement references for the benchmark of libskinny.
 * Not part of libskinny's ABI and not steps of the method: a separate shared
 * library (moe_decode_skinny_amd/libskinny_ceiling.so) that the benchmark and
 * its tests load beside libskinny.
 *
 * The decode GEMM's dominant cost is streaming its weight once ("unpooler"
 * page, vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.gemm.unpooler,
 * module description: weights are loaded first, and the call is one pass over
 * them).  These calls measure, on the caller's device and stream, what one
 * launch costs by itself, how fast one launch can stream a buffer the way the
 * GEMM kernels stream weights, and how fast when it also ends as a GEMM
 * workgroup does (words combined across its waves through LDS, then stored),
 * so that a GEMM call's time can be set against the ceiling a single launch
 * reaches.
 *
 * Conventions: pointers are device pointers owned by the caller; `stream` is
 * a hipStream_t (NULL = the default stream) of the calling thread's current
 * HIP device, which must be a gfx950 GPU; work is only enqueued.  A bad
 * argument returns a negative status (the skinny_status values of skinny.h)
 * and enqueues nothing, with the reason in skinny_ceiling_last_error().
 */
#ifndef SKINNY_CEILING_H
#define SKINNY_CEILING_H

#ifdef __cplusplus
extern "C" {
#endif

/* Measurement reference (unpooler page, module description: the cost of one
 * call is its weight stream): launches one empty 64-thread workgroup.
 * Errors: -3 (no device, or not gfx950), -4 (launch refused). */
int skinny_ceiling_empty(void *stream);

/* Measurement reference (unpooler page, module description: the cost of one
 * call is its weight stream): reads the `bytes` bytes at src once, with
 * bytes / (8192 * loads_per_lane) workgroups of 512 threads; thread t of
 * workgroup b issues loads_per_lane 16-byte loads with the streaming cache
 * policy, load i at byte b * 8192 * loads_per_lane + 8192 i + 16 t, all
 * before the first use.
 *   src             device bytes, 16-byte aligned
 *   bytes           a positive multiple of 8192 * loads_per_lane, below 2^31
 *   sink            device u32 [bytes / (8192 * loads_per_lane)]; word b is
 *                   set to 1 only if some thread's XOR of the 32-bit words it
 *                   read equals 0x5EC0DE42, and is otherwise left as it was
 *   loads_per_lane  1, 2, 4 or 8
 * Errors: -1 (bad pointer, alignment or size), -3, -4. */
int skinny_ceiling_stream(const void *src, long long bytes, void *sink, int loads_per_lane,
                          void *stream);

/* Measurement reference (unpooler page, module description: the cost of one
 * call is its weight stream, and the call ends by storing its result): the
 * loads of skinny_ceiling_stream, same layout and sizes, then each
 * workgroup b stores 64 words:
 *   out[b * 64 + l] = XOR over waves w = 0..7 and loads i of the four 32-bit
 *                     words thread 64 w + l read in load i
 *   out   device u32 [64 * bytes / (8192 * loads_per_lane)], 4-byte aligned
 * Each wave's words pass through LDS and wave 0 combines them after a
 * barrier, as a GEMM workgroup sums its waves' partials before its store.
 * Errors: -1 (bad pointer, alignment or size), -3, -4. */
int skinny_ceiling_stream_store(const void *src, long long bytes, void *out, int loads_per_lane,
                                void *stream);

/* The reason for this thread's last non-zero status, "" if none (as
 * skinny_last_error does for libskinny; unpooler page,
 * Unpooler.unsupported: a call that cannot run gives its reason). */
const char *skinny_ceiling_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_CEILING_H */
