/*
 * libskinny — the small-M decode GEMM and its NVFP4 expert-input epilogue for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed follows three vLLM API pages on the Muse Spark specialized
 * decode:
 *   - "vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.gemm.unpooler"
 *     (module description; Unpooler.run; Unpooler.unsupported;
 *     launch_unsupported): y[M, N] = x[M, K] @ W[N, K]^T for 1 to 16 tokens,
 *     BF16 operands and result, FP32 sums, split-K partials added in an order
 *     that only the launch shape decides, so repeated runs give equal bits.
 *   - "vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.moe.pooler_gather"
 *     (module description; compile_norm_quant; cvt_e2m1x8_f32;
 *     cvt_f32_to_e4m3; nvfp4_compute_output_scale): RMSNorm with a gain
 *     center, then block-16 NVFP4 quantization.
 *   - "vllm.models.muse_spark.nvidia.specialized_decode.cutedsl.oproj.batt"
 *     (OProjection): the o_proj shard runs on the same small-M GEMM.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or keeps them.  Row-major, contiguous.
 *   - bfloat16 data is passed as its 16-bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *     enqueued; no call synchronizes with the host.
 *   - Arguments are checked on the host before anything is enqueued.  A bad
 *     argument returns a negative skinny_status and enqueues nothing;
 *     skinny_last_error() then gives the reason (thread-local string).
 *   - After skinny_init(), the compute calls allocate nothing, compile nothing
 *     and never synchronize, so they may be recorded into a HIP graph.
 */
#ifndef SKINNY_H
#define SKINNY_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum skinny_status {
  SKINNY_OK = 0,
  SKINNY_EINVAL = -1,      /* null or misaligned pointer, bad M/N/K/P, overlap */
  SKINNY_EUNSUPPORTED = -2,/* valid problem, but no launch for this shape      */
  SKINNY_EDEVICE = -3,     /* no device, or the device is not gfx950          */
  SKINNY_ELAUNCH = -4,     /* the HIP runtime refused the launch              */
  SKINNY_ENOTINIT = -5     /* compute call on a device before skinny_init()   */
} skinny_status;

/* Kernel families of the GEMM. */
enum {
  SKINNY_PATH_DOT2 = 0,    /* VALU bf16 dot2: lanes run along K, any row count  */
  SKINNY_PATH_MFMA = 1,    /* bf16 MFMA 16x16x32: 16 weight rows x 16 tokens    */
  SKINNY_PATH_MFMA_LDS = 2,/* ring only: MFMA with each wave's weights loaded
                              row by row and re-laid out through LDS; same
                              operands and results as SKINNY_PATH_MFMA        */
  SKINNY_PATH_MFMA_4X4 = 3 /* bf16 MFMA 4x4x4 in 16 blocks: lanes load along K
                              as in DOT2, then a transpose in each 4-lane
                              group gives 4 weight rows x 4 tokens a block    */
};

/* A launch shape of the GEMM: the counterpart of the unpooler page's
 * UnpoolerShape (splits, kw, accs) and the pooler page's PoolerGemmShape.
 * (M, N, K, skinny_launch) fixes the launch completely, and with it the order
 * in which every output's products are added.
 *
 *   MFMA: a workgroup owns rows = 16 F output features (F = 1, 2 or 4 MFMA
 *         tiles sharing one LDS copy of the activations) and one of `splits`
 *         K ranges; the range is cut into KW pieces of kw = 32 * chunks
 *         consecutive K, and waves = F * KW (one wave per tile and piece),
 *         each keeping `accs` FP32 accumulators.
 *   DOT2: a workgroup owns `rows` output features; each wave owns
 *         kw = 512 * chunks consecutive K (64 lanes x 8 bf16 per chunk);
 *         waves = ceil(K / (splits * kw)) <= 16 (more than 8 only for the
 *         register-light variants).
 *   MFMA_4X4: a workgroup owns rows = 4 or 8 output features; each wave owns
 *         kw = 128 * chunks consecutive K (16 blocks x 8 bf16 per chunk,
 *         chunks 4 or 8: whole groups of 512 K, loaded as 1 KiB row pieces)
 *         and the workgroup's tokens in sets of 4; waves = ceil(K / (splits *
 *         kw)) <= 16.  `accs` = H token groups (1, 2 or 4; a tile
 *         decomposition along M): group h takes tokens 4Qh .. 4Qh + 4Q - 1,
 *         Q = ceil(ceil(M / H) / 4) rounded up to 1, 2 or 4 sets, and every
 *         group must get a token (ceil(M / 4Q) == H); H = 1 is all M tokens
 *         in each workgroup.  A token's sums do not depend on H.
 * In all three, wave partials are summed in LDS in wave order; with splits > 1
 * each workgroup writes an FP32 partial and splits 0..S-1 are summed in that
 * order: by the last workgroup of the output block to finish (MFMA_4X4) or by
 * a second kernel on the same stream (the others). */
typedef struct skinny_launch {
  int path;   /* SKINNY_PATH_MFMA, SKINNY_PATH_DOT2 or SKINNY_PATH_MFMA_4X4 */
  int splits; /* S in {1, 2, 4, 8, 16}: workgroups along K per output block   */
  int waves;  /* waves per workgroup (see above)                             */
  int chunks; /* K chunks per wave: MFMA 1..16, DOT2 1, 2, 4, MFMA_4X4 4, 8  */
  int accs;   /* MFMA: accumulators per wave, 1, 2 or 4; MFMA_4X4: token
                 groups, 1, 2 or 4; DOT2: 1                                  */
  int rows;   /* features per workgroup: MFMA 16, 32, 64; DOT2 2..16;
                 MFMA_4X4 4, 8                                                */
} skinny_launch;

/* Prepare `device` (a HIP ordinal) for the compute calls (unpooler page,
 * Unpooler: the layer is set up ahead of time, outside graph capture, after
 * which its run call may be recorded into a graph and needs no allocation;
 * pooler_gather page, Pooler: the same for the pooler): checks that it is a gfx950 GPU, allocates the
 * library's split-K workspace on it (8 MiB of FP32 partials, enough for
 * S * M * N <= 2^21, and 512 KiB of split hand-off counters, zeroed) and the
 * dual norm's buffer (512 KiB of per-slice sums), sets the kernels' LDS
 * limits, and looks up the device's address of the static scratch array of
 * skinny_gemm_bf16_noalloc and zeroes that array's counters.
 * Call it before any graph capture.  Idempotent.  Returns SKINNY_OK,
 * SKINNY_EDEVICE or SKINNY_ELAUNCH (allocation failure). */
int skinny_init(int device);

/* Every call below runs on the calling thread's current HIP device (as set by
 * hipSetDevice), which must have been prepared by skinny_init; every pointer
 * it takes must be memory of that device, and the stream a stream of it. */

/* y[M, N] = bf16( x[M, K] @ W[N, K]^T ), FP32 accumulation (unpooler page,
 * module description and Unpooler.run).
 *   x       bf16 [M, K], 16-byte aligned
 *   W       bf16 [N, K], 16-byte aligned
 *   y       bf16 [M, N], 16-byte aligned; only these M rows are written
 *   M       1..16 tokens
 *   N       output features, N > 0, N % 16 == 0, N <= 2^24
 *   K       reduction length, K > 0, K % 8 == 0 (16-byte rows); the longest
 *           K with a launch is 16 splits x 16 waves x the widest DOT2 wave
 *           slice: 524288 for M <= 4, 262144 for M <= 8, 131072 for M <= 16
 *           (longer K: SKINNY_EUNSUPPORTED)
 *   splits  0 = let the chooser pick; otherwise S in {1, 2, 4, 8, 16}
 * x, W and y must not overlap.  The result is bitwise identical for the same
 * (M, N, K, launch) on one device.  A launch with S > 1 uses the device's
 * workspace: the 16-block path (SKINNY_PATH_MFMA_4X4) adds the splits inside
 * its one kernel (the last of each output block's workgroups to finish, with
 * self-resetting counters), the other paths enqueue a second kernel for it;
 * the splits are added in the order s = 0..S-1 either way.  Two such calls
 * must not run concurrently on different streams of one device (calls on one
 * stream are ordered).
 * For some measured shapes the chosen launch runs as a persistent walk over
 * the output blocks (the layer-ring kernel with one item, see
 * skinny_choose_walk); the result is still bitwise that of
 * skinny_gemm_bf16_launch at the launch skinny_choose returns.
 * Errors: SKINNY_EINVAL, SKINNY_EUNSUPPORTED, SKINNY_ENOTINIT, SKINNY_ELAUNCH. */
int skinny_gemm_bf16(const void *x, const void *W, void *y, int M, int N,
                     int K, int splits, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): skinny_gemm_bf16 with the
 * same arguments, chooser, kernels and bits, except that a launch with
 * splits > 1 keeps its FP32 partials (2^18 floats at most) and, on the
 * 16-block path, its split hand-off counters (2048 words, each on its own
 * 256 bytes) in a static device array of the library (1.5 MiB, one per
 * device, held until the process ends; its address is looked up by
 * skinny_init) instead of the workspace skinny_init allocates.  The call
 * allocates and frees nothing.  skinny_init zeroes the counters and every
 * hand-off returns its counter to zero, so they are zero between calls; the
 * partials need no clearing, since each call writes every partial it reads.
 * Every call on a device shares that device's array: calls that overlap on
 * one device (different streams, or host threads without ordering) race.
 * Errors: as skinny_gemm_bf16, and SKINNY_EUNSUPPORTED when the chosen
 * launch's splits x M x N exceeds 2^18 (skinny_gemm_bf16 takes up to 2^21). */
int skinny_gemm_bf16_noalloc(const void *x, const void *W, void *y, int M, int N,
                             int K, int splits, void *stream);

/* The same GEMM at an explicit launch shape (unpooler page, compile_unpooler:
 * one kernel per shape and launch parameters -- splits, K per wave,
 * accumulators -- shared by every layer of that shape).  For sweeps and
 * tests; arguments and errors as skinny_gemm_bf16. */
int skinny_gemm_bf16_launch(const void *x, const void *W, void *y, int M,
                            int N, int K, const skinny_launch *launch,
                            void *stream);

/* The chooser: the launch shape skinny_gemm_bf16 uses for (M, N, K, splits)
 * (unpooler page, Unpooler and compile_unpooler: a layer is built with one
 * launch shape, UNPOOLER by default, whose splits, kw and accs select the
 * compiled kernel; pooler_gather page, PoolerGemmShape: the pooler GEMM's
 * block size, outputs per block and K unroll).  Here the shape is measured
 * per (M, N, K) instead of fixed per layer.  Pure host function of its
 * arguments.  Returns SKINNY_OK and fills *out, or SKINNY_EINVAL /
 * SKINNY_EUNSUPPORTED with the reason in skinny_last_error(). */
int skinny_choose(int M, int N, int K, int splits, skinny_launch *out);

/* Why there is no launch for (M, N, K, splits): the status the GEMM would
 * return for valid pointers (unpooler page, Unpooler.unsupported and
 * launch_unsupported).  SKINNY_OK when supported; the reason otherwise in
 * skinny_last_error().  Host only. */
int skinny_gemm_unsupported(int M, int N, int K, int splits);

/* Why (M, N, K) cannot run at `launch` (unpooler page, launch_unsupported:
 * a weight shape that the given splits, K per wave and accumulators cannot
 * serve is reported with its reason); SKINNY_OK when it can.  Host only. */
int skinny_launch_unsupported(int M, int N, int K, const skinny_launch *launch);

/* The next boundary's mailbox for a zero-copy publish (unpooler page, module
 * description, zero-copy epilogue and ticket stage; pooler_gather page, module
 * description and compile_gather).  On one GPU the multicast into the
 * peers' copies becomes a store into this device buffer.
 *   data         bf16 [3][tp][capacity][width] on the device, 16-byte aligned:
 *                three stages of one slot per rank
 *   stage_state  int32 [2] on the device: [0] the stage a publish writes
 *                (0..2), [1] set to that stage by the publish; not used with
 *                a ticket (may then be NULL)
 *   ticket       NULL, or int32 [1] on the device holding stage << 16: the
 *                stage is its upper 16 bits and no stage word is written
 *   tp, rank     ranks sharing the mailbox and this rank's slot, 0 <= rank < tp
 *   capacity     token rows per slot, >= M
 *   width        columns per row, == N
 * The stage is read on the device when the kernel runs; a stage outside 0..2
 * publishes nothing (y is still stored). */
typedef struct skinny_mailbox {
  void *data;
  int *stage_state;
  const int *ticket;
  int tp, rank, capacity, width;
} skinny_mailbox;

/* The GEMM with its zero-copy publish (unpooler page, module description,
 * zero-copy epilogue and ticket stage): y as skinny_gemm_bf16 computes it, and
 * the same M rows into mailbox->data[stage][rank][0..M) with each bf16 -0.0
 * stored as +0.0 (-0.0 is the mailbox's "not yet written" sentinel); without a
 * ticket, stage_state[1] is set to the stage.  The other slots, rows >= M
 * of this slot, stage_state[0] and the ticket are not written.
 *   launch   NULL = the chooser's launch; else an explicit launch shape
 * The mailbox, stage state and ticket must not overlap x, W or y.  Two
 * publishes into one slot and stage race unless ordered on one stream.
 * Errors: SKINNY_EINVAL (also: width != N, M > capacity, bad rank),
 * SKINNY_EUNSUPPORTED, SKINNY_ENOTINIT, SKINNY_ELAUNCH. */
int skinny_gemm_bf16_publish(const void *x, const void *W, void *y, int M,
                             int N, int K, const skinny_launch *launch,
                             const skinny_mailbox *mailbox, void *stream);

/* A launch of the layer ring (skinny_gemm_bf16_ring_launch).
 *   gemm        the per-tile launch shape, splits = 1: DOT2 (rows 2, 4 or 8,
 *               chunks 1, 2, 4; waves = ceil(K / (512 chunks)) <= 8, or up to
 *               16 for the register-light variants) or MFMA
 *               (rows 16, 32, 64; chunks 1..16; accs 1 or 2; waves =
 *               rows / 16 * ceil(K / (32 chunks)) <= 16, <= 8 at 16 chunks)
 *               or MFMA_LDS (as MFMA with chunks 2..16, and the staging
 *               regions, waves x 16 x (64 chunks + 16) bytes, plus 2 KiB per
 *               wave, within the 160 KiB of LDS) or MFMA_4X4 (rows 4 or 8,
 *               chunks 4 or 8, waves = ceil(K / (128 chunks)) <= 16, accs 1:
 *               a ring tile takes all M tokens)
 *   segment     consecutive output blocks of one item a workgroup takes in a
 *               row, keeping that item's activations in registers; it
 *               divides N / gemm.rows
 *   workgroups  persistent workgroups, 1 .. count * N / (rows * segment);
 *               workgroup b takes segment slots b, b + workgroups, ...
 *   order       how slots map to segments: SKINNY_RING_ITEM_MAJOR (slot t is
 *               segment t of the item-major order) or SKINNY_RING_XCD_LOCAL
 *               (when workgroups is a multiple of 8, slot t of the first
 *               8 (count / 8) items belongs to an item congruent to t mod 8,
 *               so all segments of such an item run on one of the eight XCDs
 *               and its activations reach one L2; the other items, and any
 *               workgroup count that is not a multiple of 8, item-major).
 *               The order never changes a result. */
enum { SKINNY_RING_ITEM_MAJOR = 0, SKINNY_RING_XCD_LOCAL = 1 };
typedef struct skinny_ring_launch {
  skinny_launch gemm;
  int segment;
  int workgroups;
  int order;
} skinny_ring_launch;

/* The layer ring: `count` independent GEMMs y_i = bf16(x_i @ W_i^T) of one
 * shape (M, N, K) in one persistent launch (unpooler page, module
 * description: weight loads are issued ahead of the wait on the previous
 * kernel and activation loads after it, which overlaps one layer's weight
 * stream with the tail of the layer before).  Each workgroup has the weights of its next tile in
 * flight while it multiplies, reduces and stores the current one.
 *   x, W, y   HOST arrays of `count` device pointers, read during the call
 *             only; x[i] bf16 [M, K], W[i] bf16 [N, K], y[i] bf16 [M, N], all
 *             16-byte aligned
 *   count     1..64 items
 *   M, N, K   as for skinny_gemm_bf16
 * The items run concurrently: no y[i] may overlap any x[j], W[j] or another
 * y[j] (a chain whose x[i + 1] is y[i] needs one call per item).  Every y[i]
 * is bitwise identical to skinny_gemm_bf16_launch at the ring's gemm shape
 * (with MFMA for MFMA_LDS; when that shape is also a valid single-call
 * launch), whatever the segment and workgroup count.  Uses no workspace, so ring calls on
 * different streams may overlap.
 * Errors: SKINNY_EINVAL, SKINNY_EUNSUPPORTED, SKINNY_ENOTINIT, SKINNY_ELAUNCH. */
int skinny_gemm_bf16_ring(const void *const *x, const void *const *W,
                          void *const *y, int count, int M, int N, int K,
                          void *stream);

/* The ring at an explicit launch (see skinny_ring_launch; unpooler page,
 * module description and compile_unpooler, as for skinny_gemm_bf16_ring and
 * skinny_gemm_bf16_launch).  Arguments and errors as skinny_gemm_bf16_ring. */
int skinny_gemm_bf16_ring_launch(const void *const *x, const void *const *W,
                                 void *const *y, int count, int M, int N,
                                 int K, const skinny_ring_launch *launch,
                                 void *stream);

/* The ring's chooser: the launch skinny_gemm_bf16_ring uses for (M, N, K,
 * count) (unpooler page, Unpooler and compile_unpooler, as for
 * skinny_choose).  Host only.  SKINNY_OK, or SKINNY_EINVAL /
 * SKINNY_EUNSUPPORTED with the reason in skinny_last_error(). */
int skinny_ring_choose(int M, int N, int K, int count, skinny_ring_launch *out);

/* Why (M, N, K, count) cannot run at the ring launch `launch` (unpooler
 * page, launch_unsupported, as for skinny_launch_unsupported); SKINNY_OK
 * when it can.  Host only. */
int skinny_ring_launch_unsupported(int M, int N, int K, int count,
                                   const skinny_ring_launch *launch);

/* How skinny_gemm_bf16 runs (M, N, K, splits), for profiling and tests: on
 * SKINNY_OK, out->segment == 0 means the plain kernel at out->gemm (the
 * launch skinny_choose returns); otherwise the call is exactly
 * skinny_gemm_bf16_ring_launch with one item at *out (out->gemm then has the
 * same arithmetic as skinny_choose's launch; SKINNY_PATH_MFMA_LDS stands for
 * SKINNY_PATH_MFMA with the ring's staged weight loads).  Weight loads go
 * ahead of the activations (unpooler page, module description); the walk
 * keeps one block's weights in flight while the previous block is
 * finished.  Pure host function; errors as skinny_choose. */
int skinny_choose_walk(int M, int N, int K, int splits, skinny_ring_launch *out);

/* The NVFP4 expert input (pooler_gather page, module description and
 * compile_norm_quant; nvfp4_compute_output_scale; cvt_e2m1x8_f32;
 * cvt_f32_to_e4m3), for each of the M rows of r:
 *   yn   = bf16( r * rsqrt(mean(r^2) + eps) * (norm_w + gain_center) )
 *   per 16-column block b:  sf_b = e4m3fn_rn_satfinite(gs * amax_b(|yn|) / 6)
 *                           os_b = gs / dec(sf_b), 0 when dec(sf_b) == 0
 *                           q_j  = e2m1_rn_satfinite(yn_j * os_b)
 *   r            bf16 [M, P], 16-byte aligned
 *   norm_w       bf16 [P], 16-byte aligned
 *   gain_center, eps   FP32 scalars (host values)
 *   global_scale FP32 [1] on the device, 4-byte aligned
 *   a            u8 [M, P / 2]: byte i = q_{2i} | q_{2i+1} << 4 (even column in
 *                the low nibble), 8-byte aligned
 *   a_sf         u8 [M, P / 16]: e4m3fn scale bytes, row-major, not swizzled
 *   M >= 1 rows; P > 0, P % 16 == 0
 * r and the outputs must not overlap.  Errors: SKINNY_EINVAL,
 * SKINNY_ENOTINIT, SKINNY_ELAUNCH. */
int skinny_rmsnorm_nvfp4(const void *r, const void *norm_w, float gain_center,
                         float eps, const float *global_scale, void *a,
                         void *a_sf, int M, int P, void *stream);

/* The BF16 edge-layer form of the same norm (pooler_gather page, module
 * description, "BF16 edge layers"): y = yn above, bf16 [M, P], 16-byte
 * aligned, with no quantization.  Same arguments and errors otherwise. */
int skinny_rmsnorm_bf16(const void *r, const void *norm_w, float gain_center,
                        float eps, void *y, int M, int P, void *stream);

/* The single-GPU dual norm after o_proj (oproj.batt page, AttentionBoundary:
 * post_attn_norm, gated add into the FP32 residual stream in place,
 * pre_ffn_norm into a BF16 output; the multi-GPU all-reduce before it is the
 * identity on one GPU).  The pages print neither the kernel nor its
 * constants; this computes the reading
 *   h_j        = bf16( p_j / sqrt(mean(p^2) + post_eps) * g_j ),
 *                g_j = post_w_j + post_gain_center, or 1 if post_w is NULL
 *   residual_j = f32( a_j * residual_j + beta_j * h_j ),
 *                a_j = alpha_j, or alpha_scalar if alpha is NULL
 *   out_j      = bf16( s_j / sqrt(mean(s^2) + pre_eps) * (next_w_j + pre_gain_center) )
 * per row, s being the updated residual row (binary64 arithmetic, one
 * rounding per narrowing).
 *   partial      bf16 [M, H]
 *   residual     float [M, H], read and written in place
 *   post_w       bf16 [H] or NULL; alpha bf16 [H] or NULL; beta, next_w bf16 [H]
 *   out          bf16 [M, H]
 *   M >= 1 rows; H > 0, H % 16 == 0; every array 16-byte aligned
 * partial, residual and out must not overlap, nor a weight the residual or
 * out.  Rows of H >= 2048 run as two kernels that pass per-slice sums
 * through the device's dual-norm buffer (from skinny_init): two such calls
 * must not run concurrently on different streams of one device (calls on
 * one stream are ordered).  Errors: SKINNY_EINVAL, SKINNY_ENOTINIT,
 * SKINNY_ELAUNCH. */
int skinny_dual_norm(const void *partial, float *residual, const void *post_w,
                     float post_gain_center, float post_eps, const void *alpha,
                     float alpha_scalar, const void *beta, const void *next_w,
                     float pre_gain_center, float pre_eps, void *out, int M, int H,
                     void *stream);

/* The reason for the last non-OK status on this thread, "" if none
 * (unpooler page, Unpooler.unsupported: the reason string a call that
 * cannot run gives, which Unpooler raises as ValueError(reason)).  The
 * string is thread-local and valid until this thread's next call. */
const char *skinny_last_error(void);

/* Not a step of the method: the library's ABI version, major * 100 + minor. */
int skinny_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_H */
