/*
 * Oracle for the small-M decode GEMM and the RMSNorm -> NVFP4 expert input.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * CPU statement of what the GPU library computes.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path (the HIP library and its binding) never does.  It shares no
 * code, header, table or constant with the HIP sources.
 *
 * All arithmetic is IEEE binary64.  Products of two bfloat16 values are exact
 * in binary64 (8 + 8 significant bits), and every rounding to a narrow format
 * is done once, directly from the binary64 value.
 *
 * Sources (the three vLLM API pages on the Muse Spark specialized decode):
 *   [unpooler]  page "...specialized_decode.cutedsl.gemm.unpooler", module
 *               description: y[M, N] = x[M, K] @ W[N, K]^T for 1 to 16
 *               tokens, with BF16 operands and result and sums kept in FP32.
 *   [pooler]    page "...specialized_decode.cutedsl.moe.pooler_gather", module
 *               description: y = bf16(x * rsqrt(mean(x**2) + eps) *
 *               (weight + gain_center)), then NVFP4 over 16-column blocks:
 *               codes packed two to a byte in a, uint8 [b, P/2], the even
 *               column's code in bits 0-3; one float8_e4m3fn scale per
 *               block in a_sf, [b, P/16], row-major (no swizzle).
 *   [cvt]       same page, cvt_e2m1x8_f32 / cvt_f32_to_e4m3: round to nearest
 *               even with saturation to the largest finite value.
 *   [oscale]    same page, nvfp4_compute_output_scale: the output scale is the
 *               reciprocal of (decoded scale * reciprocal of global_scale),
 *               and 0 when the decoded scale is 0.
 *   [publish]   unpooler page, module description (zero-copy epilogue and
 *               ticket stage) and Unpooler.run; pooler_gather page, module
 *               description (BF16 edge layers: -0.0 is the mailbox sentinel,
 *               so publishers store -0.0 as +0.0) and compile_gather (the
 *               mailbox is BF16 [3, tp, capacity, hidden / tp]).
 *   [dual]      page "...specialized_decode.cutedsl.oproj.batt",
 *               AttentionBoundary: the partial goes through post_attn_norm,
 *               a gated add into the FP32 residual stream (in place, with
 *               the connection's alpha and beta) and pre_ffn_norm into the
 *               BF16 output; the post norm may have no weight.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - block scale: sf = e4m3(global_scale * amax / 6), 6 being the largest
 *     e2m1 magnitude (the kernel body is not printed);
 *   - the norm output is rounded to bfloat16 once, from the exact product;
 *   - a negative value that rounds to zero in e2m1 keeps its sign (code 0x8).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Readings for [publish] (the mailbox's body is not printed): the stage
 * state is int32 [2], [0] the stage a publish writes (the pages' NEXT_STAGE)
 * and [1] the word a publish sets to it (ACTIVE_STAGE); a ticket holds
 * stage << 16 and the stage is its upper 16 bits; a stage outside 0..2
 * publishes nothing. */

/* Readings for [dual] (the dual norm's body and constants are not printed;
 * PARITY UNPINNED by the pages beyond the order of its steps): both norms are
 * the pooler page's RMSNorm with their own eps and gain center, rounded to
 * bfloat16 once; a post norm without a weight scales by 1; the gated add is
 * stream = f32(alpha * stream + beta * h) with h the bfloat16 post-norm
 * output, alpha a scalar or per channel, beta per channel (bfloat16
 * parameters), one rounding to binary32 from binary64; the pre norm reads
 * the updated stream. */

/* ---------------------------------------------------------------- bfloat16 */

/* Value of a bfloat16 bit pattern: the upper half of a binary32. */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a binary64 value to bfloat16, to nearest with ties to even, in one
 * step.  bfloat16 has an 8-bit significand (7 stored bits), exponents of
 * binary32 and subnormals with step 2^-133. */
uint16_t oracle_bf16_round(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isnan(v)) return (uint16_t)(sign | 0x7FC0u);
  double a = fabs(v);
  if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
  if (a < ldexp(1.0, -126)) {
    /* subnormal range: integer multiple of 2^-133 (128 -> smallest normal) */
    double q = nearbyint(ldexp(a, 133)); /* default mode: ties to even */
    return (uint16_t)(sign | (uint16_t)q);
  }
  int e;
  frexp(a, &e); /* a = f * 2^e, 0.5 <= f < 1 */
  double q = nearbyint(ldexp(a, 8 - e)); /* 8-bit significand in [128, 256] */
  if (q == 256.0) {
    q = 128.0;
    e += 1;
  }
  int biased = e - 1 + 127; /* a = (q / 128) * 2^(e - 1) */
  if (biased >= 255) return (uint16_t)(sign | 0x7F80u); /* overflow -> inf */
  return (uint16_t)(sign | (uint16_t)(biased << 7) | (uint16_t)((int)q - 128));
}

/* ------------------------------------------------------------- the GEMM */

/* y[m, n] = bf16( sum_k x[m, k] * W[n, k] ), k ascending, binary64 sum.
 * [unpooler] module description.  x is [M, K], W is [N, K], y is [M, N], all
 * row-major bfloat16 bit patterns.  threads > 1 runs output columns on that
 * many OpenMP threads; each element's sum is the same either way. */
void oracle_gemm_bf16(const uint16_t *x, const uint16_t *w, uint16_t *y,
                      int M, int N, int K, int threads) {
  if (threads < 1) threads = 1;
#pragma omp parallel for num_threads(threads) schedule(static)
  for (int n = 0; n < N; ++n) {
    for (int m = 0; m < M; ++m) {
      double acc = 0.0;
      for (int k = 0; k < K; ++k)
        acc += oracle_bf16_value(x[(size_t)m * K + k]) *
               oracle_bf16_value(w[(size_t)n * K + k]);
      y[(size_t)m * N + n] = oracle_bf16_round(acc);
    }
  }
}

/* The same sum for a list of (m, n) positions only: count entries of
 * rows[i], cols[i] -> out[i] (bfloat16 bits) and exact[i] (the binary64 sum
 * before rounding; may be NULL).  Used to check full-size outputs at sampled
 * positions. */
void oracle_gemm_bf16_sampled(const uint16_t *x, const uint16_t *w, int K,
                              const int *rows, const int *cols, int count,
                              uint16_t *out, double *exact) {
  for (int i = 0; i < count; ++i) {
    double acc = 0.0;
    for (int k = 0; k < K; ++k)
      acc += oracle_bf16_value(x[(size_t)rows[i] * K + k]) *
             oracle_bf16_value(w[(size_t)cols[i] * K + k]);
    out[i] = oracle_bf16_round(acc);
    if (exact) exact[i] = acc;
  }
}

/* -------------------------------------------------------- e4m3fn and e2m1 */

/* OCP float8 e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; 0x7F and 0xFF are NaN; largest finite magnitude 448. */
double oracle_e4m3_value(uint8_t code) {
  int sign = code >> 7, exp = (code >> 3) & 15, man = code & 7;
  double mag;
  if (exp == 15 && man == 7) return NAN;
  if (exp == 0)
    mag = ldexp((double)man, -9); /* subnormal: man/8 * 2^(1-7) */
  else
    mag = ldexp(1.0 + man / 8.0, exp - 7);
  return sign ? -mag : mag;
}

/* e2m1: 1 sign, 2 exponent (bias 1), 1 mantissa bit.  Magnitudes by code
 * index 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_value(uint8_t code) {
  int sign = (code >> 3) & 1, exp = (code >> 1) & 3, man = code & 1;
  double mag = exp == 0 ? 0.5 * man : ldexp(1.0 + 0.5 * man, exp - 1);
  return sign ? -mag : mag;
}

/* Round to the nearest finite code; on a tie take the code whose last
 * (mantissa) bit is 0.  Magnitudes above the largest finite value therefore
 * land on it: round-to-nearest-even with saturation ([cvt]).  Written as a
 * search over every non-negative finite code, so it is the definition. */
static uint8_t nearest_code(double a, double (*value)(uint8_t), int ncodes) {
  /* at or above the largest finite value that value is the nearest; testing
   * it first also keeps the distances below exact (both candidates around a
   * are within a factor of two of it, so a - value is exact) */
  if (isinf(a) || a >= value((uint8_t)(ncodes - 1))) return (uint8_t)(ncodes - 1);
  int best = 0;
  double best_d = fabs(a - value(0));
  for (int c = 1; c < ncodes; ++c) {
    double d = fabs(a - value((uint8_t)c));
    if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)best;
}

/* binary64 -> e4m3fn, nearest-even, saturating.  NaN -> 0x7F. */
uint8_t oracle_e4m3_encode(double v) {
  if (isnan(v)) return 0x7F;
  uint8_t mag = nearest_code(fabs(v), oracle_e4m3_value, 0x7F); /* 0x00..0x7E */
  return (uint8_t)(signbit(v) ? 0x80 | mag : mag);
}

/* binary64 -> e2m1 (4-bit code), nearest-even, saturating; the sign bit is
 * kept for values that round to zero.  NaN -> 0 (never produced here). */
uint8_t oracle_e2m1_encode(double v) {
  if (isnan(v)) return 0;
  uint8_t mag = nearest_code(fabs(v), oracle_e2m1_value, 8);
  return (uint8_t)(signbit(v) ? 0x8 | mag : mag);
}

/* ----------------------------------------------------- norm and NVFP4 */

/* One 16-element NVFP4 block of normed values yn (binary64 values of
 * bfloat16 numbers).  global_scale is the FP32 input global scale.  When
 * forced_sf >= 0 that scale byte is used instead of the computed one (so a
 * block can be re-quantized with another scale).  Outputs: codes[16] (4-bit),
 * *sf_out (e4m3fn byte), pre[16] = yn * output scale before rounding (may be
 * NULL), *os_out = the output scale (may be NULL). */
void oracle_nvfp4_block(const double *yn, double global_scale, int forced_sf,
                        uint8_t *codes, uint8_t *sf_out, double *pre,
                        double *os_out) {
  double amax = 0.0;
  for (int j = 0; j < 16; ++j)
    if (fabs(yn[j]) > amax) amax = fabs(yn[j]);
  uint8_t sf = forced_sf >= 0 ? (uint8_t)forced_sf
                              : oracle_e4m3_encode(global_scale * amax / 6.0);
  double dec = oracle_e4m3_value(sf);
  double os = dec == 0.0 ? 0.0 : global_scale / dec; /* [oscale] */
  for (int j = 0; j < 16; ++j) {
    double v = yn[j] * os;
    codes[j] = oracle_e2m1_encode(v);
    if (pre) pre[j] = v;
  }
  *sf_out = sf;
  if (os_out) *os_out = os;
}

/* RMSNorm with gain center, one bfloat16 rounding ([pooler]):
 *   yn[m, j] = bf16( r[m, j] / sqrt(mean_j r^2 + eps) * (w[j] + gain_center) )
 * r is [M, P] bfloat16 bits, w is [P] bfloat16 bits, yn is [M, P] bits. */
void oracle_rmsnorm_bf16(const uint16_t *r, const uint16_t *w,
                         double gain_center, double eps, int M, int P,
                         uint16_t *yn) {
  for (int m = 0; m < M; ++m) {
    const uint16_t *row = r + (size_t)m * P;
    double ss = 0.0;
    for (int j = 0; j < P; ++j) {
      double v = oracle_bf16_value(row[j]);
      ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / P + eps);
    for (int j = 0; j < P; ++j)
      yn[(size_t)m * P + j] = oracle_bf16_round(
          oracle_bf16_value(row[j]) * inv *
          (oracle_bf16_value(w[j]) + gain_center));
  }
}

/* The NVFP4 expert input ([pooler]): the norm above, then per 16-column block
 * the e4m3fn scale and the e2m1 codes, packed two per byte with the even
 * column in the low nibble.
 *   a    [M, P/2]  uint8
 *   a_sf [M, P/16] uint8 (e4m3fn bytes), row-major, not swizzled
 *   yn   [M, P]    bfloat16 bits of the normed row (may be NULL)
 *   pre  [M, P]    yn * output scale before e2m1 rounding (may be NULL)
 *   osc  [M, P/16] the output scale per block (may be NULL) */
void oracle_rmsnorm_nvfp4(const uint16_t *r, const uint16_t *w,
                          double gain_center, double eps, double global_scale,
                          int M, int P, uint8_t *a, uint8_t *a_sf,
                          uint16_t *yn_out, double *pre, double *osc) {
  for (int m = 0; m < M; ++m) {
    const uint16_t *row = r + (size_t)m * P;
    double ss = 0.0;
    for (int j = 0; j < P; ++j) {
      double v = oracle_bf16_value(row[j]);
      ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / P + eps);
    for (int b = 0; b < P / 16; ++b) {
      double yn[16];
      uint8_t codes[16], sf;
      double os;
      for (int j = 0; j < 16; ++j) {
        int col = b * 16 + j;
        uint16_t bits = oracle_bf16_round(oracle_bf16_value(row[col]) * inv *
                                          (oracle_bf16_value(w[col]) + gain_center));
        yn[j] = oracle_bf16_value(bits);
        if (yn_out) yn_out[(size_t)m * P + col] = bits;
      }
      oracle_nvfp4_block(yn, global_scale, -1, codes, &sf,
                         pre ? pre + (size_t)m * P + b * 16 : NULL, &os);
      for (int i = 0; i < 8; ++i)
        a[(size_t)m * (P / 2) + b * 8 + i] =
            (uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));
      a_sf[(size_t)m * (P / 16) + b] = sf;
      if (osc) osc[(size_t)m * (P / 16) + b] = os;
    }
  }
}

/* ----------------------------------------------------------------- publish */

/* [publish] The zero-copy epilogue on one GPU: rows 0..M-1 of y [M, width]
 * into this rank's slot of the mailbox [3][tp][capacity][width] at the
 * stage, with -0.0 (the sentinel) stored as +0.0; without a ticket the stage
 * word stage_state[1] is set to the stage, with one (ticket != NULL) the
 * stage state is not used.  Returns the stage, or -1 (and writes nothing) if
 * it is outside 0..2. */
int oracle_mailbox_publish(const uint16_t *y, int M, int width, uint16_t *mailbox, int tp,
                           int rank, int capacity, int32_t *stage_state,
                           const int32_t *ticket) {
  int stage = ticket ? (int)((uint32_t)ticket[0] >> 16) : stage_state[0];
  if (stage < 0 || stage > 2) return -1;
  uint16_t *slot = mailbox + ((size_t)stage * tp + rank) * (size_t)capacity * width;
  for (int t = 0; t < M; ++t)
    for (int j = 0; j < width; ++j) {
      uint16_t v = y[(size_t)t * width + j];
      slot[(size_t)t * width + j] = (v == 0x8000u) ? 0x0000u : v;
    }
  if (!ticket) stage_state[1] = stage;
  return stage;
}

/* -------------------------------------------------------------- dual norm */

/* [dual] For each row m of partial [M, H] (bf16) and stream [M, H] (binary32,
 * updated in place):
 *   h_j      = bf16(p_j / sqrt(mean(p^2) + post_eps) * g_j),
 *              g_j = post_w_j + post_gc, or 1 without a post weight
 *   stream_j = f32(a_j * stream_j + beta_j * h_j),  a_j = alpha_j or alpha_scalar
 *   out_j    = bf16(s_j / sqrt(mean(s^2) + pre_eps) * (next_w_j + pre_gc)),
 *              s = the updated stream row
 * h_out (optional) receives h.  Weights, alpha and beta are bf16 [H]. */
void oracle_dual_norm(const uint16_t *partial, float *stream, const uint16_t *post_w,
                      double post_gc, double post_eps, const uint16_t *alpha,
                      double alpha_scalar, const uint16_t *beta, const uint16_t *next_w,
                      double pre_gc, double pre_eps, int M, int H, uint16_t *out,
                      uint16_t *h_out) {
  for (int m = 0; m < M; ++m) {
    const uint16_t *p = partial + (size_t)m * H;
    float *st = stream + (size_t)m * H;
    double ss = 0.0;
    for (int j = 0; j < H; ++j) {
      double v = oracle_bf16_value(p[j]);
      ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / H + post_eps);
    for (int j = 0; j < H; ++j) {
      double g = post_w ? oracle_bf16_value(post_w[j]) + post_gc : 1.0;
      uint16_t h = oracle_bf16_round(oracle_bf16_value(p[j]) * inv * g);
      if (h_out) h_out[(size_t)m * H + j] = h;
      double a = alpha ? oracle_bf16_value(alpha[j]) : alpha_scalar;
      double v = a * (double)st[j] + oracle_bf16_value(beta[j]) * oracle_bf16_value(h);
      st[j] = (float)v;
    }
    double ss2 = 0.0;
    for (int j = 0; j < H; ++j) ss2 += (double)st[j] * (double)st[j];
    double inv2 = 1.0 / sqrt(ss2 / H + pre_eps);
    for (int j = 0; j < H; ++j)
      out[(size_t)m * H + j] = oracle_bf16_round(
          (double)st[j] * inv2 * (oracle_bf16_value(next_w[j]) + pre_gc));
  }
}
