/*
 * oracle.c -- plain fp64 reference of the layer-boundary completion path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the bench's
 * CPU-baseline leg may load this library. The product path never calls it,
 * and it shares no code, header or table with the HIP library.
 *
 * Sources (the SGLang developer guide "Layer boundaries", and the study note
 * "SGLang flashinfer_allreduce_fusion精读"):
 *   - Layer boundaries, section "Residual stream", state table: a stream is
 *     Initial (no residual, no contribution), Written (a residual, nothing
 *     pending) or Pending (a contribution, with or without a residual). The
 *     next read initialises the residual (Initial), reads it unchanged
 *     (Written), or completes the owed work, applies the producer's update
 *     and then reads (Pending).
 *   - Same section, helper table: completing a contribution is a step of its
 *     own, distinct from folding it into the residual.
 *   - Section "Residual update and input read": the plain update is an add,
 *     and the fused add+norm read normalises the FP32 sum rather than a
 *     separately rounded copy of it.
 *   - Section "Producer contracts and output state" and section "Enter and
 *     leave the layer stack": a deferred MoE finalize is owed work whose
 *     completion is the weighted combination of the expert rows of each
 *     token.
 *   - Study note, forward section (fusion diagram): the fused kernel does
 *     all-reduce, residual add and RMSNorm; the fallback is the all-reduce
 *     followed by the add+norm. The reduce-scatter variant normalises only
 *     the rank's own row slice.
 *
 * Everything here is evaluated in double precision, one row at a time, in the
 * order the pages give: complete the contribution, apply the update, read.
 * Inputs (bf16 bit patterns, fp32 weights/gates) are exact in double, so the
 * contribution sums are exact; only the square root, the division and the
 * products round, at double precision. Stored outputs are rounded once, from
 * the double value, to nearest-even.
 *
 * The RMSNorm read: y_h = x_h * w_h / sqrt(mean_h(x_h^2) + eps), with eps
 * (an fp32 value) inside the square root. The pages name RMSNorm without
 * printing its formula; this is the standard definition. The guide's
 * terminal finalize (section "Enter and leave the layer stack") reads a
 * GemmaRMSNorm weight instead; the page does not define it, and the reading
 * taken here is the Gemma convention of a weight stored as an offset from
 * one: y_h = x_h * (1 + w_h) / sqrt(mean_h(x_h^2) + eps). `gemma` selects it.
 *
 * Quantised read (fp8): per row, scale = max_h |y_h| / 448 and
 * q_h = e4m3(y_h / scale), OCP E4M3FN ("OFP8 Formats for Deep Learning",
 * OCP 8-bit floating point specification, 2023): bias 7, three mantissa
 * bits, largest finite 448, no infinities. A row with max |y| = 0 has scale 0
 * and all codes +0. The pages say only that the consumer input may be
 * quantised; this per-token reading is stated in the design notes. They fix
 * no precision for it, so the steps that decide a code run in the device's
 * precision, fp32: y is rounded to fp32, the scale is one fp32 division of
 * the largest |y| by 448, and each code is the e4m3 rounding of the fp32
 * quotient y / scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* bf16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits              */
/* ------------------------------------------------------------------------ */

double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Round a finite double to the nearest bf16 value, ties to even mantissa. */
uint16_t orc_bf16_round(double v) {
  double a = fabs(v);
  double r = 0.0;
  if (a != 0.0) {
    int ex;
    frexp(a, &ex);              /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;             /* a in [2^e, 2^(e+1)) */
    if (e < -126) e = -126;     /* subnormal range shares the 2^-133 step */
    double step = ldexp(1.0, e - 7);
    double n = a / step;        /* exact: division by a power of two */
    double n_r = floor(n);
    double frac = n - n_r;
    if (frac > 0.5 || (frac == 0.5 && fmod(n_r, 2.0) != 0.0)) n_r += 1.0;
    r = n_r * step;
  }
  float f = (float)r;           /* exact: r is a bf16 value */
  if (signbit(v)) f = -f;
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------ */
/* OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa; 0x7F/0xFF are NaN   */
/* ------------------------------------------------------------------------ */

double orc_e4m3_value(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);                /* subnormal: m * 2^-6 / 8 */
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/*
 * Round a double with |v| <= 448 to the nearest E4M3FN value, ties to even
 * code (even mantissa). The value is rounded on the format's grid, then the
 * code is found by searching the 127 non-negative finite codes.
 */
uint8_t orc_e4m3_round(double v) {
  double a = fabs(v);
  double r = 0.0;
  if (a != 0.0) {
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    if (e < -6) e = -6;                      /* below the smallest normal 2^-6 */
    double step = ldexp(1.0, e - 3);
    double n = a / step;
    double n_r = floor(n);
    double frac = n - n_r;
    if (frac > 0.5 || (frac == 0.5 && fmod(n_r, 2.0) != 0.0)) n_r += 1.0;
    r = n_r * step;
  }
  uint8_t code = 0;
  for (int c = 0; c < 0x7F; ++c) {
    if (orc_e4m3_value((uint8_t)c) == r) {
      code = (uint8_t)c;
      break;
    }
  }
  if (signbit(v)) code |= 0x80;
  return code;
}

/* ------------------------------------------------------------------------ */
/* The steps of one boundary, for one token row                             */
/* ------------------------------------------------------------------------ */

/* Complete owed work, plain TP partials: s_h = sum_p c_p[t, h]. */
static void complete_partials_row(int64_t H, int P, const uint16_t* const* partials, int64_t ld,
                                  int64_t t, double* s, double* mag) {
  for (int64_t h = 0; h < H; ++h) {
    s[h] = 0.0;
    mag[h] = 0.0;
  }
  for (int p = 0; p < P; ++p) {
    const uint16_t* row = partials[p] + t * ld;
    for (int64_t h = 0; h < H; ++h) {
      double c = orc_bf16_value(row[h]);
      s[h] += c;
      mag[h] += fabs(c);
    }
  }
}

/*
 * Complete owed work, deferred MoE finalize: token t's contribution is the
 * gate-weighted sum of its k expert-output rows,
 *   s_h = sum_j gate[t, j] * E[idx[t, j], h].
 * idx is in gather form: the row of E that holds pick j of token t. A row
 * index outside [0, n_rows) contributes nothing.
 */
static void complete_moe_row(int64_t H, int k, const uint16_t* E, int64_t ld_e, int64_t n_rows,
                             const int32_t* idx, const float* gate, int64_t t, double* s,
                             double* mag) {
  for (int64_t h = 0; h < H; ++h) {
    s[h] = 0.0;
    mag[h] = 0.0;
  }
  for (int j = 0; j < k; ++j) {
    int64_t e = idx[t * k + j];
    if (e < 0 || e >= n_rows) continue;
    double g = (double)gate[t * k + j];
    const uint16_t* row = E + e * ld_e;
    for (int64_t h = 0; h < H; ++h) {
      double c = g * orc_bf16_value(row[h]);
      s[h] += c;
      mag[h] += fabs(c);
    }
  }
}

/* Apply the producer's plain update: x = r + s; no residual means r = 0. */
static void apply_update_row(int64_t H, const uint16_t* r, const double* s, double* x,
                             double* mag) {
  for (int64_t h = 0; h < H; ++h) {
    double rv = r ? orc_bf16_value(r[h]) : 0.0;
    x[h] = rv + s[h];
    mag[h] += fabs(rv);
  }
}

/* RMSNorm scale of a row: 1 / sqrt(mean_h(x_h^2) + eps). */
static double rms_inverse(int64_t H, const double* x, float eps) {
  double sum_sq = 0.0;
  for (int64_t h = 0; h < H; ++h) sum_sq += x[h] * x[h];
  return 1.0 / sqrt(sum_sq / (double)H + (double)eps);
}

/* The read: y_h = x_h * inv * w_h, or x_h * inv * (1 + w_h) for a Gemma weight. */
static void normalise_row(int64_t H, const double* x, double inv, const float* w, int gemma,
                          double* y) {
  for (int64_t h = 0; h < H; ++h) {
    double scale = gemma ? 1.0 + (double)w[h] : (double)w[h];
    y[h] = x[h] * inv * scale;
  }
}

static void store_bf16_row(int64_t H, const double* v, uint16_t* out) {
  for (int64_t h = 0; h < H; ++h) out[h] = orc_bf16_round(v[h]);
}

/* Per-token fp8, decided in fp32: y32 = fp32(y), scale = fp32(max |y32| / 448),
 * q = e4m3(clamp(fp32(y32 / scale))). */
static float store_fp8_row(int64_t H, const double* y, uint8_t* q) {
  float amax = 0.0f;
  for (int64_t h = 0; h < H; ++h) {
    const float a = fabsf((float)y[h]);
    if (a > amax) amax = a;
  }
  const float scale = amax / 448.0f;
  for (int64_t h = 0; h < H; ++h) {
    if (scale == 0.0f) {
      q[h] = 0x00;
      continue;
    }
    float v = (float)y[h] / scale;
    if (v > 448.0f) v = 448.0f;
    if (v < -448.0f) v = -448.0f;
    q[h] = orc_e4m3_round((double)v);
  }
  return scale;
}

static void copy_out(int64_t H, const double* v, double* dst) {
  if (dst) memcpy(dst, v, sizeof(double) * (size_t)H);
}

/* ------------------------------------------------------------------------ */
/* Exported operations. Row tensors are row-major with a leading dimension  */
/* in elements. Reduced inputs (partials, expert index, gates) are indexed  */
/* by global token row row_begin + i; residual and outputs by slice row i.  */
/* The optional double arrays x_exact / y_exact / mag are [rows, H] dense:  */
/* mag is the magnitude sum |r| + sum |terms| used to bound fp32 error.     */
/* ------------------------------------------------------------------------ */

typedef struct {
  double *s, *x, *y, *mag;
} scratch_t;

static int scratch_alloc(scratch_t* w, int64_t H) {
  w->s = (double*)malloc(sizeof(double) * (size_t)H);
  w->x = (double*)malloc(sizeof(double) * (size_t)H);
  w->y = (double*)malloc(sizeof(double) * (size_t)H);
  w->mag = (double*)malloc(sizeof(double) * (size_t)H);
  return (w->s && w->x && w->y && w->mag) ? 0 : -1;
}

static void scratch_free(scratch_t* w) {
  free(w->s);
  free(w->x);
  free(w->y);
  free(w->mag);
}

/* Read from the Initial state: the residual is initialised from the stack
 * input x_in, and y = norm(x_in). */
int orc_enter_norm(int64_t rows, int64_t H, const uint16_t* x_in, int64_t ld_x, const float* w,
                   float eps, int gemma, uint16_t* res_out, int64_t ld_ro, uint16_t* y_out,
                   int64_t ld_y, double* y_exact) {
  scratch_t b;
  if (scratch_alloc(&b, H)) return -1;
  for (int64_t i = 0; i < rows; ++i) {
    for (int64_t h = 0; h < H; ++h) b.x[h] = orc_bf16_value(x_in[i * ld_x + h]);
    double inv = rms_inverse(H, b.x, eps);
    normalise_row(H, b.x, inv, w, gemma, b.y);
    if (res_out) memcpy(res_out + i * ld_ro, x_in + i * ld_x, sizeof(uint16_t) * (size_t)H);
    store_bf16_row(H, b.y, y_out + i * ld_y);
    copy_out(H, b.y, y_exact ? y_exact + i * H : NULL);
  }
  scratch_free(&b);
  return 0;
}

/* Read from the Written state: y = norm(residual), no update. */
int orc_written_norm(int64_t rows, int64_t H, const uint16_t* res, int64_t ld_r, const float* w,
                     float eps, int gemma, uint16_t* y_out, int64_t ld_y, double* y_exact) {
  return orc_enter_norm(rows, H, res, ld_r, w, eps, gemma, NULL, 0, y_out, ld_y, y_exact);
}

/* Read from the Pending state with P plain partials: complete, fold, norm.
 * residual may be NULL (a Pending stream without a residual): then x = s.
 * Exactly one of y_out (bf16 read) or q_out/scale_out (fp8 read) is used. */
int orc_fold_norm(int64_t rows, int64_t H, int64_t row_begin, int P,
                  const uint16_t* const* partials, int64_t ld_p, const uint16_t* residual,
                  int64_t ld_r, const float* w, float eps, int gemma, uint16_t* res_out,
                  int64_t ld_ro, uint16_t* y_out, int64_t ld_y, uint8_t* q_out, int64_t ld_q,
                  float* scale_out, double* x_exact, double* y_exact, double* mag) {
  scratch_t b;
  if (scratch_alloc(&b, H)) return -1;
  for (int64_t i = 0; i < rows; ++i) {
    complete_partials_row(H, P, partials, ld_p, row_begin + i, b.s, b.mag);
    apply_update_row(H, residual ? residual + i * ld_r : NULL, b.s, b.x, b.mag);
    double inv = rms_inverse(H, b.x, eps);
    normalise_row(H, b.x, inv, w, gemma, b.y);
    store_bf16_row(H, b.x, res_out + i * ld_ro);
    if (y_out) store_bf16_row(H, b.y, y_out + i * ld_y);
    if (q_out) scale_out[i] = store_fp8_row(H, b.y, q_out + i * ld_q);
    copy_out(H, b.x, x_exact ? x_exact + i * H : NULL);
    copy_out(H, b.y, y_exact ? y_exact + i * H : NULL);
    copy_out(H, b.mag, mag ? mag + i * H : NULL);
  }
  scratch_free(&b);
  return 0;
}

/* Read from the Pending state with a deferred MoE finalize: the weighted
 * gather-sum is completed and folded in one pass, then normalised. */
int orc_moe_fold_norm(int64_t rows, int64_t H, int64_t row_begin, int k, const uint16_t* E,
                      int64_t ld_e, int64_t n_rows_e, const int32_t* idx, const float* gate,
                      const uint16_t* residual, int64_t ld_r, const float* w, float eps,
                      int gemma, uint16_t* res_out, int64_t ld_ro, uint16_t* y_out, int64_t ld_y,
                      uint8_t* q_out, int64_t ld_q, float* scale_out, double* x_exact,
                      double* y_exact, double* mag) {
  scratch_t b;
  if (scratch_alloc(&b, H)) return -1;
  for (int64_t i = 0; i < rows; ++i) {
    complete_moe_row(H, k, E, ld_e, n_rows_e, idx, gate, row_begin + i, b.s, b.mag);
    apply_update_row(H, residual ? residual + i * ld_r : NULL, b.s, b.x, b.mag);
    double inv = rms_inverse(H, b.x, eps);
    normalise_row(H, b.x, inv, w, gemma, b.y);
    store_bf16_row(H, b.x, res_out + i * ld_ro);
    if (y_out) store_bf16_row(H, b.y, y_out + i * ld_y);
    if (q_out) scale_out[i] = store_fp8_row(H, b.y, q_out + i * ld_q);
    copy_out(H, b.x, x_exact ? x_exact + i * H : NULL);
    copy_out(H, b.y, y_exact ? y_exact + i * H : NULL);
    copy_out(H, b.mag, mag ? mag + i * H : NULL);
  }
  scratch_free(&b);
  return 0;
}

/* complete_output: finish the owed sum only, leaving the update pending.
 * The completed contribution is stored as bf16 (the only rounded
 * intermediate of the path, by the definition of this call).
 * add_to_output (guide, section "Auxiliary capture and extra
 * contributions"): the contribution is completed first and then the extra
 * tensor is added exactly once; `extra` (nullable, [T, H] bf16, global rows)
 * selects it. */
static void add_extra_row(int64_t H, const uint16_t* extra, double* s, double* mag) {
  for (int64_t h = 0; h < H; ++h) {
    double e = orc_bf16_value(extra[h]);
    s[h] += e;
    mag[h] += fabs(e);
  }
}

int orc_complete_partials(int64_t rows, int64_t H, int64_t row_begin, int P,
                          const uint16_t* const* partials, int64_t ld_p, const uint16_t* extra,
                          int64_t ld_x, uint16_t* out, int64_t ld_o, double* s_exact,
                          double* mag) {
  scratch_t b;
  if (scratch_alloc(&b, H)) return -1;
  for (int64_t i = 0; i < rows; ++i) {
    complete_partials_row(H, P, partials, ld_p, row_begin + i, b.s, b.mag);
    if (extra) add_extra_row(H, extra + (row_begin + i) * ld_x, b.s, b.mag);
    store_bf16_row(H, b.s, out + i * ld_o);
    copy_out(H, b.s, s_exact ? s_exact + i * H : NULL);
    copy_out(H, b.mag, mag ? mag + i * H : NULL);
  }
  scratch_free(&b);
  return 0;
}

int orc_complete_moe(int64_t rows, int64_t H, int64_t row_begin, int k, const uint16_t* E,
                     int64_t ld_e, int64_t n_rows_e, const int32_t* idx, const float* gate,
                     const uint16_t* extra, int64_t ld_x, uint16_t* out, int64_t ld_o,
                     double* s_exact, double* mag) {
  scratch_t b;
  if (scratch_alloc(&b, H)) return -1;
  for (int64_t i = 0; i < rows; ++i) {
    complete_moe_row(H, k, E, ld_e, n_rows_e, idx, gate, row_begin + i, b.s, b.mag);
    if (extra) add_extra_row(H, extra + (row_begin + i) * ld_x, b.s, b.mag);
    store_bf16_row(H, b.s, out + i * ld_o);
    copy_out(H, b.s, s_exact ? s_exact + i * H : NULL);
    copy_out(H, b.mag, mag ? mag + i * H : NULL);
  }
  scratch_free(&b);
  return 0;
}

/* snapshot (guide, section "Auxiliary capture and extra contributions"): a
 * plain bf16 copy of the residual the pending update would produce,
 * bf16(r + s), computed on the side; the residual and the owed work are left
 * as they are. P = 0 (nothing owed) copies the residual. */
int orc_snapshot(int64_t rows, int64_t H, int64_t row_begin, int P,
                 const uint16_t* const* partials, int64_t ld_p, const uint16_t* residual,
                 int64_t ld_r, uint16_t* out, int64_t ld_o, double* x_exact, double* mag) {
  scratch_t b;
  if (scratch_alloc(&b, H)) return -1;
  for (int64_t i = 0; i < rows; ++i) {
    complete_partials_row(H, P, partials, ld_p, row_begin + i, b.s, b.mag);
    apply_update_row(H, residual ? residual + i * ld_r : NULL, b.s, b.x, b.mag);
    store_bf16_row(H, b.x, out + i * ld_o);
    copy_out(H, b.x, x_exact ? x_exact + i * H : NULL);
    copy_out(H, b.mag, mag ? mag + i * H : NULL);
  }
  scratch_free(&b);
  return 0;
}
