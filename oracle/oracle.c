/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the fused
 * residual + gate + LayerNorm/RMSNorm + scale/shift row operation.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the product path.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes, and where that comes from:
 *   - The two operations and their operand order are those of the custom ops
 *     flydsl_fused_residual_norm_scale_shift(residual, x, gate, weight, bias,
 *     scale, shift, norm_type, eps) and flydsl_norm_scale_shift(x, weight,
 *     bias, scale, shift, norm_type, eps) in the reproduction snippet of the
 *     "Microbenchmark" section of sglang PR #36349 ("[AMD][Diffusion] Migrate
 *     FlyDSL fused norm kernels to the v0.3.0 stable API").  The pages never
 *     print the formula; the reading used here is: the gate scales the branch
 *     output x, the residual stream is updated first, the updated stream is
 *     normalised, then the optional affine weight/bias, then the modulation
 *     n * (1 + scale) + shift.
 *   - LayerNorm without affine parameters ("elementwise_affine=False") for the
 *     WAN2.2 norm1/norm_out calls: same page, "Result" / "Microbenchmark".
 *   - eps = 1e-6, the value the kernels use: sglang PR #33144, "Modifications".
 *     Here eps is an argument and honoured (every workload passes 1e-6).
 *   - Broadcast operands are a dense (1, C) row that every activation row
 *     reads; per-row scale/shift; a 4D per-frame (B, F, 1, C) layout: sglang
 *     PR #33144, "Modifications" and "Accuracy Tests".
 *   - Frames are frame-major token blocks (49 latent frames x 3600 tokens =
 *     sequence 176400): sglang PR #36349, "Microbenchmark".
 *
 * Precision: the residual update is the exact residual + gate * x rounded
 * once to binary32 (a fused multiply-add), then once to bf16.  The product of
 * two bf16 values is exact in binary32 down to the normal range; below it a
 * separately rounded product could round twice, or lose the sign of a
 * product that underflows to zero, so the single rounding is written out
 * with fmaf.  Everything after it is binary64, with a two-pass
 * (mean, then centred squares) variance with the biased 1/D estimator, and a
 * single correctly rounded conversion of the binary64 result to the output
 * type (bf16 by default; binary32; or FP8 E4M3 with a per-row scale).
 *
 * Extensions beyond the pages' ops (each the plainest reading): binary32
 * weight/bias (the pages pass fp32 affine parameters that the prior-art
 * kernel casts to bf16 -- sglang PR #36349 "Microbenchmark" snippet; sglang PR
 * #33144 "Known gaps"), a binary32 output (the pages note the two ops handle
 * their output dtype differently -- same "Known gaps"), and an FP8 E4M3 output
 * with a per-row scale for an FP8 consumer (the pages run WAN2.2 with FP8
 * attention enabled -- sglang PR #36349 "Command").
 *
 * Build: plain C11, -ffp-contract=off, no fast-math, no flush-to-zero.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- bf16 conversions ------------------------------------------------- */

/* A bf16 value is the high half of a binary32 value; widening is exact. */
static float bf16_to_f32(uint16_t h) {
  uint32_t bits = (uint32_t)h << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

double orc_bf16_to_f64(uint16_t h) { return (double)bf16_to_f32(h); }

/*
 * Correct rounding of a binary64 value to bf16 (8 significand bits, exponent
 * range of binary32).  The value is split as |t| = m * q where q is the bf16
 * quantum (unit in the last place) of the binade of |t| -- 2^(e-7) for
 * 2^e <= |t| < 2^(e+1), and the fixed subnormal quantum 2^-133 below 2^-126.
 * |t| / q is exact (q is a power of two), rint() rounds it to the nearest
 * integer with ties to even (the default rounding mode), and the product
 * with q is exact again.  A result of 2^128 or more is an overflow to Inf.
 */
uint16_t orc_f64_to_bf16(double t) {
  if (isnan(t)) return 0x7FC0;
  uint16_t sign = signbit(t) ? 0x8000 : 0x0000;
  double a = fabs(t);
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  if (a == 0.0) return sign;
  int e2;
  (void)frexp(a, &e2);          /* a = f * 2^e2 with 0.5 <= f < 1 */
  int e = e2 - 1;               /* 2^e <= a < 2^(e+1) */
  if (e < -126) e = -126;       /* subnormal bf16: fixed quantum */
  double q = ldexp(1.0, e - 7);
  double r = rint(a / q) * q;
  if (r >= 0x1.0p128) return (uint16_t)(sign | 0x7F80);
  float f = (float)r;           /* exact: r has at most 8 significant bits */
  uint32_t bits;
  memcpy(&bits, &f, sizeof bits);
  return (uint16_t)(sign | (uint16_t)(bits >> 16));
}

/*
 * Correct rounding of a binary64 value to OCP FP8 E4M3 ("e4m3fn": 4 exponent
 * bits with bias 7, 3 mantissa bits, no infinities, NaN = S.1111.111, largest
 * finite 1.75 * 2^8 = 448, subnormals m * 2^-9), saturating: a value whose
 * rounded magnitude would exceed 448 (|t| >= 464) becomes +-448.  NaN -> 0x7F.
 * Same split as the bf16 routine: quantum 2^(e-3) in the binade of |t|, fixed
 * 2^-9 below 2^-6, rint() to the nearest integer with ties to even.
 */
uint8_t orc_f64_to_e4m3(double t) {
  if (isnan(t)) return 0x7F;
  uint8_t sign = signbit(t) ? 0x80 : 0x00;
  double a = fabs(t);
  if (a == 0.0) return sign;
  int e2;
  (void)frexp(a, &e2);
  int e = e2 - 1;               /* 2^e <= a < 2^(e+1) (or +inf) */
  if (e < -6) e = -6;           /* subnormal: fixed quantum 2^-9 */
  if (e > 8) e = 8;             /* beyond the top binade: saturates below */
  double q = ldexp(1.0, e - 3);
  double r = isinf(a) ? 512.0 : rint(a / q) * q;
  if (r > 448.0) r = 448.0;     /* saturate */
  uint8_t code;
  if (r < 0x1.0p-6) {
    code = (uint8_t)(r / 0x1.0p-9);                 /* subnormal (or zero) */
  } else {
    int er;
    double m = frexp(r, &er);                       /* r = m * 2^er, 0.5 <= m < 1 */
    int exp_field = (er - 1) + 7;
    int mant = (int)((m * 2.0 - 1.0) * 8.0);        /* exact: r has 4 significant bits */
    code = (uint8_t)((exp_field << 3) | mant);
  }
  return (uint8_t)(sign | code);
}

void orc_f64_to_e4m3_array(const double* in, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_e4m3(in[i]);
}

void orc_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16((double)in[i]);
}

void orc_f64_to_bf16_array(const double* in, uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16(in[i]);
}

/* ---- the residual update ---------------------------------------------- */

/* residual + gate * x: the exact value rounded once to binary32 (fmaf, or
 * the plain sum without a gate), then once to bf16. */
static uint16_t residual_update(uint16_t res, const uint16_t* gate_or_null, uint16_t x) {
  float r = bf16_to_f32(res);
  float xv = bf16_to_f32(x);
  float s = gate_or_null ? fmaf(bf16_to_f32(*gate_or_null), xv, r) : r + xv;
  return orc_f64_to_bf16((double)s);
}

void orc_residual_array(const uint16_t* res, const uint16_t* gate, const uint16_t* x,
                        uint16_t* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = residual_update(res[i], gate ? &gate[i] : NULL, x[i]);
}

/* ---- modulation layouts ----------------------------------------------- */

/*
 * Activation row r = b*L + l (batch b, token l).  BCAST: the one (1, C) row.
 * ROW: row r of a (B, L, C) tensor.  FRAME: row b*F + f of a (B, F, 1, C)
 * tensor, where token l lies in frame f = l / (L / F).
 */
int64_t orc_mod_row(int kind, int64_t frames, int64_t r, int64_t L) {
  int64_t b = r / L;
  int64_t l = r % L;
  switch (kind) {
    case ORC_BCAST: return 0;
    case ORC_ROW: return r;
    case ORC_FRAME: return b * frames + l / (L / frames);
    default: return -1;
  }
}

static int layout_ok(int kind, int64_t frames, int64_t L) {
  if (kind == ORC_BCAST || kind == ORC_ROW) return 1;
  if (kind == ORC_FRAME) return frames >= 1 && L % frames == 0;
  return 0;
}

/* ---- one row ------------------------------------------------------------ */

static double operand(const void* p, int f32, int64_t c) {
  return f32 ? (double)((const float*)p)[c] : orc_bf16_to_f64(((const uint16_t*)p)[c]);
}

/*
 * Normalise the binary64 row h[0..D) and apply affine + modulation, giving the
 * binary64 row t.  LayerNorm: mean and biased variance (two passes).  RMSNorm:
 * mean of squares.  eps is added inside the square root.  weight and bias are
 * bf16, or binary32 when affine_f32.
 * Output by y_dtype: bf16 (y is uint16_t), binary32 (float, nearest-even
 * cast of t), or FP8 E4M3 with a per-row scale: y_scale = max|t| / 448 as a
 * binary32 value, and each element is the E4M3 rounding of t / y_scale
 * (when y_scale is 0: 0 for finite elements, NaN for NaN ones).
 */
static void norm_row(const double* h, double* t, int64_t D, int is_rms, double eps,
                     const void* w, const void* bias, int affine_f32,
                     const uint16_t* scale_row, const uint16_t* shift_row,
                     int y_dtype, void* y_row, float* y_scale, double* t_row) {
  double mean = 0.0;
  if (!is_rms) {
    double sum = 0.0;
    for (int64_t c = 0; c < D; ++c) sum += h[c];
    mean = sum / (double)D;
  }
  double sq = 0.0;
  for (int64_t c = 0; c < D; ++c) {
    double d = h[c] - mean;
    sq += d * d;
  }
  double var = sq / (double)D;
  double rho = 1.0 / sqrt(var + eps);
  for (int64_t c = 0; c < D; ++c) {
    double n = (h[c] - mean) * rho;
    if (w) n = n * operand(w, affine_f32, c);
    if (bias) n = n + operand(bias, affine_f32, c);
    t[c] = n * (1.0 + orc_bf16_to_f64(scale_row[c])) + orc_bf16_to_f64(shift_row[c]);
    if (t_row) t_row[c] = t[c];
  }
  if (y_dtype == ORC_Y_BF16) {
    for (int64_t c = 0; c < D; ++c) ((uint16_t*)y_row)[c] = orc_f64_to_bf16(t[c]);
  } else if (y_dtype == ORC_Y_F32) {
    for (int64_t c = 0; c < D; ++c) ((float*)y_row)[c] = (float)t[c];
  } else {
    double amax = 0.0;
    for (int64_t c = 0; c < D; ++c)
      if (fabs(t[c]) > amax) amax = fabs(t[c]);
    float s = (float)(amax / 448.0);
    *y_scale = s;
    /* A row whose elements are all zero or NaN has scale 0: its zeros encode
     * as 0 and its NaNs stay NaN. */
    for (int64_t c = 0; c < D; ++c)
      ((uint8_t*)y_row)[c] = s > 0.0f ? orc_f64_to_e4m3(t[c] / (double)s)
                                      : (isnan(t[c]) ? orc_f64_to_e4m3(t[c]) : 0);
  }
}

static int64_t y_elem_bytes(int y_dtype) {
  return y_dtype == ORC_Y_F32 ? 4 : (y_dtype == ORC_Y_FP8 ? 1 : 2);
}

static int common_args_ok(const void* x, const void* weight, const void* bias,
                          const void* scale, const void* shift, int64_t B, int64_t L,
                          int64_t D, int ss_kind, int64_t ss_frames, float eps,
                          int64_t row0, int64_t nrows, const void* y) {
  if (!x || !scale || !shift || !y) return 0;
  if (bias && !weight) return 0;
  if (B < 0 || L < 0 || D < 1) return 0;
  if (!(eps >= 0.0f) || isinf(eps)) return 0;
  if (row0 < 0 || nrows < 0 || row0 + nrows > B * L) return 0;
  if (B * L > 0 && !layout_ok(ss_kind, ss_frames, L)) return 0;
  return 1;
}

int orc_fused_ex(const uint16_t* x, const uint16_t* residual, const uint16_t* gate,
                 const void* weight, const void* bias, const uint16_t* scale,
                 const uint16_t* shift, int64_t B, int64_t L, int64_t D, int is_rms,
                 int gate_kind, int64_t gate_frames, int ss_kind, int64_t ss_frames, float eps,
                 int affine_f32, int y_dtype, int64_t row0, int64_t nrows, void* y,
                 float* y_scale, uint16_t* residual_out, double* t_out) {
  if (!common_args_ok(x, weight, bias, scale, shift, B, L, D, ss_kind, ss_frames, eps,
                      row0, nrows, y))
    return ORC_EINVAL;
  if (!residual || !residual_out) return ORC_EINVAL;
  if (gate && B * L > 0 && !layout_ok(gate_kind, gate_frames, L)) return ORC_EINVAL;
  if (y_dtype < ORC_Y_BF16 || y_dtype > ORC_Y_FP8 || (y_dtype == ORC_Y_FP8 && !y_scale))
    return ORC_EINVAL;
  if (nrows == 0) return ORC_OK;

  double* h = (double*)malloc((size_t)D * 2 * sizeof(double));
  if (!h) return ORC_EINVAL;
  for (int64_t r = row0; r < row0 + nrows; ++r) {
    const uint16_t* g_row = gate ? gate + orc_mod_row(gate_kind, gate_frames, r, L) * D : NULL;
    int64_t is = orc_mod_row(ss_kind, ss_frames, r, L);
    for (int64_t c = 0; c < D; ++c) {
      int64_t k = (r - row0) * D + c;
      uint16_t ro = residual_update(residual[k], g_row ? &g_row[c] : NULL, x[k]);
      residual_out[k] = ro;
      h[c] = orc_bf16_to_f64(ro);
    }
    norm_row(h, h + D, D, is_rms, (double)eps, weight, bias, affine_f32, scale + is * D,
             shift + is * D, y_dtype, (char*)y + (r - row0) * D * y_elem_bytes(y_dtype),
             y_scale ? y_scale + (r - row0) : NULL, t_out ? t_out + (r - row0) * D : NULL);
  }
  free(h);
  return ORC_OK;
}

int orc_nss_ex(const uint16_t* x, const void* weight, const void* bias,
               const uint16_t* scale, const uint16_t* shift, int64_t B, int64_t L, int64_t D,
               int is_rms, int ss_kind, int64_t ss_frames, float eps, int affine_f32,
               int y_dtype, int64_t row0, int64_t nrows, void* y, float* y_scale,
               double* t_out) {
  if (!common_args_ok(x, weight, bias, scale, shift, B, L, D, ss_kind, ss_frames, eps,
                      row0, nrows, y))
    return ORC_EINVAL;
  if (y_dtype < ORC_Y_BF16 || y_dtype > ORC_Y_FP8 || (y_dtype == ORC_Y_FP8 && !y_scale))
    return ORC_EINVAL;
  if (nrows == 0) return ORC_OK;

  double* h = (double*)malloc((size_t)D * 2 * sizeof(double));
  if (!h) return ORC_EINVAL;
  for (int64_t r = row0; r < row0 + nrows; ++r) {
    int64_t is = orc_mod_row(ss_kind, ss_frames, r, L);
    for (int64_t c = 0; c < D; ++c) h[c] = orc_bf16_to_f64(x[(r - row0) * D + c]);
    norm_row(h, h + D, D, is_rms, (double)eps, weight, bias, affine_f32, scale + is * D,
             shift + is * D, y_dtype, (char*)y + (r - row0) * D * y_elem_bytes(y_dtype),
             y_scale ? y_scale + (r - row0) : NULL, t_out ? t_out + (r - row0) * D : NULL);
  }
  free(h);
  return ORC_OK;
}

int orc_fused(const uint16_t* x, const uint16_t* residual, const uint16_t* gate,
              const uint16_t* weight, const uint16_t* bias,
              const uint16_t* scale, const uint16_t* shift,
              int64_t B, int64_t L, int64_t D, int is_rms,
              int gate_kind, int64_t gate_frames, int ss_kind, int64_t ss_frames,
              float eps, int64_t row0, int64_t nrows,
              uint16_t* y, uint16_t* residual_out, double* t_out) {
  return orc_fused_ex(x, residual, gate, weight, bias, scale, shift, B, L, D, is_rms, gate_kind,
                      gate_frames, ss_kind, ss_frames, eps, 0, ORC_Y_BF16, row0, nrows, y, NULL,
                      residual_out, t_out);
}

int orc_nss(const uint16_t* x, const uint16_t* weight, const uint16_t* bias,
            const uint16_t* scale, const uint16_t* shift,
            int64_t B, int64_t L, int64_t D, int is_rms,
            int ss_kind, int64_t ss_frames, float eps,
            int64_t row0, int64_t nrows, uint16_t* y, double* t_out) {
  return orc_nss_ex(x, weight, bias, scale, shift, B, L, D, is_rms, ss_kind, ss_frames, eps, 0,
                    ORC_Y_BF16, row0, nrows, y, NULL, t_out);
}
