/*
 * oracle.h -- plain CPU oracle for the fused residual + gate + norm +
 * scale/shift row operation of video diffusion transformers.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path includes, links or
 * calls this.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code with the HIP library.
 *
 * All activations and modulation operands are bf16 bit patterns (uint16_t),
 * row-major, row stride D.  Arithmetic: the residual sum in binary32 (one
 * rounding to bf16), everything after it in binary64, one final rounding of
 * the binary64 result to bf16.  Round-to-nearest-even everywhere.
 */
#ifndef RN_ORACLE_H
#define RN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Modulation layouts (how an activation row picks its gate / scale / shift row). */
enum { ORC_BCAST = 0, ORC_ROW = 1, ORC_FRAME = 2 };

/* Status codes of the oracle entry points. */
enum { ORC_OK = 0, ORC_EINVAL = 1 };

/* Output types of y. */
enum { ORC_Y_BF16 = 0, ORC_Y_F32 = 1, ORC_Y_FP8 = 2 };

/* bf16 <-> binary64.  bf16 -> double is exact.  double -> bf16 is the
 * correctly rounded (nearest, ties to even) bf16 value; NaN -> 0x7FC0;
 * overflow -> +-Inf; bf16 subnormals kept. */
double   orc_bf16_to_f64(uint16_t h);
uint16_t orc_f64_to_bf16(double t);

/* binary64 -> OCP FP8 E4M3 (e4m3fn), nearest-even, saturating to +-448;
 * NaN -> 0x7F. */
uint8_t orc_f64_to_e4m3(double t);
void orc_f64_to_e4m3_array(const double* in, uint8_t* out, int64_t n);

/* Elementwise helpers for exhaustive checks: out[i] = bf16 RNE of in[i]. */
void orc_f32_to_bf16_array(const float* in, uint16_t* out, int64_t n);
void orc_f64_to_bf16_array(const double* in, uint16_t* out, int64_t n);

/* Elementwise residual update: out[i] = bf16(f32(res[i]) + f32(gate[i])*f32(x[i]))
 * (gate == NULL means gate = 1). */
void orc_residual_array(const uint16_t* res, const uint16_t* gate, const uint16_t* x,
                        uint16_t* out, int64_t n);

/* Modulation row selected by activation row r (0 <= r < B*L). */
int64_t orc_mod_row(int kind, int64_t frames, int64_t r, int64_t L);

/*
 * Fused op on rows [row0, row0 + nrows) of a [B, L, D] problem.
 *   residual_out = bf16(residual + gate * x)            (binary32 sum)
 *   h            = residual_out, as binary64
 *   n            = (h - mean) / sqrt(var + eps)          (LayerNorm)
 *                  h / sqrt(mean(h^2) + eps)             (RMSNorm)
 *   n            = n * weight (+ bias)                   (if given)
 *   t            = n * (1 + scale) + shift
 *   y            = bf16(t)
 * x, residual, y, residual_out and t_out address activation row row0 (their
 * first row is row row0); gate, weight, bias, scale and shift address whole
 * tensors (the modulation row is found from the global row index).
 * gate, weight, bias may be NULL (absent); bias requires weight.
 * t_out (may be NULL) receives the binary64 t before rounding.
 * Returns ORC_OK, or ORC_EINVAL for inconsistent arguments.
 */
int orc_fused(const uint16_t* x, const uint16_t* residual, const uint16_t* gate,
              const uint16_t* weight, const uint16_t* bias,
              const uint16_t* scale, const uint16_t* shift,
              int64_t B, int64_t L, int64_t D, int is_rms,
              int gate_kind, int64_t gate_frames, int ss_kind, int64_t ss_frames,
              float eps, int64_t row0, int64_t nrows,
              uint16_t* y, uint16_t* residual_out, double* t_out);

/*
 * Extended forms: weight/bias are binary32 when affine_f32 (else bf16), and y
 * is bf16 (uint16_t), binary32 (float) or FP8 E4M3 (uint8_t) by y_dtype; for
 * FP8, y_scale[i] receives the per-row scale max|t| / 448 (binary32) of row
 * row0 + i and y holds the E4M3 codes of t / y_scale.
 */
int orc_fused_ex(const uint16_t* x, const uint16_t* residual, const uint16_t* gate,
                 const void* weight, const void* bias, const uint16_t* scale,
                 const uint16_t* shift, int64_t B, int64_t L, int64_t D, int is_rms,
                 int gate_kind, int64_t gate_frames, int ss_kind, int64_t ss_frames, float eps,
                 int affine_f32, int y_dtype, int64_t row0, int64_t nrows, void* y,
                 float* y_scale, uint16_t* residual_out, double* t_out);

int orc_nss_ex(const uint16_t* x, const void* weight, const void* bias,
               const uint16_t* scale, const uint16_t* shift, int64_t B, int64_t L, int64_t D,
               int is_rms, int ss_kind, int64_t ss_frames, float eps, int affine_f32,
               int y_dtype, int64_t row0, int64_t nrows, void* y, float* y_scale,
               double* t_out);

/* Norm-scale-shift: the same with h = x and no residual output. */
int orc_nss(const uint16_t* x, const uint16_t* weight, const uint16_t* bias,
            const uint16_t* scale, const uint16_t* shift,
            int64_t B, int64_t L, int64_t D, int is_rms,
            int ss_kind, int64_t ss_frames, float eps,
            int64_t row0, int64_t nrows, uint16_t* y, double* t_out);

#ifdef __cplusplus
}
#endif
#endif
