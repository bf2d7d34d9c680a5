/*
 * resnorm.h -- C ABI of the MI355X (gfx950) fused residual-norm library.
 *
 * The row-wise hot path of a video diffusion transformer block: a gated
 * residual update followed by LayerNorm or RMSNorm and the adaLN-style
 * scale/shift modulation, on [B, L, D] bf16 activations.  The two operations
 * are those of the custom ops flydsl_fused_residual_norm_scale_shift and
 * flydsl_norm_scale_shift, with the same operand order (sglang PR #36349,
 * "[AMD][Diffusion] Migrate FlyDSL fused norm kernels to the v0.3.0 stable
 * API", section "Microbenchmark", reproduction snippet), and the
 * specialisation matrix is_rms x has_gate x has_weight plus the broadcast,
 * per-row and 4D per-frame modulation layouts (sglang PR #33144, same title,
 * sections "Modifications" and "Accuracy Tests").
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers to bf16 data (raw bits), owned
 *     by the caller, contiguous row-major, 16-byte aligned.  Row stride = D.
 *   - The library never allocates, frees or synchronises.  Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the null stream) and the call returns;
 *     the outputs are valid once the stream reaches that point.
 *   - Activation row r = b * L + l (batch b, token l), 0 <= r < B * L.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     non-OK status nothing was enqueued and rn_last_error() describes the
 *     problem.  There is no fallback path: an unsupported case is an error.
 *     (The pages' history is of silent fallbacks: an unavailable fused kernel
 *     quietly replaced by the native path -- sglang PR #36349, "Motivation";
 *     sglang PR #33144, "Motivation".)
 *   - The host keeps, per thread, the last call it validated with its launch
 *     plan: a call that repeats it exactly (same pointers, sizes, flags,
 *     layouts, eps and element types) is enqueued without validating again.
 *   - B * L == 0 is valid and enqueues nothing.
 *   - Exact aliasing y == x and residual_out == residual is allowed (each
 *     element is read before it is overwritten, by the same thread); any other
 *     overlap between an output and another operand is RN_EINVAL.
 *   - The library is thread-safe; calls that overlap in time and write the
 *     same memory race, as any two kernels would.
 *
 * Performance note: the kernels stream every operand once, so their rate is
 * set by HBM, and on MI355X it also depends on where the caller's buffers sit
 * in physical memory: which third of it (96 GiB of the 288 GiB part) each
 * streamed tensor lies in.  With both outputs in one third (as four
 * back-to-back allocations are) the fused op measured 75-79.5 % of 8 TB/s,
 * with the outputs in two different thirds 82-83 %.  Physical addresses are
 * not visible to the caller; the Python package's hbm module measures a good
 * placement inside one large allocation (96 GiB is enough: 81.8 % for the
 * fused op at B 1, L 176400, D 5120) by timing these entry points.
 */
#ifndef RESNORM_H
#define RESNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RN_OK = 0,
  RN_EINVAL = 1,        /* invalid argument (null/misaligned pointer, bad shape, flag/pointer mismatch, overlap) */
  RN_EUNSUPPORTED = 2,  /* valid but outside what the kernels support (D > RN_D_MAX, B*L >= 2^31) */
  RN_ELAUNCH = 3        /* the HIP runtime refused the launch (see rn_last_error) */
} rn_status;

/* Bits of `flags`. */
enum {
  RN_RMS = 1u << 0,     /* RMSNorm (no centring) instead of LayerNorm */
  RN_GATE = 1u << 1,    /* residual_out = residual + gate * x (else residual + x); fused op only */
  RN_WEIGHT = 1u << 2,  /* multiply the normalised row by weight[D] */
  RN_BIAS = 1u << 3     /* then add bias[D]; requires RN_WEIGHT */
};

/* How an activation row selects its row of a modulation operand (gate, or
 * scale and shift, which share one layout). */
typedef enum {
  RN_BCAST = 0,  /* one dense (1, D) row shared by every activation row (every batch too) */
  RN_ROW = 1,    /* a (B, L, D) tensor: row r */
  RN_FRAME = 2   /* a (B, F, 1, D) tensor, tokens frame-major: row b*F + l / (L/F); needs L % F == 0 */
} rn_layout_kind;

typedef struct {
  int32_t kind;    /* rn_layout_kind */
  int32_t frames;  /* F for RN_FRAME (>= 1); ignored otherwise */
} rn_layout;

/* Largest supported row width. */
#define RN_D_MAX 16384

/* Element types for rn_ext. */
enum {
  RN_DTYPE_BF16 = 0,      /* bfloat16 */
  RN_DTYPE_F32 = 1,       /* IEEE binary32 */
  RN_DTYPE_FP8_E4M3 = 2   /* OCP FP8 E4M3 ("e4m3fn"): max 448, no infinities */
};

/* Optional element types of the *_ex entry points (a NULL rn_ext pointer
 * means all bf16). */
typedef struct {
  int32_t affine_dtype;  /* weight and bias: RN_DTYPE_BF16 or RN_DTYPE_F32 */
  int32_t y_dtype;       /* y: RN_DTYPE_BF16, RN_DTYPE_F32 or RN_DTYPE_FP8_E4M3 */
  void* y_scale;         /* RN_DTYPE_FP8_E4M3 only (else NULL): [B*L] binary32 per-row
                            scales written by the call, y = y_scale[r] * e4m3 */
} rn_ext;

/*
 * resnorm_fused_fwd -- gated residual update + norm + modulation.
 *
 * For every activation row r and column c (sglang PR #36349, "Microbenchmark":
 * flydsl_fused_residual_norm_scale_shift(residual, x, gate, weight, bias,
 * scale, shift, norm_type, eps); the formula is this library's reading of it):
 *   s                   = f32(residual[r,c]) + f32(gate[g(r),c]) * f32(x[r,c])
 *                         (the exact value rounded once to binary32, as a fused
 *                         multiply-add rounds it; also when gate * x falls below
 *                         the binary32 normal range)
 *   residual_out[r,c]   = bf16_rne(s)
 *   h                   = residual_out[r, :] as f32
 *   LayerNorm:  n = (h - mean(h)) * rsqrt(var(h) + eps)    (biased variance, 1/D)
 *   RMSNorm:    n = h * rsqrt(mean(h^2) + eps)
 *   n = n * weight[c] (+ bias[c])                            (if RN_WEIGHT / RN_BIAS)
 *   y[r,c]             = bf16_rne(n * (1 + scale[s(r),c]) + shift[s(r),c])
 * g(r), s(r) are the rows selected by gate_layout and ss_layout.
 *
 *   y, residual_out  [B*L, D] outputs (y may be x; residual_out may be residual)
 *   x, residual      [B*L, D] inputs
 *   gate             rows per gate_layout; must be NULL iff !(flags & RN_GATE)
 *                    (without RN_GATE, gate_layout is ignored)
 *   weight, bias     [D]; NULL iff the corresponding flag is clear
 *   scale, shift     rows per ss_layout; required
 *   B, L, D          B, L >= 0; 8 <= D <= RN_D_MAX, D % 8 == 0
 *   flags            RN_RMS | RN_GATE | RN_WEIGHT | RN_BIAS
 *   eps              finite, >= 0 (added inside the square root)
 *   stream           hipStream_t to enqueue on
 * Returns RN_OK once enqueued, else an error status (nothing enqueued).
 */
rn_status resnorm_fused_fwd(void* y, void* residual_out, const void* x, const void* residual,
                            const void* gate, const void* weight, const void* bias,
                            const void* scale, const void* shift, int64_t B, int64_t L,
                            int64_t D, uint32_t flags, rn_layout gate_layout,
                            rn_layout ss_layout, float eps, void* stream);

/*
 * norm_scale_shift_fwd -- norm + modulation without residual or gate
 * (flydsl_norm_scale_shift(x, weight, bias, scale, shift, norm_type, eps),
 * sglang PR #36349, "Microbenchmark"): the formula above with h = x.
 *
 *   y       [B*L, D] output (may be x)
 *   x       [B*L, D] input
 *   weight, bias, scale, shift, B, L, D, eps, stream: as above
 *   flags   RN_RMS | RN_WEIGHT | RN_BIAS (RN_GATE is RN_EINVAL)
 */
rn_status norm_scale_shift_fwd(void* y, const void* x, const void* weight, const void* bias,
                               const void* scale, const void* shift, int64_t B, int64_t L,
                               int64_t D, uint32_t flags, rn_layout ss_layout, float eps,
                               void* stream);

/*
 * resnorm_fused_fwd_ex / norm_scale_shift_fwd_ex -- the same operations with
 * other element types (rn_ext; NULL = all bf16):
 *   - binary32 weight / bias, used at full precision (the pages' fused-affine
 *     call passes fp32 affine parameters: sglang PR #36349, "Microbenchmark";
 *     the prior-art kernel casts them to bf16: sglang PR #33144, "Known gaps");
 *   - binary32 y: the binary32 result before the final rounding, rounded to
 *     nearest even (the pages note the two ops treat their output dtype
 *     differently: sglang PR #33144, "Known gaps");
 *   - FP8 E4M3 y with a per-row scale, for an FP8 consumer (the pages' WAN2.2
 *     runs enable FP8 attention: sglang PR #36349, "Command"): for each row,
 *     y_scale[r] = max_c |t[r,c]| / 448 and y[r,c] = E4M3(t[r,c] / y_scale[r]),
 *     nearest even (0 for an all-zero row).  y is then [B*L, D] bytes.
 * residual_out is bf16 in every case.  Errors as above, plus RN_EINVAL for an
 * unknown dtype, a y_scale that is missing for FP8 (or given otherwise) or
 * not 4-byte aligned, and overlaps of y_scale with any operand.
 */
rn_status resnorm_fused_fwd_ex(void* y, void* residual_out, const void* x, const void* residual,
                               const void* gate, const void* weight, const void* bias,
                               const void* scale, const void* shift, int64_t B, int64_t L,
                               int64_t D, uint32_t flags, rn_layout gate_layout,
                               rn_layout ss_layout, float eps, const rn_ext* ext, void* stream);

rn_status norm_scale_shift_fwd_ex(void* y, const void* x, const void* weight, const void* bias,
                                  const void* scale, const void* shift, int64_t B, int64_t L,
                                  int64_t D, uint32_t flags, rn_layout ss_layout, float eps,
                                  const rn_ext* ext, void* stream);

/* Text describing the last non-OK status returned on the calling thread
 * (empty if none).  The pointer stays valid until the thread's next call.
 * Every refusal carries its reason, because the failure this library is
 * built against is the silent one: the pages describe fused kernels that
 * fell back to the native path without a word (sglang PR #36349,
 * "Motivation"; sglang PR #33144, "Motivation"). */
const char* rn_last_error(void);

/* Launch shape the library would use for a problem (host-only query; no
 * device work, usable without a GPU): 16-byte vectors per lane and operand,
 * waves per activation row, waves and rows per workgroup, workgroup size,
 * the number of workgroups (laid out over a second grid dimension when one
 * dimension would exceed 2^32 - 1 work-items), and the consecutive rows
 * each wave handles in turn (1, or 4 for the norm-only op with weight
 * from 12 Mi elements (B * L * D >= 12582912) when every aligned group of 4
 * rows shares its scale/shift row: the wave then loads weight, bias, scale
 * and shift once for its 4 rows).  `fused` selects resnorm_fused_fwd (1) or
 * norm_scale_shift_fwd (0); the layouts matter because per-row modulation
 * operands add HBM streams, which changes the preferred shape, and so does
 * the row count (small problems are latency-bound).  The answer is for bf16
 * weight/bias; rn_describe_launch_ex takes the element types of the *_ex
 * entry points (binary32 weight/bias hold twice the registers per vector
 * and may get a shorter per-wave span; the output type does not change the
 * shape). */
typedef struct {
  int32_t vec_per_lane;
  int32_t waves_per_row;
  int32_t waves_per_block;
  int32_t rows_per_block;
  int32_t block_threads;
  int64_t grid_blocks;
  int32_t rows_per_wave;
} rn_launch_info;

rn_status rn_describe_launch(int64_t B, int64_t L, int64_t D, uint32_t flags, int32_t fused,
                             rn_layout gate_layout, rn_layout ss_layout, rn_launch_info* info);
/* The same for the *_ex entry points' element types (ext may be NULL: all
 * bf16).  RN_EINVAL for an unknown affine_dtype; both forms refuse, with the
 * launch's status and message, the shapes and layouts a launch would refuse
 * (pointers are not examined). */
rn_status rn_describe_launch_ex(int64_t B, int64_t L, int64_t D, uint32_t flags, int32_t fused,
                                rn_layout gate_layout, rn_layout ss_layout, const rn_ext* ext,
                                rn_launch_info* info);

/* Library version string. */
const char* rn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RESNORM_H */
