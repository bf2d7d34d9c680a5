/*
 * oracle_check.c -- drives every oracle entry point under AddressSanitizer and
 * UndefinedBehaviorSanitizer (CPU only; built and run by
 * tests/test_sanitize_cpu.py).
 *
 * Every buffer is allocated at its exact size, so a read or write one element
 * past any tensor is reported.  Inputs come from the seeded generator, with
 * some rows replaced by degenerate values (zeros, constants, infinities,
 * NaNs, magnitudes near the bf16 maximum).  The program checks only return
 * codes; the oracle's values are pinned elsewhere.  Exit status 0 and no
 * sanitizer report means clean.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

void synth_fill(uint16_t* out, int64_t n, int64_t idx0, uint64_t seed, uint32_t workload,
                uint32_t tensor, int dist, double a, double b, int64_t row_len,
                double stress_p, double stress_mul);

static int failures = 0;
static long calls = 0;

#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      fprintf(stderr, __VA_ARGS__);      \
      fputc('\n', stderr);               \
      ++failures;                        \
    }                                    \
  } while (0)

static uint16_t* bf16_tensor(int64_t n, uint32_t tensor, double mean, double sd) {
  uint16_t* p = (uint16_t*)malloc((size_t)(n > 0 ? n : 1) * sizeof *p);
  if (!p) abort();
  synth_fill(p, n, 0, 42, 900, tensor, 0, mean, sd, 0, 0.0, 1.0);
  return p;
}

static float* f32_tensor(int64_t n, uint32_t tensor, double mean, double sd) {
  uint16_t* h = bf16_tensor(n, tensor, mean, sd);
  float* p = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof *p);
  if (!p) abort();
  for (int64_t i = 0; i < n; ++i) {
    uint32_t b = (uint32_t)h[i] << 16;
    memcpy(&p[i], &b, sizeof b);
    p[i] *= 1.0f + 0x1p-12f * (float)(i % 7); /* values bf16 cannot hold */
  }
  free(h);
  return p;
}

/* Replace a few rows of x by degenerate rows. */
static void degenerate_rows(uint16_t* x, int64_t rows, int64_t D) {
  static const uint16_t fill[] = {0x0000, 0x3FC0, 0x7F80, 0xFF80, 0x7FC0, 0x7F7F, 0x0001};
  for (int64_t r = 0; r < rows && r < (int64_t)(sizeof fill / sizeof fill[0]); ++r) {
    if (r % 2 == 1) continue; /* keep some ordinary rows between them */
    for (int64_t c = 0; c < D; ++c) x[r * D + c] = fill[r];
  }
}

static int64_t mod_rows(int kind, int64_t frames, int64_t B, int64_t L) {
  return kind == ORC_BCAST ? 1 : kind == ORC_ROW ? B * L : B * frames;
}

static void run_case(int fused, int rms, int gate_kind, int ss_kind, int aff, int y_dtype,
                     int64_t B, int64_t L, int64_t D, int64_t frames, int degenerate) {
  const int64_t R = B * L;
  const int64_t gframes = gate_kind == ORC_FRAME ? frames : 0;
  const int64_t sframes = ss_kind == ORC_FRAME ? frames : 0;
  uint16_t* x = bf16_tensor(R * D, 1, 0.0, 1.0);
  uint16_t* res = fused ? bf16_tensor(R * D, 2, 0.0, 1.0) : NULL;
  uint16_t* gate = (fused && gate_kind >= 0)
                       ? bf16_tensor(mod_rows(gate_kind, frames, B, L) * D, 3, 0.5, 0.3)
                       : NULL;
  const int64_t ss = mod_rows(ss_kind, frames, B, L) * D;
  uint16_t* scale = bf16_tensor(ss, 4, 0.0, 0.1);
  uint16_t* shift = bf16_tensor(ss, 5, 0.0, 0.1);
  const int has_w = aff >= 1, has_b = aff == 2 || aff == 4, f32 = aff >= 3;
  void* w = NULL;
  void* bsp = NULL;
  if (has_w) w = f32 ? (void*)f32_tensor(D, 6, 1.0, 0.05) : (void*)bf16_tensor(D, 6, 1.0, 0.05);
  if (has_b) bsp = f32 ? (void*)f32_tensor(D, 7, 0.0, 0.1) : (void*)bf16_tensor(D, 7, 0.0, 0.1);
  if (degenerate) degenerate_rows(x, R, D);
  const size_t ysz = y_dtype == ORC_Y_F32 ? 4 : y_dtype == ORC_Y_FP8 ? 1 : 2;
  /* a sub-range of rows: the oracle must touch only those rows of the row
   * operands and outputs */
  const int64_t row0 = R > 2 ? 1 : 0;
  const int64_t nrows = R > 2 ? R - 2 : R;
  void* y = malloc((size_t)(nrows > 0 ? nrows : 1) * D * ysz);
  float* ys = y_dtype == ORC_Y_FP8 ? (float*)malloc((size_t)(nrows > 0 ? nrows : 1) * sizeof(float)) : NULL;
  uint16_t* ro = fused ? (uint16_t*)malloc((size_t)(nrows > 0 ? nrows : 1) * D * 2) : NULL;
  double* t = (double*)malloc((size_t)(nrows > 0 ? nrows : 1) * D * sizeof(double));
  int st;
  if (fused) {
    st = orc_fused_ex(x + row0 * D, res + row0 * D, gate, w, bsp, scale, shift, B, L, D, rms,
                      gate_kind < 0 ? ORC_BCAST : gate_kind, gframes, ss_kind, sframes, 1e-6f, f32,
                      y_dtype, row0, nrows, y, ys, ro, t);
    if (aff <= 2 && y_dtype == ORC_Y_BF16) {
      int st2 = orc_fused(x + row0 * D, res + row0 * D, gate, (const uint16_t*)w,
                          (const uint16_t*)bsp, scale, shift, B, L, D, rms,
                          gate_kind < 0 ? ORC_BCAST : gate_kind, gframes, ss_kind, sframes, 1e-6f,
                          row0, nrows, (uint16_t*)y, ro, NULL);
      CHECK(st2 == ORC_OK, "orc_fused status %d", st2);
    }
  } else {
    st = orc_nss_ex(x + row0 * D, w, bsp, scale, shift, B, L, D, rms, ss_kind, sframes, 1e-6f, f32,
                    y_dtype, row0, nrows, y, ys, t);
    if (aff <= 2 && y_dtype == ORC_Y_BF16) {
      int st2 = orc_nss(x + row0 * D, (const uint16_t*)w, (const uint16_t*)bsp, scale, shift, B, L,
                        D, rms, ss_kind, sframes, 1e-6f, row0, nrows, (uint16_t*)y, NULL);
      CHECK(st2 == ORC_OK, "orc_nss status %d", st2);
    }
  }
  CHECK(st == ORC_OK, "status %d: fused=%d rms=%d gate=%d ss=%d aff=%d y=%d B=%lld L=%lld D=%lld",
        st, fused, rms, gate_kind, ss_kind, aff, y_dtype, (long long)B, (long long)L, (long long)D);
  ++calls;
  free(x), free(res), free(gate), free(scale), free(shift), free(w), free(bsp);
  free(y), free(ys), free(ro), free(t);
}

static void invalid_arguments(void) {
  const int64_t D = 16, B = 1, L = 6;
  uint16_t* x = bf16_tensor(B * L * D, 1, 0, 1);
  uint16_t* s = bf16_tensor(B * L * D, 4, 0, 0.1);
  uint16_t* w = bf16_tensor(D, 6, 1, 0.05);
  uint16_t* y = (uint16_t*)malloc(B * L * D * 2);
  uint16_t* ro = (uint16_t*)malloc(B * L * D * 2);
  /* bias without weight */
  CHECK(orc_fused(x, x, NULL, NULL, w, s, s, B, L, D, 0, ORC_BCAST, 0, ORC_BCAST, 0, 1e-6f, 0, B * L,
                  y, ro, NULL) == ORC_EINVAL, "bias without weight accepted");
  /* frames that do not divide L, zero frames, unknown kinds */
  CHECK(orc_nss(x, NULL, NULL, s, s, B, L, D, 0, ORC_FRAME, 4, 1e-6f, 0, B * L, y, NULL) == ORC_EINVAL,
        "L %% F != 0 accepted");
  CHECK(orc_nss(x, NULL, NULL, s, s, B, L, D, 0, ORC_FRAME, 0, 1e-6f, 0, B * L, y, NULL) == ORC_EINVAL,
        "F = 0 accepted");
  CHECK(orc_nss(x, NULL, NULL, s, s, B, L, D, 0, 7, 0, 1e-6f, 0, B * L, y, NULL) == ORC_EINVAL,
        "unknown layout accepted");
  /* rows outside the problem */
  CHECK(orc_nss(x, NULL, NULL, s, s, B, L, D, 0, ORC_BCAST, 0, 1e-6f, 4, 3, y, NULL) == ORC_EINVAL,
        "row range past the end accepted");
  CHECK(orc_nss_ex(x, NULL, NULL, s, s, B, L, D, 0, ORC_BCAST, 0, 1e-6f, 0, 9, 0, B * L, y, NULL, NULL) ==
            ORC_EINVAL, "unknown y type accepted");
  free(x), free(s), free(w), free(y), free(ro);
}

static void elementwise(void) {
  enum { N = 1 << 16 };
  float* f = (float*)malloc(N * sizeof *f);
  double* d = (double*)malloc(N * sizeof *d);
  uint16_t* h = (uint16_t*)malloc(N * sizeof *h);
  uint8_t* q = (uint8_t*)malloc(N);
  for (uint32_t i = 0; i < N; ++i) {
    /* a spread of binary32 patterns: every exponent, both signs, NaNs, infinities */
    uint32_t bits = (i << 16) | (i * 2654435761u >> 16);
    memcpy(&f[i], &bits, sizeof bits);
    d[i] = (double)f[i] * (1.0 + 0x1p-30);
  }
  orc_f32_to_bf16_array(f, h, N);
  orc_f64_to_bf16_array(d, h, N);
  orc_f64_to_e4m3_array(d, q, N);
  uint16_t* a = bf16_tensor(N, 8, 0, 1);
  uint16_t* b = bf16_tensor(N, 9, 0, 1);
  orc_residual_array(a, b, h, h, N);
  orc_residual_array(a, NULL, h, h, N);
  for (int64_t r = 0; r < 64; ++r) {
    CHECK(orc_mod_row(ORC_BCAST, 0, r, 16) == 0, "bcast row");
    CHECK(orc_mod_row(ORC_ROW, 0, r, 16) == r, "per-row row");
    CHECK(orc_mod_row(ORC_FRAME, 4, r, 16) == (r / 16) * 4 + (r % 16) / 4, "per-frame row");
  }
  calls += 6;
  free(f), free(d), free(h), free(q), free(a), free(b);
}

int main(void) {
  static const int64_t widths[] = {8, 24, 1000, 5120, 16384};
  static const int ykinds[] = {ORC_Y_BF16, ORC_Y_F32, ORC_Y_FP8};
  for (size_t wi = 0; wi < sizeof widths / sizeof widths[0]; ++wi) {
    const int64_t D = widths[wi];
    for (int fused = 0; fused <= 1; ++fused)
      for (int rms = 0; rms <= 1; ++rms)
        for (int gk = fused ? -1 : -1; gk <= (fused ? ORC_FRAME : -1); ++gk)
          for (int sk = ORC_BCAST; sk <= ORC_FRAME; ++sk)
            for (int aff = 0; aff <= 4; ++aff)
              for (int yi = 0; yi < 3; ++yi) {
                const int64_t B = (aff + yi) % 2 ? 2 : 1, L = 6;
                run_case(fused, rms, gk, sk, aff, ykinds[yi], B, L, D, 3, (aff + sk) % 2);
              }
  }
  /* one row, and the empty problem */
  run_case(1, 0, ORC_BCAST, ORC_BCAST, 0, ORC_Y_BF16, 1, 1, 5120, 1, 0);
  run_case(0, 1, -1, ORC_ROW, 4, ORC_Y_FP8, 1, 1, 8, 1, 1);
  run_case(1, 1, ORC_FRAME, ORC_FRAME, 2, ORC_Y_F32, 0, 6, 64, 3, 0);
  invalid_arguments();
  elementwise();
  printf("oracle_check: %ld calls, %d failures\n", calls, failures);
  return failures ? 1 : 0;
}
