// rn_args.h -- the kernel argument block shared by the host launcher and the
// gfx950 row kernels, and the table of compiled specialisations.
#pragma once

#include <stdint.h>

namespace rn {

// One workgroup = kWavesPerBlock waves; each wave owns one activation row.
constexpr int kWaveSize = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWaveSize * kWavesPerBlock;

// Per-lane register-cache widths (16-byte vectors of 8 bf16 per lane) that are
// compiled.  A row of D columns needs ceil(D / 8 / 64) vectors per lane; the
// launcher picks the smallest compiled width that covers it and the tail
// lanes are masked.  32 covers D = 16384.
constexpr int kVecWidths[] = {1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32};
constexpr int kNumVecWidths = sizeof(kVecWidths) / sizeof(kVecWidths[0]);

// Kernel arguments (one struct, passed by value).
struct RowArgs {
  const void* x;
  const void* residual;
  const void* gate;
  const void* weight;
  const void* bias;
  const void* scale;
  const void* shift;
  void* y;
  void* residual_out;
  uint32_t rows;       // B * L
  uint32_t L;          // tokens per batch
  uint32_t d;          // row width in elements (multiple of 8)
  uint32_t nvec;       // d / 8
  float eps;
  // modulation row selection: kind 0 = broadcast, 1 = per row, 2 = per frame
  int32_t gate_kind;
  uint32_t gate_frames;
  uint32_t gate_tokens_per_frame;
  int32_t ss_kind;
  uint32_t ss_frames;
  uint32_t ss_tokens_per_frame;
};

typedef void (*KernelFn)(RowArgs);

// Affine variants.
enum { kAffNone = 0, kAffWeight = 1, kAffWeightBias = 2 };

// Kernel lookup; each returns nullptr for an uncompiled combination.
// vec_index indexes kVecWidths.
KernelFn fused_ln_kernel(bool gate, int aff, int vec_index);
KernelFn fused_rms_kernel(bool gate, int aff, int vec_index);
KernelFn nss_ln_kernel(int aff, int vec_index);
KernelFn nss_rms_kernel(int aff, int vec_index);

}  // namespace rn
