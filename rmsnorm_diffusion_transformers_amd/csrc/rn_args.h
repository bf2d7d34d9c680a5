// rn_args.h -- the kernel argument block shared by the host launcher and the
// gfx950 row kernels, and the table of compiled specialisations.
#pragma once

#include <stdint.h>

namespace rn {

constexpr int kWaveSize = 64;

// Compiled shapes: W waves per activation row, RPB rows per workgroup (a
// workgroup is W * RPB waves), VPT 16-byte vectors per lane.  One wave holds
// a W-th of a row, VPT vectors of 8 bf16 per lane per operand, so a shape
// covers rows of up to 64 * W * VPT vectors (D = 512 * W * VPT); tail lanes of
// shorter rows are masked.
//
// Choice (measured on MI355X; each rule from sweeps over every compiled shape).
// The large-problem rules were re-measured in one process on two placements
// of the tensors -- torch's back-to-back allocations (every stream in one
// third of physical HBM) and a spread placement (the outputs in two other
// thirds) -- each pick against the shape it displaces; the figures are
// rule pick vs displaced shape, in % of 8 TB/s:
//   * a problem that streams at most 4 tensors through HBM (x, y, and the
//     residual pair of the fused op; broadcast / per-frame modulation rows
//     come from L2) and has more than kMidRows rows runs best with long
//     per-wave rows: the first shape with W < 10, in table order, that
//     covers D and keeps VPT * (row operands loaded) <= kVgprBudget -- one
//     wave per row at D = 5120 (L = 90000-176400);
//   * a problem that also streams per-row scale/shift (or a per-row gate)
//     runs best with 10 waves per row and 1-4 vectors per lane (shorter
//     per-wave spans and more rows in flight), once D >= kManyStreamsMinD
//     (fused RMS + weight, D 10240: 75.9 vs 73.3 back to back, 81.9 vs
//     82.3 spread; fused LN, D 5120: 74.6 vs 71.7, 81.1 vs 81.5 -- a gain
//     where the streams share a third, a wash where they do not);
//   * from D >= kSplitMinD, problems of a few hundred rows leave most SIMDs
//     idle with one wave per row and are bound by each row's load -> reduce
//     -> store chain, so the row is split so that each wave holds 2-5
//     vectors per lane: 4 waves per row up to kSmallRows rows, then 2 waves
//     while D <= 3072 and 4 above, up to kMidRowsSplit4 rows (up to 2 *
//     kSmallRows below D = 2560), then 2 up to kMidRows (from D >= 2560);
//     the sweep at 64-4096 rows found these 10-30 % faster than one wave per
//     row (e.g. 512 rows, D = 5120: 6.3 -> 5.3 us);
//   * at most kTinyRows rows with 4096 < D <= 5120 use 10 waves of one
//     vector each (L = 16, D = 5120: 2.8 us per call in a HIP graph);
//   * the fused op keeps one wave per row (when it fits the register budget)
//     from 2 * kSmallRows + 1 up to kFusedOneWaveRows rows: with its loads
//     ordered, spaced and prioritised it measured 5-18 % faster there than
//     2 or 4 waves per row (e.g. D = 5120, 1024 rows: 9.8 -> 8.3 us);
//   * the norm-only op with weight (and bias), from kMultiRowMinElems
//     elements (rows x D), when every aligned group of K rows shares one
//     scale/shift row, runs a multi-row shape (K > 1): each wave loads the
//     shared rows -- weight, bias, scale, shift -- once and then streams K
//     consecutive rows through them, instead of re-reading up to 60 KB of
//     shared rows from L2 for every 10 KB activation row.  The first
//     multi-row shape that covers D (at most 5 vectors per lane, so the
//     shared rows stay in registers at 2 waves per SIMD) measured faster
//     than the one-row shapes at every point of a sweep from 12.6 M
//     elements up, D = 512 to 10240, by 0.5-66 % (D = 5120, L = 176400:
//     binary32 weight/bias 0.69 -> 0.61 ms, bf16 0.92 -> 0.61 ms), and
//     slower below about 8 M elements, where 4x fewer waves leave part of
//     the chip idle (re-measured, binary32 / bf16 weight+bias at D 5120 and
//     binary32 at D 2048: 73.8 / 74.2 / 79.0 vs 66.0 / 70.8 / 62.6 back to
//     back, 77.3 / 77.4 / 79.5 vs 66.5 / 72.8 / 64.2 spread).  K = 4 beat K = 2 and
//     K = 8; prefetching the next row before the current row's stores did
//     not help on balance.  The fused op and the norm-only op without
//     affine ran slower as multi-row shapes.
//   * the norm-only op without affine, from kMultiRowMinElems elements, runs
//     its one-wave shapes of 8 or 10 vectors per lane with 2 rows per
//     workgroup instead of 4 (the twins at the end of the table): with the
//     tensors at a measured HBM placement, D = 5120 78.0 -> 79.5 % of 8 TB/s
//     and D = 4096 78.8-79.6 -> 80.0 %; on back-to-back allocations within
//     +-0.4 % at D = 5120 and 74.4 -> 75.6 % at D = 4096 (re-measured: D 5120
//     75.0 vs 75.3 back to back, 79.1 vs 77.6 spread; D 4096 76.5 vs 75.1,
//     80.3 vs 78.9).  At 4 vectors per lane 2 rows per workgroup were slower
//     (D = 2048: 81.1 -> 80.2 %), at 6 the same.
struct Shape {
  int w;
  int vpt;
  int rpb;
  int k = 1;  // consecutive rows per wave
};
// One-row shapes sorted by W, then VPT (the planner takes the first fit of a
// given W), then the multi-row shapes in the same order, then twins of
// one-row shapes with fewer rows per workgroup (never a first fit: they
// follow shapes of the same W and VPT).
constexpr Shape kShapes[] = {{1, 1, 4},  {1, 2, 4},  {1, 3, 4},  {1, 4, 4},  {1, 5, 4},
                             {1, 6, 4},  {1, 8, 4},  {1, 10, 4}, {2, 3, 2},  {2, 4, 2},
                             {2, 5, 2},  {2, 6, 2},  {2, 8, 2},  {2, 10, 2}, {4, 2, 1},
                             {4, 3, 1},  {4, 4, 1},  {4, 5, 1},  {4, 6, 1},  {4, 8, 1},
                             {10, 1, 1}, {10, 2, 1}, {10, 3, 1}, {10, 4, 1},
                             // multi-row shapes (norm-only with weight)
                             {1, 1, 4, 4}, {1, 2, 4, 4}, {1, 3, 4, 4}, {1, 4, 4, 4},
                             {1, 5, 4, 4}, {2, 3, 2, 4}, {2, 4, 2, 4}, {2, 5, 2, 4},
                             {4, 3, 1, 4}, {4, 4, 1, 4}, {4, 5, 1, 4},
                             // two rows per workgroup (large norm-only problems)
                             {1, 8, 2}, {1, 10, 2}};
constexpr int kManyStreamsMinD = 2560;
constexpr int kSplitMinD = 2048;
constexpr int kTinyRows = 128;
constexpr int kSmallRows = 256;
constexpr int kMidRowsSplit4 = 768;
constexpr int kMidRows = 1536;
constexpr int kFusedOneWaveRows = 1024;
constexpr int64_t kMultiRowMinElems = 12 << 20;
constexpr int kNumShapes = sizeof(kShapes) / sizeof(kShapes[0]);
// VPT x operands per row kept below this: all loads of a row are in flight at
// once, 4 VGPRs per vector per operand, and about 2 waves per SIMD is enough
// to saturate HBM with this access pattern.
constexpr int kVgprBudget = 52;
// The norm-only op with weight keeps weight and bias live through the
// epilogue next to the whole row (the fused op's x and gate die after the
// residual update), so its kernels need more registers per operand vector:
// 253-292 VGPRs at 5 operands x VPT 10 (one wave per SIMD), against 224 for
// the fused op with gate.  Its tighter budget moves it to 2 x 5 vectors at
// D = 4608-5120 and 4 x 5 at D = 8704-10240, measured 21 % and 24-32 %
// faster at 16384-176400 rows with per-row scale/shift (which keeps it off
// the multi-row shapes) and no slower on small problems (re-measured, bf16
// weight + bias, per-row scale/shift, D 5120: 77.4 vs 62.8 back to back,
// 79.7 vs 63.2 spread).
constexpr int kVgprBudgetNormAffine = 48;
// Spacing of loads / stores, in units of 8 cycles (s_nop 7); the streamed
// row loads of the fused op with one wave per row, and of the norm-only op
// with binary32 weight/bias, have their own.
constexpr int kPaceLoads = 0;
constexpr int kPaceFusedRowLoads = 1;
constexpr int kPaceStores = 2;
// binary32 y: twice the stores per row, spaced wider (measured 2 % faster
// than kPaceStores at L = 176400, D = 5120; re-measured in one process, the
// fused op with per-frame modulation: 68.6 % of 8 TB/s against 66.8 % at
// 16 cycles on back-to-back allocations, but 80.8 % against 82.1 % with the
// outputs in other thirds of HBM -- kept for ordinary allocations)
constexpr int kPaceStoresF32 = 4;

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
  float* y_scale;      // FP8 output: per-row scale (else unused)
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

// Affine variants: none, bf16 weight, bf16 weight + bias, binary32 weight,
// binary32 weight + bias.
enum { kAffNone = 0, kAffW16 = 1, kAffWB16 = 2, kAffW32 = 3, kAffWB32 = 4 };
constexpr int kNumAff = 5;

// Output types of y.
enum { kOutBf16 = 0, kOutF32 = 1, kOutFp8 = 2 };

// Kernel lookup; nullptr for an uncompiled combination.  shape indexes
// kShapes; out is a kOut* value.
KernelFn fused_kernel(bool rms, int out, bool gate, int aff, int shape);
KernelFn nss_kernel(bool rms, int out, int aff, int shape);

}  // namespace rn
