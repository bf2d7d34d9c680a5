// rn_row_kernel.hpp -- gfx950 row kernel for the fused residual + gate +
// LayerNorm/RMSNorm + scale/shift operation and its norm-only variant.
//
// The operation (sglang PR #36349, "Microbenchmark": operand order of
// flydsl_fused_residual_norm_scale_shift / flydsl_norm_scale_shift; layouts
// and specialisations from sglang PR #33144, "Modifications"):
//   residual_out = bf16(residual + gate * x)         [binary32, one rounding]
//   h            = residual_out (fused) or x (norm-only)
//   n            = (h - mean) * rsqrt(var + eps)     [LayerNorm]
//                = h * rsqrt(mean(h^2) + eps)        [RMSNorm]
//   n            = n * weight (+ bias)
//   y            = bf16(n * (1 + scale) + shift)
//
// Design (HBM-bound; no matrix cores -- nothing here is a contraction):
//   * W wave64s own one activation row and a workgroup holds RPB row slots
//     (W * RPB waves).  A slot takes K consecutive rows in turn (K = 1 for
//     most shapes; 4 for the multi-row shapes, which load the rows shared by
//     the K rows -- weight, bias, scale, shift -- once per wave instead of
//     once per row).  Row indices are wave-uniform, so per-row quantities
//     (descriptors, modulation row, statistics) live in SGPRs.
//   * Every global access is a 128-bit buffer load/store (8 bf16 per lane) on
//     a per-row buffer descriptor whose range is exactly the row: lanes past
//     the end of a ragged row read zeros and their stores are dropped by the
//     hardware range check.
//   * All loads of a row -- x, residual, gate, weight, bias, scale, shift --
//     are issued before its first store, in a measured order and (one wave
//     per row) at raised wave priority.  Loads and stores share the in-order
//     vmcnt counter on gfx9, so a load issued after a store could only be
//     waited for together with that store; issuing every load first keeps the
//     store latency off the critical path.  (On the multi-row shapes the
//     shared rows are loaded once, before the first row, and each further
//     row's own loads follow the previous row's stores.)
//   * Loads are issued PL x 8 cycles apart and stores PS x 8 cycles apart
//     (s_nop): measured on MI355X, back-to-back bursts of 128-bit stores from
//     every wave stream several percent slower than lightly spaced ones.
//   * Streamed tensors (x, residual in; y, residual_out out) use the
//     non-temporal policy; modulation rows use the default policy, so the
//     broadcast and per-frame rows stay resident in L2.
//   * The row stays in VGPRs (bf16-packed) between the statistics and the
//     epilogue, so HBM sees each byte once.
//   * The fused op with one wave per row stages weight and bias in LDS: the
//     workgroup's waves fill it with buffer loads that write LDS directly
//     (no registers), issued before the rows' loads, and the epilogue reads
//     each vector's weight and bias back with ds_read_b128 (LDS reads wait on
//     lgkmcnt, not on the stores' vmcnt).  The registers then hold only the
//     row operands, so the fused affine op keeps one wave per row.
//   * Statistics in fp32.  LayerNorm: the mean, then the centred sum of squares
//     over the register-resident row.  RMSNorm: the sum of squares.  Wave
//     reductions are DPP (xor 1, xor 2, half-row mirror, row mirror) then the
//     gfx950 permlane16/permlane32 swaps; with W > 1 the per-wave totals are
//     combined through LDS in a fixed order.  Every lane and every wave of a
//     row ends with the bit-identical total.  Rows of finite values whose
//     binary32 sums overflow, and (with eps below 2^-100) rows whose variance
//     falls below 2^-100, are recomputed on the row scaled by a power of two
//     (a branch the common path only tests for).
//   * fp32 -> bf16 with v_cvt_pk_bf16_f32 (round to nearest even; fp32
//     denormals are kept in these kernels).
//   * Output y is bf16, binary32, or OCP FP8 E4M3 with a per-row scale
//     max|t| / 448 (compile-time; the FP8 kernels take a row maximum before
//     converting with v_cvt_pk_fp8_f32).
//   * weight / bias are bf16 or binary32 (compile-time).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rn_args.h"

namespace rn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Buffer descriptor word 3 for gfx9-family raw buffers (32-bit data format,
// no swizzle); num_records is in bytes.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy immediates of buffer instructions on gfx950: bit 1 = nt.
constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kRsrcWord3);
}

// Spacing after a memory instruction; the scheduling barrier keeps the
// compiler from regrouping the instructions into a burst.
template <int PACE>
__device__ __forceinline__ void pace() {
  if constexpr (PACE > 0) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < PACE; ++i) asm volatile("s_nop 7");
  }
}

template <int POLICY, int PACE>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
  pace<PACE>();
  return v;
}

template <int POLICY, int PACE>
__device__ __forceinline__ void store16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POLICY);
  pace<PACE>();
}

// s_waitcnt on vmcnt alone (expcnt and lgkmcnt at their maxima, i.e. not
// waited for): the gfx9 encoding keeps vmcnt bits 3:0 in bits 3:0 of the
// immediate and bits 5:4 in bits 15:14.
constexpr int kVmcntMax = 63;
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N <= kVmcntMax, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// bf16 pair <-> fp32: the low half of a dword is the element at the lower
// address.  Widening is a shift; narrowing is one v_cvt_pk_bf16_f32.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

struct Add {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct Max {
  __device__ __forceinline__ float operator()(float a, float b) const { return __builtin_fmaxf(a, b); }
};
// Maximum that propagates NaN (either operand NaN -> NaN), the same on both
// partners of a reduction step.
struct MaxNaN {
  __device__ __forceinline__ float operator()(float a, float b) const {
    return (a > b || a != a) ? a : b;
  }
};

// Whether a binary32 row statistic overflowed, decided the same way by every
// wave of the workgroup (a branch on it holds barriers when rows span
// several waves): from the row's own total when the workgroup holds one row
// or each wave is a row of its own; otherwise from the partial sums every
// row of the workgroup left in LDS.
template <int W, int RPB>
__device__ __forceinline__ bool overflowed(float total, const float* red) {
  bool any;
  if constexpr (W == 1 || RPB == 1) {
    any = !__builtin_isfinite(total);
  } else {
    any = false;
#pragma unroll
    for (int q = 0; q < RPB; ++q) {
      float t = red[q * W];
#pragma unroll
      for (int p = 1; p < W; ++p) t += red[q * W + p];
      any = any || !__builtin_isfinite(t);
    }
  }
  return __builtin_amdgcn_readfirstlane((int)any) != 0;
}

// Whether a row's variance takes the rescaled recomputation, decided the
// same way by every wave of the workgroup (as overflowed()): a binary32 sum
// of squares that overflowed, or a variance below `floor` (2^-100 when eps
// is below it, else -1: never), where the squares of tiny centred values
// underflow binary32.  The variances are formed as the rows formed theirs
// (partials in LDS order, times 1/D).
template <int W, int RPB>
__device__ __forceinline__ bool var_rescale(float var, const float* red, float inv_d, float floor) {
  bool any;
  if constexpr (W == 1 || RPB == 1) {
    any = !__builtin_isfinite(var) || var < floor;
  } else {
    any = false;
#pragma unroll
    for (int q = 0; q < RPB; ++q) {
      float t = red[q * W];
#pragma unroll
      for (int p = 1; p < W; ++p) t += red[q * W + p];
      const float v = t * inv_d;
      any = any || !__builtin_isfinite(v) || v < floor;
    }
  }
  return __builtin_amdgcn_readfirstlane((int)any) != 0;
}

// Power of two s = 2^-k that brings a finite, nonzero magnitude m into
// [1, 2); k = 0 (s = 1) when m is 0, infinite or NaN.
__device__ __forceinline__ int scale_exp(float m) {
  return (__builtin_isfinite(m) && m > 0.f) ? __builtin_amdgcn_frexp_expf(m) - 1 : 0;
}

// Reduction over the 64 lanes of a wave; every lane returns the same bits.
// Each step combines a lane's value with its partner's in an order that is
// the same on both partners, so the result is identical across lanes.
template <class OPR>
__device__ __forceinline__ float wave_reduce(float v, OPR op) {
  v = op(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]: partner lane ^ 1
  v = op(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]: partner lane ^ 2
  v = op(v, dpp<0x141>(v));  // row_half_mirror: the other quad of the 8-lane group
  v = op(v, dpp<0x140>(v));  // row_mirror: the other 8-lane half of the 16-lane row
  {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(p[0]), __uint_as_float(p[1]));  // rows 2k and 2k+1
  }
  {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = op(__uint_as_float(p[0]), __uint_as_float(p[1]));  // lanes 0-31 and 32-63
  }
  return v;
}

// Reduction over the W waves of one row.  Each wave's result goes to LDS;
// after the barrier every wave of the row combines the W partials in the same
// order.
template <int W, class OPR>
__device__ __forceinline__ float row_reduce(float v, OPR op, float* red, uint32_t wave,
                                            uint32_t slot) {
  v = wave_reduce(v, op);
  if constexpr (W > 1) {
    if ((threadIdx.x & (kWaveSize - 1)) == 0) red[wave] = v;
    __syncthreads();
    v = red[slot * W];
#pragma unroll
    for (int p = 1; p < W; ++p) v = op(v, red[slot * W + p]);
  }
  return v;
}

// Modulation row for activation row `row` = b * L + l.
__device__ __forceinline__ uint32_t mod_row(int32_t kind, uint32_t frames, uint32_t tpf,
                                            uint32_t row, uint32_t b, uint32_t l) {
  if (kind == 0) return 0;
  if (kind == 1) return row;
  return b * frames + l / tpf;
}

// What a kernel computes: LayerNorm or RMSNorm, fused residual or norm-only,
// gate, affine variant, output type.
template <bool RMS_, bool FUSED_, bool GATE_, int AFF_, int OUT_>
struct Op {
  static constexpr bool rms = RMS_;
  static constexpr bool fused = FUSED_;
  static constexpr bool gate = GATE_;
  static constexpr bool has_w = AFF_ != kAffNone;
  static constexpr bool has_b = AFF_ == kAffWB16 || AFF_ == kAffWB32;
  static constexpr bool aff32 = AFF_ == kAffW32 || AFF_ == kAffWB32;
  static constexpr int out = OUT_;
};

// An affine operand (weight or bias) for VPT vectors of 8 elements: bf16
// (one 16-byte vector each) or binary32 (two).
template <bool F32, int VPT>
struct AffineRow {
  u32x4 v[VPT][F32 ? 2 : 1];
  template <int PL>
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t base) {
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if constexpr (F32) {
        v[i][0] = load16<kPolicyDefault, PL>(r, base * 2u + i * 2048u);
        v[i][1] = load16<kPolicyDefault, PL>(r, base * 2u + i * 2048u + 16u);
      } else {
        v[i][0] = load16<kPolicyDefault, PL>(r, base + i * 1024u);
      }
    }
  }
  // element 2j (lo) and 2j+1 (hi) of vector i
  __device__ __forceinline__ float lo(int i, int j) const {
    if constexpr (F32) return __uint_as_float(v[i][j >> 1][(j & 1) * 2]);
    else return lo_f32(v[i][0][j]);
  }
  __device__ __forceinline__ float hi(int i, int j) const {
    if constexpr (F32) return __uint_as_float(v[i][j >> 1][(j & 1) * 2 + 1]);
    else return hi_f32(v[i][0][j]);
  }
};

// Weight (and bias) of a one-wave-per-row workgroup, staged in LDS by its
// RPB waves with buffer loads that write LDS directly.  LDS block (o, v, q)
// (1 KB: one 16-byte entry per lane) holds, for lane l, the 16-byte half q
// of operand o's vector v of that lane -- global chunk F * (v * 64 + l) + q
// -- so the epilogue's reads are contiguous across the wave.  Chunks past
// the end of a ragged row read as zeros.
template <class OP, int VPT, int RPB>
__device__ __forceinline__ void fill_affine_lds(const RowArgs& a, u32x4* lds, uint32_t wave,
                                                uint32_t lane) {
  constexpr int F = OP::aff32 ? 2 : 1;
  constexpr int NBLK = (OP::has_b ? 2 : 1) * VPT * F;
  const uint32_t abytes = a.d * (OP::aff32 ? 4u : 2u);
  const auto rw = row_rsrc(a.weight, abytes);
  const auto rb = row_rsrc(OP::has_b ? a.bias : a.weight, abytes);
#pragma unroll
  for (int i = 0; i < (NBLK + RPB - 1) / RPB; ++i) {
    const uint32_t blk = wave + (uint32_t)(i * RPB);
    if (blk < (uint32_t)NBLK) {
      const uint32_t o = blk / (VPT * F);
      const uint32_t rem = blk - o * (VPT * F);
      const uint32_t vi = rem / F;
      const uint32_t q = rem - vi * F;
      const uint32_t off = (F * (vi * kWaveSize + lane) + q) * 16u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          o ? rb : rw, (__attribute__((address_space(3))) void*)&lds[blk * kWaveSize], 16, off, 0, 0,
          kPolicyDefault);
    }
  }
}

// Position of one activation row: its index (0 past the last row), its byte
// offset, and the byte range of its buffers (0 past the last row, which
// turns every access into a no-op).
struct RowPos {
  uint32_t r;
  uint32_t bytes;
  uint64_t off;
  bool live;
};

template <class OP, int SHAPE>
__global__ __launch_bounds__(kWaveSize * kShapes[SHAPE].w * kShapes[SHAPE].rpb)
void row_kernel(const RowArgs a) {
  constexpr int W = kShapes[SHAPE].w;
  constexpr int VPT = kShapes[SHAPE].vpt;
  constexpr int RPB = kShapes[SHAPE].rpb;
  constexpr int K = kShapes[SHAPE].k;
  // weight / bias staged in LDS: the fused op, one wave per row, one row per
  // slot (measured 0.7-7.6 % faster than its previous shapes at D = 2048 to
  // 5120; the norm-only op, with fewer row operands, ran 2-5 % slower so)
  constexpr bool kLds = OP::fused && OP::has_w && W == 1 && K == 1;
  constexpr int F = OP::aff32 ? 2 : 1;
  constexpr int NBLK = (OP::has_b ? 2 : 1) * VPT * F;
  [[maybe_unused]] __shared__ u32x4 aff_lds[kLds ? NBLK * kWaveSize : 1];
  constexpr int PL = kPaceLoads;
  constexpr int PS = OP::out == kOutF32 ? kPaceStoresF32 : kPaceStores;
  static_assert(W * RPB * kWaveSize <= 1024, "workgroup size");
  // Cross-wave partials.  With several rows per slot (K > 1) and several
  // waves per row, one barrier per row does not keep a wave that has moved
  // on to row k + 1 from overwriting its row-k partial before a slower wave
  // of the row has read it (RMSNorm has a single barrier per row).  Rows
  // alternate between two copies by parity: row k + 2 writes copy k & 1
  // only after the barrier of row k + 1, which every wave reaches after
  // its reads of row k.
  constexpr int NBUF = (K > 1 && W > 1) ? 2 : 1;
  constexpr int NRED = W * RPB;
  [[maybe_unused]] __shared__ float red_sum_buf[NBUF * NRED];
  [[maybe_unused]] __shared__ float red_sq_buf[NBUF * NRED];
  [[maybe_unused]] __shared__ float red_max_buf[NBUF * NRED];

  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & (kWaveSize - 1);
  const uint32_t slot = wave / W;  // row slot in the workgroup
  const uint32_t part = wave % W;  // which contiguous part of the row this wave holds
  // Workgroups are numbered x-fastest over a 2D grid: the dispatch counts
  // work-items per dimension in 32 bits, so large problems spill into y.
  // A row slot holds K consecutive rows, the first at `first`.
  const uint32_t first = ((blockIdx.y * gridDim.x + blockIdx.x) * RPB + slot) * K;
  // With W > 1 every wave must reach the barriers, so a wave past the last
  // row keeps going with its memory operations disabled (zero-range buffers).
  auto at = [&](uint32_t row) {
    RowPos p;
    p.live = row < a.rows;
    p.bytes = p.live ? a.d * 2u : 0u;
    p.r = p.live ? row : 0u;
    p.off = (uint64_t)p.r * (a.d * 2u);
    return p;
  };
  // (a workgroup that stages weight/bias in LDS keeps every wave to the barrier)
  if constexpr (W == 1 && !kLds) {
    if (first >= a.rows) return;
  }
  const RowPos p0 = at(first);
  // Modulation rows of the slot's first row; with K > 1 the host guarantees
  // that all K rows share them.
  const uint32_t b = p0.r / a.L;
  const uint32_t l = p0.r - b * a.L;
  const uint32_t srow = mod_row(a.ss_kind, a.ss_frames, a.ss_tokens_per_frame, p0.r, b, l);
  // lane-local byte offset of vector v (bf16): this wave's part, then 1 KB per vector
  const uint32_t base = (part * VPT * kWaveSize + lane) * 16u;

  const auto rs_sc = row_rsrc((const char*)a.scale + (uint64_t)srow * (a.d * 2u), p0.bytes);
  const auto rs_sh = row_rsrc((const char*)a.shift + (uint64_t)srow * (a.d * 2u), p0.bytes);

  // ---- every load of a row, before any store ----
  // The order of the groups of loads is fixed at compile time (a run-time
  // choice merges paths whose loads are counted in different orders, and
  // the waits after the merge then cover every load).  One row per slot,
  // measured on MI355X at L = 90000-176400 (1-5 % on the whole kernel): ten
  // waves per row (the shapes chosen when per-row scale/shift or gate are
  // streamed from HBM): the activation rows, gate, weight/bias,
  // scale/shift; otherwise the shared rows ahead of the activation rows --
  // without affine: gate, scale/shift, activation rows; with affine:
  // scale/shift, activation rows, gate, weight/bias.  Several rows per
  // slot: the shared rows once, then each row's activation rows.
  u32x4 h[VPT];  // x (norm-only) or residual, later the bf16-packed residual_out
  [[maybe_unused]] u32x4 xv[VPT];
  [[maybe_unused]] u32x4 gv[VPT];
  [[maybe_unused]] AffineRow<OP::aff32, VPT> wv, bv;
  u32x4 sc[VPT], sh[VPT];
  const uint32_t aff_bytes = p0.live ? a.d * (OP::aff32 ? 4u : 2u) : 0u;
  auto load_gate = [&]() {
    if constexpr (OP::fused && OP::gate) {
      const uint32_t grow = mod_row(a.gate_kind, a.gate_frames, a.gate_tokens_per_frame, p0.r, b, l);
      const auto rs_g = row_rsrc((const char*)a.gate + (uint64_t)grow * (a.d * 2u), p0.bytes);
#pragma unroll
      for (int v = 0; v < VPT; ++v) gv[v] = load16<kPolicyDefault, PL>(rs_g, base + v * 1024u);
    }
  };
  // per-row scale/shift stream like the activations; shared rows stay cached
  auto load_ss = [&](auto policy) {
    constexpr int P = decltype(policy)::value;
#pragma unroll
    for (int v = 0; v < VPT; ++v) sc[v] = load16<P, PL>(rs_sc, base + v * 1024u);
#pragma unroll
    for (int v = 0; v < VPT; ++v) sh[v] = load16<P, PL>(rs_sh, base + v * 1024u);
  };
  auto load_affine = [&]() {
    if constexpr (OP::has_w) wv.template load<PL>(row_rsrc(a.weight, aff_bytes), base);
    if constexpr (OP::has_b) bv.template load<PL>(row_rsrc(a.bias, aff_bytes), base);
  };
  auto load_rows = [&](const RowPos& p) {
    const auto rs_x = row_rsrc((const char*)a.x + p.off, p.bytes);
    if constexpr (OP::fused) {
      // the fused op's 2 x VPT streamed loads, spaced (one wave per row):
      // measured 1 % faster at L = 176400, D = 5120; the norm-only op's VPT
      // loads run best unspaced
      constexpr int PLR = W == 1 ? kPaceFusedRowLoads : PL;
      const auto rs_r = row_rsrc((const char*)a.residual + p.off, p.bytes);
#pragma unroll
      for (int v = 0; v < VPT; ++v) xv[v] = load16<kPolicyStream, PLR>(rs_x, base + v * 1024u);
#pragma unroll
      for (int v = 0; v < VPT; ++v) h[v] = load16<kPolicyStream, PLR>(rs_r, base + v * 1024u);
    } else {
      // norm-only with binary32 weight/bias (L2-heavy: 60 KB of shared rows
      // per 10 KB row of x at D = 5120): spaced loads measured 8 % faster;
      // the other norm-only variants run best unspaced
      constexpr int PLN = OP::aff32 ? kPaceFusedRowLoads : PL;
#pragma unroll
      for (int v = 0; v < VPT; ++v) h[v] = load16<kPolicyStream, PLN>(rs_x, base + v * 1024u);
    }
  };
  auto load_ss_any = [&]() {
    if (a.ss_kind == 1) load_ss(std::integral_constant<int, kPolicyStream>{});
    else load_ss(std::integral_constant<int, kPolicyDefault>{});
  };
  // ---- the rest of a row, once its loads are issued ----
  auto process = [&](const RowPos& p, uint32_t copy) __attribute__((always_inline)) {
    float* const red_sum = red_sum_buf + copy * NRED;
    float* const red_sq = red_sq_buf + copy * NRED;
    float* const red_max = red_max_buf + copy * NRED;
    // ---- residual update (fused) ----
    if constexpr (OP::fused) {
      const auto rs_ro = row_rsrc((const char*)a.residual_out + p.off, p.bytes);
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float s0, s1;
          if constexpr (OP::gate) {
            // residual + gate * x rounded once: the fused multiply-add rounds
            // the exact sum.  (gate * x alone is exact in binary32 unless it
            // falls below the normal range, where rounding it first could also
            // lose the sign of a product that underflows to zero.)
            s0 = __builtin_fmaf(lo_f32(gv[v][j]), lo_f32(xv[v][j]), lo_f32(h[v][j]));
            s1 = __builtin_fmaf(hi_f32(gv[v][j]), hi_f32(xv[v][j]), hi_f32(h[v][j]));
          } else {
            s0 = lo_f32(h[v][j]) + lo_f32(xv[v][j]);
            s1 = hi_f32(h[v][j]) + hi_f32(xv[v][j]);
          }
          o[j] = pack_bf16(s0, s1);
        }
        store16<kPolicyStream, PS>(o, rs_ro, base + v * 1024u);
        h[v] = o;
      }
    }

    // ---- statistics (fp32) ----
    const float inv_d = 1.0f / (float)a.d;
    float mean = 0.f;
    // LayerNorm: mean * D - total, the rounding error of mean = total / D
    // times D (exact in binary32: a multiple of ulp(mean) below D * ulp(mean)
    // in magnitude).  For a row whose values sit within a few bf16 ulps of
    // each other (|mean| >> std) the error is comparable to the centred
    // values, and the normalisation would magnify it by |mean| / std; the
    // epilogue adds it back, scaled by rstd / D, in the fused multiply-add
    // that applies rstd.  (A row holding an infinity or a NaN gets NaN here,
    // as it does everywhere.)
    float mean_err = 0.f;
    float sq = 0.f;
    if constexpr (!OP::rms) {
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) sum += lo_f32(h[v][j]) + hi_f32(h[v][j]);
      const float total = row_reduce<W>(sum, Add{}, red_sum, wave, slot);
      mean = total / (float)a.d;
      mean_err = __builtin_fmaf(mean, (float)a.d, -total);
      // Finite values summing beyond the binary32 range (|h| ~ 1e34 and more):
      // the mean again from h * 2^-k, k from the row's largest magnitude (a
      // power of two, exact for every element that stays inside the binary32
      // range; the others are negligible next to the largest), scaled back.
      // Done before the variance pass, so that pass and the epilogue share
      // the centred values.  A row holding an infinity or a NaN keeps its
      // non-finite mean.
      if (overflowed<W, RPB>(mean, red_sum)) {
        float m = 0.f;
        const MaxNaN mx;
#pragma unroll
        for (int v = 0; v < VPT; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            m = mx(m, mx(__builtin_fabsf(lo_f32(h[v][j])), __builtin_fabsf(hi_f32(h[v][j]))));
        m = row_reduce<W>(m, mx, red_max, wave, slot);
        const int k = __builtin_isfinite(mean) ? 0 : scale_exp(m);
        const float s = __builtin_ldexpf(1.0f, -k);
        float sum2 = 0.f;
#pragma unroll
        for (int v = 0; v < VPT; ++v)
#pragma unroll
          for (int j = 0; j < 4; ++j) sum2 += lo_f32(h[v][j]) * s + hi_f32(h[v][j]) * s;
        const float total2 = row_reduce<W>(sum2, Add{}, red_sum, wave, slot);
        const float mean2 = total2 / (float)a.d;
        if (k != 0) {
          mean = __builtin_ldexpf(mean2, k);
          mean_err = __builtin_ldexpf(__builtin_fmaf(mean2, (float)a.d, -total2), k);
        }
      }
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        float part_sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d0 = lo_f32(h[v][j]) - mean;
          const float d1 = hi_f32(h[v][j]) - mean;
          part_sq = __builtin_fmaf(d0, d0, part_sq);
          part_sq = __builtin_fmaf(d1, d1, part_sq);
        }
        // lanes past the end of a ragged row hold zeros, which are not zero
        // after centring: leave them out.
        sq += (base / 16u + (uint32_t)(v * kWaveSize) < a.nvec) ? part_sq : 0.f;
      }
    } else {
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float h0 = lo_f32(h[v][j]);
          const float h1 = hi_f32(h[v][j]);
          sq = __builtin_fmaf(h0, h0, sq);
          sq = __builtin_fmaf(h1, h1, sq);
        }
    }
    float var = row_reduce<W>(sq, Add{}, red_sq, wave, slot) * inv_d;
    // Rounding can leave the variance slightly negative: lift it to 0.  A NaN
    // variance (a row holding an infinity or a NaN) must stay NaN.
    var = var < 0.f ? 0.f : var;
    float rstd = __builtin_amdgcn_rsqf(var + a.eps);
    // Finite centred values whose squares sum beyond the binary32 range
    // (|h - mean| ~ 1e17-1e19 and more), or, when eps is below 2^-100, a
    // variance below 2^-100 (centred values below ~1e-15, whose squares lose
    // bits in the binary32 subnormal range or underflow to 0): the
    // variance again from (h - mean) * 2^-k, k from the largest centred
    // magnitude, and rstd = 2^-k / sqrt(var' + eps * 2^-2k) (kept as it was
    // if eps * 2^-2k leaves the binary32 range: then eps alone decides
    // rstd).  Only rstd changes, so the epilogue is the same for every row.
    // Centred values in the binary32 subnormal range would need an rstd
    // beyond it and stay as computed.
    constexpr float kVarFloor = 0x1p-100f;
    const float var_floor = a.eps < kVarFloor ? kVarFloor : -1.f;
    if (var_rescale<W, RPB>(var, red_sq, inv_d, var_floor)) {
      float m = 0.f;
      const MaxNaN mx;
#pragma unroll
      for (int v = 0; v < VPT; ++v)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool in_row = base / 16u + (uint32_t)(v * kWaveSize) < a.nvec;
          const float d0 = in_row ? __builtin_fabsf(lo_f32(h[v][j]) - mean) : 0.f;
          const float d1 = in_row ? __builtin_fabsf(hi_f32(h[v][j]) - mean) : 0.f;
          m = mx(m, mx(d0, d1));
        }
      m = row_reduce<W>(m, mx, red_max, wave, slot);
      const int k = (__builtin_isfinite(var) && !(var < var_floor)) ? 0 : scale_exp(m);
      float sq2 = 0.f;
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        float part_sq = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d0 = __builtin_ldexpf(lo_f32(h[v][j]) - mean, -k);
          const float d1 = __builtin_ldexpf(hi_f32(h[v][j]) - mean, -k);
          part_sq = __builtin_fmaf(d0, d0, part_sq);
          part_sq = __builtin_fmaf(d1, d1, part_sq);
        }
        sq2 += (base / 16u + (uint32_t)(v * kWaveSize) < a.nvec) ? part_sq : 0.f;
      }
      float var2 = row_reduce<W>(sq2, Add{}, red_sq, wave, slot) * inv_d;
      var2 = var2 < 0.f ? 0.f : var2;
      const float den = __builtin_ldexpf(a.eps, -2 * k) + var2;
      if (k != 0 && __builtin_isfinite(den)) rstd = __builtin_ldexpf(__builtin_amdgcn_rsqf(den), -k);
    }
    [[maybe_unused]] const float nlo = mean_err * (inv_d * rstd);

    // weight / bias of vector v: from registers, or (staged in LDS) read into
    // wl / bl by read_lds(v) before the vector's outputs are computed
    [[maybe_unused]] AffineRow<OP::aff32, 1> wl, bl;
    auto read_lds = [&](int v) {
      if constexpr (kLds) {
#pragma unroll
        for (int q = 0; q < F; ++q) {
          wl.v[0][q] = aff_lds[(v * F + q) * kWaveSize + lane];
          if constexpr (OP::has_b) bl.v[0][q] = aff_lds[((VPT + v) * F + q) * kWaveSize + lane];
        }
      }
    };
    auto wval = [&](int v, int j, int k) -> float {
      if constexpr (kLds) return k ? wl.hi(0, j) : wl.lo(0, j);
      else return k ? wv.hi(v, j) : wv.lo(v, j);
    };
    auto bval = [&](int v, int j, int k) -> float {
      if constexpr (kLds) return k ? bl.hi(0, j) : bl.lo(0, j);
      else return k ? bv.hi(v, j) : bv.lo(v, j);
    };
    // t for element 2j (k = 0) or 2j+1 (k = 1) of vector v
    auto tval = [&](int v, int j, int k) -> float {
      const float hv = k ? hi_f32(h[v][j]) : lo_f32(h[v][j]);
      float n;
      if constexpr (OP::rms) n = hv * rstd;
      else n = __builtin_fmaf(hv - mean, rstd, nlo);
      if constexpr (OP::has_w && OP::has_b) {
        n = __builtin_fmaf(n, wval(v, j, k), bval(v, j, k));
      } else if constexpr (OP::has_w) {
        n *= wval(v, j, k);
      }
      const float s = k ? hi_f32(sc[v][j]) : lo_f32(sc[v][j]);
      const float t = k ? hi_f32(sh[v][j]) : lo_f32(sh[v][j]);
      return __builtin_fmaf(n, 1.0f + s, t);
    };

    // ---- epilogue from the register cache ----
    if constexpr (OP::out == kOutBf16) {
      {
        const auto rs_y = row_rsrc((const char*)a.y + p.off, p.bytes);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
          read_lds(v);
          u32x4 o;
#pragma unroll
          for (int j = 0; j < 4; ++j) o[j] = pack_bf16(tval(v, j, 0), tval(v, j, 1));
          store16<kPolicyStream, PS>(o, rs_y, base + v * 1024u);
        }
      }
    } else if constexpr (OP::out == kOutF32) {
      {
        // binary32 y: 32 bytes per lane per vector, two 16-byte stores
        const auto rs_y = row_rsrc((const char*)a.y + (uint64_t)p.r * (a.d * 4u), p.live ? a.d * 4u : 0u);
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
          read_lds(v);
          u32x4 o0, o1;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            o0[2 * j] = __float_as_uint(tval(v, j, 0));
            o0[2 * j + 1] = __float_as_uint(tval(v, j, 1));
            o1[2 * j] = __float_as_uint(tval(v, j + 2, 0));
            o1[2 * j + 1] = __float_as_uint(tval(v, j + 2, 1));
          }
          // each store covers every other 16-byte chunk of a 2 KB span; the
          // default policy lets L2 merge the pair into whole lines
          store16<kPolicyDefault, PS>(o0, rs_y, base * 2u + v * 2048u);
          store16<kPolicyDefault, PS>(o1, rs_y, base * 2u + v * 2048u + 16u);
        }
      }
    } else {
      // FP8 E4M3 y with a per-row scale: the row maximum of |t| first (lanes
      // past a ragged row's end are left out), then t * 448 / max converted.
      float amax = 0.f;
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        read_lds(v);
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(tval(v, j, 0)),
                                                 __builtin_fabsf(tval(v, j, 1))));
        amax = (base / 16u + (uint32_t)(v * kWaveSize) < a.nvec) ? __builtin_fmaxf(amax, m) : amax;
      }
      amax = row_reduce<W>(amax, Max{}, red_max, wave, slot);
      const float inv = amax > 0.f ? 448.0f / amax : 0.f;
      const auto rs_y = row_rsrc((const char*)a.y + (uint64_t)p.r * a.d, p.live ? a.d : 0u);
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        read_lds(v);
        uint32_t w0 = 0, w1 = 0;
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(tval(v, 0, 0) * inv, tval(v, 0, 1) * inv, w0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(tval(v, 1, 0) * inv, tval(v, 1, 1) * inv, w0, true);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(tval(v, 2, 0) * inv, tval(v, 2, 1) * inv, w1, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(tval(v, 3, 0) * inv, tval(v, 3, 1) * inv, w1, true);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64((u32x2){w0, w1}, rs_y, base / 2u + v * 512u, 0,
                                              kPolicyStream);
        pace<PS>();
      }
      if (p.live && part == 0 && lane == 0) a.y_scale[p.r] = amax / 448.0f;
    }
  };

  if constexpr (K == 1) {
    // With one wave per row, a wave issues its loads at raised priority, so
    // that the SIMD's other wave (busy with arithmetic or stores) does not
    // delay them: measured ~1 % on the norm-only op, neutral on the fused one.
    // Not with several waves per row: there it delays the row's other waves
    // at the barriers (-12 % measured with binary32 weight/bias).
    if constexpr (W == 1) __builtin_amdgcn_s_setprio(3);
    if constexpr (kLds) {
      fill_affine_lds<OP, VPT, RPB>(a, aff_lds, wave, lane);
      load_gate();
      load_ss_any();
      load_rows(p0);
    } else if constexpr (W == 10) {
      load_rows(p0);
      load_gate();
      load_affine();
      load_ss_any();
    } else if constexpr (OP::has_w) {
      load_ss_any();
      load_rows(p0);
      load_gate();
      load_affine();
    } else {
      load_gate();
      load_ss_any();
      load_rows(p0);
    }
    if constexpr (W == 1) __builtin_amdgcn_s_setprio(0);
    if constexpr (kLds) {
      // Every wave's LDS fill must have landed before any wave reads LDS.
      // The fills were issued first and vmcnt counts loads in issue order,
      // so waiting until no more than the loads issued after them (gate,
      // scale/shift, x, residual) are outstanding covers exactly the fills
      // and leaves the row's own loads in flight.  No store has been issued
      // yet.  The barrier then makes every wave's fill visible to all.
      constexpr int kAfterFills = (OP::gate ? VPT : 0) + 2 * VPT + 2 * VPT;
      vmcnt_wait<(kAfterFills < kVmcntMax ? kAfterFills : kVmcntMax)>();
      __syncthreads();
    }
    process(p0, 0);
  } else {
    // K consecutive rows share the slot's modulation rows and the affine
    // rows: those are loaded once, then each row streams its own operands
    // through them.
    if constexpr (W == 1) __builtin_amdgcn_s_setprio(3);
    load_ss_any();
    load_gate();
    load_affine();
    if constexpr (W == 1) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const RowPos p = at(first + (uint32_t)k);
      if constexpr (W == 1) {
        if (!p.live) break;
      }
      if constexpr (W == 1) __builtin_amdgcn_s_setprio(3);
      load_rows(p);
      if constexpr (W == 1) __builtin_amdgcn_s_setprio(0);
      process(p, (uint32_t)(k & (NBUF - 1)));
    }
  }
}

// Whether a shape is compiled for an operation: multi-row shapes only for
// the norm-only op with weight, the one the planner gives them to.
template <class OP, int SHAPE>
constexpr bool compiled() {
  return kShapes[SHAPE].k == 1 || (!OP::fused && OP::has_w);
}

// Table of one operation over every compiled shape.
template <class OP>
KernelFn kernel_for_shape(int shape) {
  switch (shape) {
#define RN_CASE(i)                      \
  case i:                               \
    if constexpr (compiled<OP, i>())    \
      return row_kernel<OP, i>;         \
    else                                \
      return nullptr;
    RN_CASE(0) RN_CASE(1) RN_CASE(2) RN_CASE(3) RN_CASE(4) RN_CASE(5) RN_CASE(6) RN_CASE(7)
    RN_CASE(8) RN_CASE(9) RN_CASE(10) RN_CASE(11) RN_CASE(12) RN_CASE(13) RN_CASE(14)
    RN_CASE(15) RN_CASE(16) RN_CASE(17) RN_CASE(18) RN_CASE(19) RN_CASE(20) RN_CASE(21)
    RN_CASE(22) RN_CASE(23) RN_CASE(24) RN_CASE(25) RN_CASE(26) RN_CASE(27) RN_CASE(28)
    RN_CASE(29) RN_CASE(30) RN_CASE(31) RN_CASE(32) RN_CASE(33) RN_CASE(34)
    RN_CASE(35) RN_CASE(36)
#undef RN_CASE
    default:
      return nullptr;
  }
}

static_assert(kNumShapes == 37, "kernel_for_shape lists every shape");

// Table of one (norm, op, gate, output) family over the affine variants.
template <bool RMS, bool FUSED, bool GATE, int OUT>
KernelFn kernel_for(int aff, int shape) {
  switch (aff) {
    case kAffNone: return kernel_for_shape<Op<RMS, FUSED, GATE, kAffNone, OUT>>(shape);
    case kAffW16: return kernel_for_shape<Op<RMS, FUSED, GATE, kAffW16, OUT>>(shape);
    case kAffWB16: return kernel_for_shape<Op<RMS, FUSED, GATE, kAffWB16, OUT>>(shape);
    case kAffW32: return kernel_for_shape<Op<RMS, FUSED, GATE, kAffW32, OUT>>(shape);
    case kAffWB32: return kernel_for_shape<Op<RMS, FUSED, GATE, kAffWB32, OUT>>(shape);
    default: return nullptr;
  }
}

}  // namespace rn
