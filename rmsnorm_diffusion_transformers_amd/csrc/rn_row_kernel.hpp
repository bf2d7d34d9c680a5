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
//   * W wave64s own one activation row and a workgroup holds RPB rows
//     (W * RPB waves).  Row indices are wave-uniform, so per-row quantities
//     (descriptors, modulation row, statistics) live in SGPRs.
//   * Every global access is a 128-bit buffer load/store (8 bf16 per lane) on
//     a per-row buffer descriptor whose range is exactly the row: lanes past
//     the end of a ragged row read zeros and their stores are dropped by the
//     hardware range check.
//   * All loads of a row -- x, residual, gate, weight, bias, scale, shift --
//     are issued before its first store.  Loads and stores share the in-order
//     vmcnt counter on gfx9, so a load issued after a store could only be
//     waited for together with that store; issuing every load first keeps the
//     store latency off the critical path.
//   * Loads are issued PL x 8 cycles apart and stores PS x 8 cycles apart
//     (s_nop): measured on MI355X, back-to-back bursts of 128-bit stores from
//     every wave stream several percent slower than lightly spaced ones.
//   * Streamed tensors (x, residual in; y, residual_out out) use the
//     non-temporal policy; modulation rows use the default policy, so the
//     broadcast and per-frame rows stay resident in L2.
//   * The row stays in VGPRs (bf16-packed) between the statistics and the
//     epilogue, so HBM sees each byte once.
//   * Statistics in fp32.  LayerNorm: the mean, then the centred sum of squares
//     over the register-resident row.  RMSNorm: the sum of squares.  Wave
//     reductions are DPP (xor 1, xor 2, half-row mirror, row mirror) then the
//     gfx950 permlane16/permlane32 swaps; with W > 1 the per-wave totals are
//     combined through LDS in a fixed order.  Every lane and every wave of a
//     row ends with the bit-identical total.
//   * fp32 -> bf16 with v_cvt_pk_bf16_f32 (round to nearest even; fp32
//     denormals are kept in these kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Sum over the 64 lanes of a wave; every lane returns the same bits.  Each
// step adds a lane's value to its partner's in an order that is the same on
// both partners, so the result is identical across lanes.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: partner lane ^ 1
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: partner lane ^ 2
  v += dpp<0x141>(v);  // row_half_mirror: the other quad of the 8-lane group
  v += dpp<0x140>(v);  // row_mirror: the other 8-lane half of the 16-lane row
  {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);  // rows 2k and 2k+1
  }
  {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);  // lanes 0-31 and 32-63
  }
  return v;
}

// Total over the W waves of one row.  Each wave's total goes to LDS; after the
// barrier every wave of the row adds the W partials in the same order.
template <int W>
__device__ __forceinline__ float row_sum(float v, float* red, uint32_t wave, uint32_t slot) {
  v = wave_sum(v);
  if constexpr (W > 1) {
    if ((threadIdx.x & (kWaveSize - 1)) == 0) red[wave] = v;
    __syncthreads();
    v = red[slot * W];
#pragma unroll
    for (int p = 1; p < W; ++p) v += red[slot * W + p];
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

template <bool RMS, bool FUSED, bool GATE, int AFF, int VPT, int W, int RPB, int PL, int PS>
__global__ __launch_bounds__(kWaveSize * W * RPB) void row_kernel(const RowArgs a) {
  static_assert(W * RPB * kWaveSize <= 1024, "workgroup size");
  constexpr int kRowsPerBlock = RPB;
  [[maybe_unused]] __shared__ float red_sum[W * RPB];
  [[maybe_unused]] __shared__ float red_sq[W * RPB];

  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & (kWaveSize - 1);
  const uint32_t slot = wave / W;  // row slot in the workgroup
  const uint32_t part = wave % W;  // which contiguous part of the row this wave holds
  const uint32_t row = blockIdx.x * kRowsPerBlock + slot;
  // With W > 1 every wave must reach the barriers, so a wave past the last
  // row keeps going with its memory operations disabled (zero-range buffers).
  const bool live = row < a.rows;
  if constexpr (W == 1) {
    if (!live) return;
  }
  const uint32_t row_bytes = live ? a.d * 2u : 0u;
  const uint32_t r = live ? row : 0u;
  const uint64_t row_off = (uint64_t)r * (a.d * 2u);
  const uint32_t b = r / a.L;
  const uint32_t l = r - b * a.L;
  const uint32_t srow = mod_row(a.ss_kind, a.ss_frames, a.ss_tokens_per_frame, r, b, l);
  // lane-local byte offset of vector v: this wave's part, then 1 KB per vector
  const uint32_t base = (part * VPT * kWaveSize + lane) * 16u;

  const auto rs_x = row_rsrc((const char*)a.x + row_off, row_bytes);
  const auto rs_y = row_rsrc((const char*)a.y + row_off, row_bytes);
  const auto rs_sc = row_rsrc((const char*)a.scale + (uint64_t)srow * (a.d * 2u), row_bytes);
  const auto rs_sh = row_rsrc((const char*)a.shift + (uint64_t)srow * (a.d * 2u), row_bytes);

  // ---- every load of the row, before any store ----
  u32x4 h[VPT];  // x (norm-only) or residual, later the bf16-packed residual_out
  [[maybe_unused]] u32x4 xv[VPT];
  [[maybe_unused]] u32x4 gv[VPT];
  [[maybe_unused]] u32x4 wv[VPT];
  [[maybe_unused]] u32x4 bv[VPT];
  u32x4 sc[VPT], sh[VPT];
  if constexpr (FUSED) {
    const auto rs_r = row_rsrc((const char*)a.residual + row_off, row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) xv[v] = load16<kPolicyStream, PL>(rs_x, base + v * 1024u);
#pragma unroll
    for (int v = 0; v < VPT; ++v) h[v] = load16<kPolicyStream, PL>(rs_r, base + v * 1024u);
    if constexpr (GATE) {
      const uint32_t grow = mod_row(a.gate_kind, a.gate_frames, a.gate_tokens_per_frame, r, b, l);
      const auto rs_g = row_rsrc((const char*)a.gate + (uint64_t)grow * (a.d * 2u), row_bytes);
#pragma unroll
      for (int v = 0; v < VPT; ++v) gv[v] = load16<kPolicyDefault, PL>(rs_g, base + v * 1024u);
    }
  } else {
#pragma unroll
    for (int v = 0; v < VPT; ++v) h[v] = load16<kPolicyStream, PL>(rs_x, base + v * 1024u);
  }
  if constexpr (AFF >= kAffWeight) {
    const auto rs_w = row_rsrc(a.weight, row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) wv[v] = load16<kPolicyDefault, PL>(rs_w, base + v * 1024u);
  }
  if constexpr (AFF >= kAffWeightBias) {
    const auto rs_b = row_rsrc(a.bias, row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) bv[v] = load16<kPolicyDefault, PL>(rs_b, base + v * 1024u);
  }
  // per-row scale/shift stream like the activations; shared rows stay cached
  if (a.ss_kind == 1) {
#pragma unroll
    for (int v = 0; v < VPT; ++v) sc[v] = load16<kPolicyStream, PL>(rs_sc, base + v * 1024u);
#pragma unroll
    for (int v = 0; v < VPT; ++v) sh[v] = load16<kPolicyStream, PL>(rs_sh, base + v * 1024u);
  } else {
#pragma unroll
    for (int v = 0; v < VPT; ++v) sc[v] = load16<kPolicyDefault, PL>(rs_sc, base + v * 1024u);
#pragma unroll
    for (int v = 0; v < VPT; ++v) sh[v] = load16<kPolicyDefault, PL>(rs_sh, base + v * 1024u);
  }

  // ---- residual update (fused) ----
  if constexpr (FUSED) {
    const auto rs_ro = row_rsrc((const char*)a.residual_out + row_off, row_bytes);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float s0, s1;
        if constexpr (GATE) {
          // gate * x is exact in binary32 (8-bit x 8-bit significands), so the
          // fused multiply-add rounds exactly once, like residual + (gate * x).
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
  float sq = 0.f;
  if constexpr (!RMS) {
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) sum += lo_f32(h[v][j]) + hi_f32(h[v][j]);
    mean = row_sum<W>(sum, red_sum, wave, slot) / (float)a.d;
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
  float var = row_sum<W>(sq, red_sq, wave, slot) * inv_d;
  var = var > 0.f ? var : 0.f;
  const float rstd = __builtin_amdgcn_rsqf(var + a.eps);

  // ---- epilogue from the register cache ----
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float n0 = (lo_f32(h[v][j]) - mean) * rstd;
      float n1 = (hi_f32(h[v][j]) - mean) * rstd;
      if constexpr (AFF == kAffWeight) {
        n0 *= lo_f32(wv[v][j]);
        n1 *= hi_f32(wv[v][j]);
      } else if constexpr (AFF == kAffWeightBias) {
        n0 = __builtin_fmaf(n0, lo_f32(wv[v][j]), lo_f32(bv[v][j]));
        n1 = __builtin_fmaf(n1, hi_f32(wv[v][j]), hi_f32(bv[v][j]));
      }
      const float t0 = __builtin_fmaf(n0, 1.0f + lo_f32(sc[v][j]), lo_f32(sh[v][j]));
      const float t1 = __builtin_fmaf(n1, 1.0f + hi_f32(sc[v][j]), hi_f32(sh[v][j]));
      o[j] = pack_bf16(t0, t1);
    }
    store16<kPolicyStream, PS>(o, rs_y, base + v * 1024u);
  }
}

// Table of one flag combination over every compiled shape.
template <bool RMS, bool FUSED, bool GATE, int AFF>
KernelFn kernel_for_shape(int shape) {
  switch (shape) {
#define RN_CASE(i) \
  case i:          \
    return row_kernel<RMS, FUSED, GATE, AFF, kShapes[i].vpt, kShapes[i].w, kShapes[i].rpb, \
                      kPaceLoads, kPaceStores>;
    RN_CASE(0) RN_CASE(1) RN_CASE(2) RN_CASE(3) RN_CASE(4) RN_CASE(5) RN_CASE(6) RN_CASE(7)
    RN_CASE(8) RN_CASE(9) RN_CASE(10) RN_CASE(11) RN_CASE(12) RN_CASE(13) RN_CASE(14)
    RN_CASE(15) RN_CASE(16) RN_CASE(17) RN_CASE(18)
#undef RN_CASE
    default:
      return nullptr;
  }
}

static_assert(kNumShapes == 19, "kernel_for_shape lists every shape");

}  // namespace rn
