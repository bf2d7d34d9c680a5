// rn_row_kernel.hpp -- gfx950 row kernel for the fused residual + gate +
// LayerNorm/RMSNorm + scale/shift operation and its norm-only variant.
//
// Design (bandwidth-bound; no matrix cores -- nothing here is a contraction):
//   * one wave64 per activation row, four rows per 256-thread workgroup; the
//     row index is wave-uniform, so every per-row quantity (base addresses,
//     modulation row, statistics) lives in scalar registers and the waves of a
//     workgroup never synchronise with each other;
//   * every global access is a 128-bit buffer load/store (8 bf16 per lane) on
//     a per-row buffer descriptor whose range is exactly the row, so lanes past
//     the end of a ragged row read zeros and their stores are dropped by the
//     hardware range check;
//   * the streamed tensors (x, residual in; y, residual_out out) use the
//     non-temporal cache policy; modulation rows (gate/scale/shift/weight/bias)
//     use the default policy so that broadcast and per-frame rows stay in L2;
//   * the whole row stays in VGPRs (bf16-packed) between the statistics and
//     the normalise/modulate epilogue, so HBM sees each byte once;
//   * statistics in fp32: LayerNorm takes the mean, then the centred sum of
//     squares over the register-resident row (two wave reductions); RMSNorm
//     takes the sum of squares.  Wave reductions are DPP (xor 1, xor 2, half
//     row mirror, row mirror) then the gfx950 permlane16/permlane32 swaps;
//     every lane ends with the bit-identical total;
//   * fp32 -> bf16 with v_cvt_pk_bf16_f32 (round to nearest even, denormals
//     kept -- fp32 denormal mode is IEEE in these kernels).
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

template <int POLICY>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
}

template <int POLICY>
__device__ __forceinline__ void store16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, POLICY);
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

// Modulation row for activation row `row` = b * L + l.
__device__ __forceinline__ uint32_t mod_row(int32_t kind, uint32_t frames, uint32_t tpf,
                                            uint32_t row, uint32_t b, uint32_t l) {
  if (kind == 0) return 0;
  if (kind == 1) return row;
  return b * frames + l / tpf;
}

template <bool RMS, bool FUSED, bool GATE, int AFF, int VPT>
__global__ __launch_bounds__(kBlockThreads) void row_kernel(const RowArgs a) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & (kWaveSize - 1);
  const uint32_t row = blockIdx.x * kWavesPerBlock + wave;
  if (row >= a.rows) return;  // whole wave

  const uint32_t row_bytes = a.d * 2u;
  const uint64_t row_off = (uint64_t)row * row_bytes;
  const uint32_t b = row / a.L;
  const uint32_t l = row - b * a.L;
  const uint32_t srow = mod_row(a.ss_kind, a.ss_frames, a.ss_tokens_per_frame, row, b, l);

  const auto rs_x = row_rsrc((const char*)a.x + row_off, row_bytes);
  const auto rs_y = row_rsrc((const char*)a.y + row_off, row_bytes);
  const auto rs_sc = row_rsrc((const char*)a.scale + (uint64_t)srow * row_bytes, row_bytes);
  const auto rs_sh = row_rsrc((const char*)a.shift + (uint64_t)srow * row_bytes, row_bytes);

  u32x4 h[VPT];   // the row, bf16-packed: residual_out (fused) or x (norm-only)
  float sum = 0.f;

  if constexpr (FUSED) {
    const auto rs_r = row_rsrc((const char*)a.residual + row_off, row_bytes);
    const auto rs_ro = row_rsrc((const char*)a.residual_out + row_off, row_bytes);
    u32x4 xv[VPT];
#pragma unroll
    for (int v = 0; v < VPT; ++v) xv[v] = load16<kPolicyStream>(rs_x, (v * kWaveSize + lane) * 16u);
#pragma unroll
    for (int v = 0; v < VPT; ++v) h[v] = load16<kPolicyStream>(rs_r, (v * kWaveSize + lane) * 16u);
    u32x4 gv[VPT];
    if constexpr (GATE) {
      const uint32_t grow = mod_row(a.gate_kind, a.gate_frames, a.gate_tokens_per_frame, row, b, l);
      const auto rs_g = row_rsrc((const char*)a.gate + (uint64_t)grow * row_bytes, row_bytes);
#pragma unroll
      for (int v = 0; v < VPT; ++v) gv[v] = load16<kPolicyDefault>(rs_g, (v * kWaveSize + lane) * 16u);
    }
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
      store16<kPolicyStream>(o, rs_ro, (v * kWaveSize + lane) * 16u);
      h[v] = o;
    }
  } else {
#pragma unroll
    for (int v = 0; v < VPT; ++v) h[v] = load16<kPolicyStream>(rs_x, (v * kWaveSize + lane) * 16u);
  }

  // ---- statistics (fp32) ----
  const float inv_d = 1.0f / (float)a.d;
  float mean = 0.f;
  float sq = 0.f;
  if constexpr (!RMS) {
#pragma unroll
    for (int v = 0; v < VPT; ++v)
#pragma unroll
      for (int j = 0; j < 4; ++j) sum += lo_f32(h[v][j]) + hi_f32(h[v][j]);
    mean = wave_sum(sum) / (float)a.d;
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d0 = lo_f32(h[v][j]) - mean;
        const float d1 = hi_f32(h[v][j]) - mean;
        part = __builtin_fmaf(d0, d0, part);
        part = __builtin_fmaf(d1, d1, part);
      }
      // lanes past the end of a ragged row hold zeros, which are not zero
      // after centring: leave them out.
      sq += ((uint32_t)(v * kWaveSize) + lane < a.nvec) ? part : 0.f;
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
  float var = wave_sum(sq) * inv_d;
  var = var > 0.f ? var : 0.f;
  const float rstd = __builtin_amdgcn_rsqf(var + a.eps);

  // ---- epilogue from the register cache ----
  [[maybe_unused]] __amdgpu_buffer_rsrc_t rs_w, rs_b;
  if constexpr (AFF >= kAffWeight) rs_w = row_rsrc(a.weight, row_bytes);
  if constexpr (AFF >= kAffWeightBias) rs_b = row_rsrc(a.bias, row_bytes);
#pragma unroll
  for (int v = 0; v < VPT; ++v) {
    const uint32_t off = (v * kWaveSize + lane) * 16u;
    const u32x4 sc = load16<kPolicyDefault>(rs_sc, off);
    const u32x4 sh = load16<kPolicyDefault>(rs_sh, off);
    [[maybe_unused]] u32x4 wv, bv;
    if constexpr (AFF >= kAffWeight) wv = load16<kPolicyDefault>(rs_w, off);
    if constexpr (AFF >= kAffWeightBias) bv = load16<kPolicyDefault>(rs_b, off);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float n0 = (lo_f32(h[v][j]) - mean) * rstd;
      float n1 = (hi_f32(h[v][j]) - mean) * rstd;
      if constexpr (AFF == kAffWeight) {
        n0 *= lo_f32(wv[j]);
        n1 *= hi_f32(wv[j]);
      } else if constexpr (AFF == kAffWeightBias) {
        n0 = __builtin_fmaf(n0, lo_f32(wv[j]), lo_f32(bv[j]));
        n1 = __builtin_fmaf(n1, hi_f32(wv[j]), hi_f32(bv[j]));
      }
      const float t0 = __builtin_fmaf(n0, 1.0f + lo_f32(sc[j]), lo_f32(sh[j]));
      const float t1 = __builtin_fmaf(n1, 1.0f + hi_f32(sc[j]), hi_f32(sh[j]));
      o[j] = pack_bf16(t0, t1);
    }
    store16<kPolicyStream>(o, rs_y, off);
  }
}

// Table of one flag combination over every compiled register-cache width.
template <bool RMS, bool FUSED, bool GATE, int AFF>
KernelFn kernel_for_width(int vec_index) {
  switch (vec_index) {
#define RN_CASE(i) \
  case i:          \
    return row_kernel<RMS, FUSED, GATE, AFF, kVecWidths[i]>;
    RN_CASE(0) RN_CASE(1) RN_CASE(2) RN_CASE(3) RN_CASE(4) RN_CASE(5) RN_CASE(6)
    RN_CASE(7) RN_CASE(8) RN_CASE(9) RN_CASE(10) RN_CASE(11) RN_CASE(12)
#undef RN_CASE
    default:
      return nullptr;
  }
}

static_assert(kNumVecWidths == 13, "kernel_for_width lists every width");

}  // namespace rn
