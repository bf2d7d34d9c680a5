// rn_dispatch.hip -- maps an operation to its compiled kernel table.
#include "rn_args.h"

namespace rn {

KernelFn kernels_fused_ln_bf16(int aff, int shape);
KernelFn kernels_fused_ln_f32(int aff, int shape);
KernelFn kernels_fused_ln_fp8(int aff, int shape);
KernelFn kernels_fused_ln_gate_bf16(int aff, int shape);
KernelFn kernels_fused_ln_gate_f32(int aff, int shape);
KernelFn kernels_fused_ln_gate_fp8(int aff, int shape);
KernelFn kernels_fused_rms_bf16(int aff, int shape);
KernelFn kernels_fused_rms_f32(int aff, int shape);
KernelFn kernels_fused_rms_fp8(int aff, int shape);
KernelFn kernels_fused_rms_gate_bf16(int aff, int shape);
KernelFn kernels_fused_rms_gate_f32(int aff, int shape);
KernelFn kernels_fused_rms_gate_fp8(int aff, int shape);
KernelFn kernels_nss_ln_bf16(int aff, int shape);
KernelFn kernels_nss_ln_f32(int aff, int shape);
KernelFn kernels_nss_ln_fp8(int aff, int shape);
KernelFn kernels_nss_rms_bf16(int aff, int shape);
KernelFn kernels_nss_rms_f32(int aff, int shape);
KernelFn kernels_nss_rms_fp8(int aff, int shape);

KernelFn fused_kernel(bool rms, int out, bool gate, int aff, int shape) {
  if (!rms && !gate) return out == kOutFp8 ? kernels_fused_ln_fp8(aff, shape) : out == kOutF32 ? kernels_fused_ln_f32(aff, shape) : kernels_fused_ln_bf16(aff, shape);
  if (!rms && gate) return out == kOutFp8 ? kernels_fused_ln_gate_fp8(aff, shape) : out == kOutF32 ? kernels_fused_ln_gate_f32(aff, shape) : kernels_fused_ln_gate_bf16(aff, shape);
  if (rms && !gate) return out == kOutFp8 ? kernels_fused_rms_fp8(aff, shape) : out == kOutF32 ? kernels_fused_rms_f32(aff, shape) : kernels_fused_rms_bf16(aff, shape);
  return out == kOutFp8 ? kernels_fused_rms_gate_fp8(aff, shape) : out == kOutF32 ? kernels_fused_rms_gate_f32(aff, shape) : kernels_fused_rms_gate_bf16(aff, shape);
}

KernelFn nss_kernel(bool rms, int out, int aff, int shape) {
  if (!rms) return out == kOutFp8 ? kernels_nss_ln_fp8(aff, shape) : out == kOutF32 ? kernels_nss_ln_f32(aff, shape) : kernels_nss_ln_bf16(aff, shape);
  return out == kOutFp8 ? kernels_nss_rms_fp8(aff, shape) : out == kOutF32 ? kernels_nss_rms_f32(aff, shape) : kernels_nss_rms_bf16(aff, shape);
}

}  // namespace rn
