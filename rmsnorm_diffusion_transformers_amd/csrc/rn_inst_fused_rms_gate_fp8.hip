// Compiled kernels: fused residual RMSNorm with gate, FP8 E4M3 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_fused_rms_gate_fp8(int aff, int shape) {
  return kernel_for<true, true, true, kOutFp8>(aff, shape);
}

}  // namespace rn
