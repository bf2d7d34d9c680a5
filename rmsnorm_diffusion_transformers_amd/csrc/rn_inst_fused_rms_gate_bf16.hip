// Compiled kernels: fused residual RMSNorm with gate, bf16 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_fused_rms_gate_bf16(int aff, int shape) {
  return kernel_for<true, true, true, kOutBf16>(aff, shape);
}

}  // namespace rn
