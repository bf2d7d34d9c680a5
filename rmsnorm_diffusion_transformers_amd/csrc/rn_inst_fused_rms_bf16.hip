// Compiled kernels: fused residual RMSNorm, bf16 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_fused_rms_bf16(int aff, int shape) {
  return kernel_for<true, true, false, kOutBf16>(aff, shape);
}

}  // namespace rn
