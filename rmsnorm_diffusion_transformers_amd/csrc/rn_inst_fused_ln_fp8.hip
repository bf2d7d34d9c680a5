// Compiled kernels: fused residual LayerNorm, FP8 E4M3 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_fused_ln_fp8(int aff, int shape) {
  return kernel_for<false, true, false, kOutFp8>(aff, shape);
}

}  // namespace rn
