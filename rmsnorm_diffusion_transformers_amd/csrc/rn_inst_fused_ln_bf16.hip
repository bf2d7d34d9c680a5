// Compiled kernels: fused residual LayerNorm, bf16 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_fused_ln_bf16(int aff, int shape) {
  return kernel_for<false, true, false, kOutBf16>(aff, shape);
}

}  // namespace rn
