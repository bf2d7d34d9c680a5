// Compiled kernels: fused residual LayerNorm, binary32 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_fused_ln_f32(int aff, int shape) {
  return kernel_for<false, true, false, kOutF32>(aff, shape);
}

}  // namespace rn
