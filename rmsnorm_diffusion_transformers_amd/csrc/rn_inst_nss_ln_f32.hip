// Compiled kernels: norm-only LayerNorm, binary32 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_nss_ln_f32(int aff, int shape) {
  return kernel_for<false, false, false, kOutF32>(aff, shape);
}

}  // namespace rn
