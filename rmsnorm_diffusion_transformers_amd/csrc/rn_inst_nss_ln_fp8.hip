// Compiled kernels: norm-only LayerNorm, FP8 E4M3 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_nss_ln_fp8(int aff, int shape) {
  return kernel_for<false, false, false, kOutFp8>(aff, shape);
}

}  // namespace rn
