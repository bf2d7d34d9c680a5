// Compiled kernels: norm-only LayerNorm, bf16 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_nss_ln_bf16(int aff, int shape) {
  return kernel_for<false, false, false, kOutBf16>(aff, shape);
}

}  // namespace rn
