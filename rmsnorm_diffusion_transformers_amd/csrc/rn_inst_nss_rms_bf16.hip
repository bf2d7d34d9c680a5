// Compiled kernels: norm-only RMSNorm, bf16 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_nss_rms_bf16(int aff, int shape) {
  return kernel_for<true, false, false, kOutBf16>(aff, shape);
}

}  // namespace rn
