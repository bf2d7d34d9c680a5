// Compiled kernels: norm-only RMSNorm, binary32 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_nss_rms_f32(int aff, int shape) {
  return kernel_for<true, false, false, kOutF32>(aff, shape);
}

}  // namespace rn
