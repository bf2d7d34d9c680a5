// Compiled kernels: fused residual RMSNorm, binary32 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_fused_rms_f32(int aff, int shape) {
  return kernel_for<true, true, false, kOutF32>(aff, shape);
}

}  // namespace rn
