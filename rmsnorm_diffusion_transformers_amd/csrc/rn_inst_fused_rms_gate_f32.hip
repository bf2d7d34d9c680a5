// Compiled kernels: fused residual RMSNorm with gate, binary32 output, every affine variant and shape.
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn kernels_fused_rms_gate_f32(int aff, int shape) {
  return kernel_for<true, true, true, kOutF32>(aff, shape);
}

}  // namespace rn
