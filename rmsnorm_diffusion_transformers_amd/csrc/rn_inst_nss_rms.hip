// Compiled specialisations: nss rms (every affine / compiled shape).
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn nss_rms_kernel(int aff, int shape) {
  if (aff == kAffNone) return kernel_for_shape<true, false, false, kAffNone>(shape);
  if (aff == kAffWeight) return kernel_for_shape<true, false, false, kAffWeight>(shape);
  if (aff == kAffWeightBias) return kernel_for_shape<true, false, false, kAffWeightBias>(shape);
  return nullptr;
}

}  // namespace rn
