// Compiled specialisations: nss ln (every affine / compiled shape).
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn nss_ln_kernel(int aff, int shape) {
  if (aff == kAffNone) return kernel_for_shape<false, false, false, kAffNone>(shape);
  if (aff == kAffWeight) return kernel_for_shape<false, false, false, kAffWeight>(shape);
  if (aff == kAffWeightBias) return kernel_for_shape<false, false, false, kAffWeightBias>(shape);
  return nullptr;
}

}  // namespace rn
