// Compiled specialisations: fused rms (every gate / affine / compiled shape).
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn fused_rms_kernel(bool gate, int aff, int shape) {
  if (gate) {
    if (aff == kAffNone) return kernel_for_shape<true, true, true, kAffNone>(shape);
    if (aff == kAffWeight) return kernel_for_shape<true, true, true, kAffWeight>(shape);
    if (aff == kAffWeightBias) return kernel_for_shape<true, true, true, kAffWeightBias>(shape);
  } else {
    if (aff == kAffNone) return kernel_for_shape<true, true, false, kAffNone>(shape);
    if (aff == kAffWeight) return kernel_for_shape<true, true, false, kAffWeight>(shape);
    if (aff == kAffWeightBias) return kernel_for_shape<true, true, false, kAffWeightBias>(shape);
  }
  return nullptr;
}

}  // namespace rn
