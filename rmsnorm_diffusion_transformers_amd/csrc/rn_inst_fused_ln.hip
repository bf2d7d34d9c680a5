// Compiled specialisations: fused ln (every gate / affine / register-cache width).
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn fused_ln_kernel(bool gate, int aff, int vec_index) {
  if (gate) {
    if (aff == kAffNone) return kernel_for_width<false, true, true, kAffNone>(vec_index);
    if (aff == kAffWeight) return kernel_for_width<false, true, true, kAffWeight>(vec_index);
    if (aff == kAffWeightBias) return kernel_for_width<false, true, true, kAffWeightBias>(vec_index);
  } else {
    if (aff == kAffNone) return kernel_for_width<false, true, false, kAffNone>(vec_index);
    if (aff == kAffWeight) return kernel_for_width<false, true, false, kAffWeight>(vec_index);
    if (aff == kAffWeightBias) return kernel_for_width<false, true, false, kAffWeightBias>(vec_index);
  }
  return nullptr;
}

}  // namespace rn
