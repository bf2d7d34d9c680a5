// Compiled specialisations: nss ln (every affine / register-cache width).
#include "rn_row_kernel.hpp"

namespace rn {

KernelFn nss_ln_kernel(int aff, int vec_index) {
  if (aff == kAffNone) return kernel_for_width<false, false, false, kAffNone>(vec_index);
  if (aff == kAffWeight) return kernel_for_width<false, false, false, kAffWeight>(vec_index);
  if (aff == kAffWeightBias) return kernel_for_width<false, false, false, kAffWeightBias>(vec_index);
  return nullptr;
}

}  // namespace rn
