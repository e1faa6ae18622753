// Instances of the single-launch forward kernels for EPT = 16 (hidden width
// 4096).
#include "fused_kernels.h"

namespace cfm {

const void* fused_kernel_e16(bool select, bool recx, bool env) {
  if (!select) return env ? reinterpret_cast<const void*>(&k_dense_fused<16, true>)
                          : reinterpret_cast<const void*>(&k_dense_fused<16, false>);
  if (recx) return env ? reinterpret_cast<const void*>(&k_select_fused<16, true, true>)
                       : reinterpret_cast<const void*>(&k_select_fused<16, true, false>);
  return env ? reinterpret_cast<const void*>(&k_select_fused<16, false, true>)
             : reinterpret_cast<const void*>(&k_select_fused<16, false, false>);
}

}  // namespace cfm
