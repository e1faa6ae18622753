// Instances of the single-launch forward kernels for EPT = 4 (hidden width
// 1024).
#include "fused_kernels.h"

namespace cfm {

const void* fused_kernel_e4(bool select, bool recx, bool env) {
  if (!select) return env ? reinterpret_cast<const void*>(&k_dense_fused<4, true>)
                          : reinterpret_cast<const void*>(&k_dense_fused<4, false>);
  if (recx) return env ? reinterpret_cast<const void*>(&k_select_fused<4, true, true>)
                       : reinterpret_cast<const void*>(&k_select_fused<4, true, false>);
  return env ? reinterpret_cast<const void*>(&k_select_fused<4, false, true>)
             : reinterpret_cast<const void*>(&k_select_fused<4, false, false>);
}

}  // namespace cfm
