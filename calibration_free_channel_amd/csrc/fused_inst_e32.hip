// Instances of the single-launch forward kernels for EPT = 32 (hidden width
// 8192).
#include "fused_kernels.h"

namespace cfm {

const void* fused_kernel_e32(bool select, bool recx, bool env) {
  if (!select) return env ? reinterpret_cast<const void*>(&k_dense_fused<32, true>)
                          : reinterpret_cast<const void*>(&k_dense_fused<32, false>);
  if (recx) return env ? reinterpret_cast<const void*>(&k_select_fused<32, true, true>)
                       : reinterpret_cast<const void*>(&k_select_fused<32, true, false>);
  return env ? reinterpret_cast<const void*>(&k_select_fused<32, false, true>)
             : reinterpret_cast<const void*>(&k_select_fused<32, false, false>);
}

}  // namespace cfm
