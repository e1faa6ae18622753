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


// The prescreened instances (several tokens per launch, screen run before it).
const void* fused_kernel_e4_ps(bool recx) {
  return recx ? reinterpret_cast<const void*>(&k_select_fused<4, true, false, 0, 0, 1, true>)
              : reinterpret_cast<const void*>(&k_select_fused<4, false, false, 0, 0, 1, true>);
}

// The multi-sub-chunk instance of the plain method (several sub-chunks of
// channels per workgroup, screen inside the launch).
const void* fused_kernel_e4_ms() {
  return reinterpret_cast<const void*>(&k_select_fused<4, false, false, 0, 0, 1, false, true>);
}

}  // namespace cfm
