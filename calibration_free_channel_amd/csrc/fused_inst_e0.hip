// Instances of the single-launch forward kernels for EPT = 0 (hidden width
// below 1024 except 512).
#include "fused_kernels.h"

namespace cfm {

const void* fused_kernel_e0(bool select, bool recx, bool env) {
  if (!select) return env ? reinterpret_cast<const void*>(&k_dense_fused<0, true>)
                          : reinterpret_cast<const void*>(&k_dense_fused<0, false>);
  if (recx) return env ? reinterpret_cast<const void*>(&k_select_fused<0, true, true>)
                       : reinterpret_cast<const void*>(&k_select_fused<0, true, false>);
  return env ? reinterpret_cast<const void*>(&k_select_fused<0, false, true>)
             : reinterpret_cast<const void*>(&k_select_fused<0, false, false>);
}


// The prescreened instances (several tokens per launch, screen run before it).
const void* fused_kernel_e0_ps(bool recx) {
  return recx ? reinterpret_cast<const void*>(&k_select_fused<0, true, false, 0, 0, 1, true>)
              : reinterpret_cast<const void*>(&k_select_fused<0, false, false, 0, 0, 1, true>);
}

// The multi-sub-chunk instance of the plain method (several sub-chunks of
// channels per workgroup, screen inside the launch).
const void* fused_kernel_e0_ms() {
  return reinterpret_cast<const void*>(&k_select_fused<0, false, false, 0, 0, 1, false, true>);
}

}  // namespace cfm
