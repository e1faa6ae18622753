// Instances of the single-launch forward kernels for EPT = 8 (hidden width
// 2048).
#include "fused_kernels.h"

namespace cfm {

// The lean instance of the plain method at this width: 8 output chunks per
// workgroup (one pair per XCD, 32 workgroups each), rank 64, at most 160 kept
// channels (5 per group of 8 threads).
const void* fused_kernel_e8_lean() {
  return reinterpret_cast<const void*>(&k_select_fused<8, false, false, 8, 8, 5>);
}

const void* fused_kernel_e8(bool select, bool recx, bool env) {
  if (!select) return env ? reinterpret_cast<const void*>(&k_dense_fused<8, true>)
                          : reinterpret_cast<const void*>(&k_dense_fused<8, false>);
  if (recx) return env ? reinterpret_cast<const void*>(&k_select_fused<8, true, true>)
                       : reinterpret_cast<const void*>(&k_select_fused<8, true, false>);
  return env ? reinterpret_cast<const void*>(&k_select_fused<8, false, true>)
             : reinterpret_cast<const void*>(&k_select_fused<8, false, false>);
}


// The prescreened instances (several tokens per launch, screen run before it).
const void* fused_kernel_e8_ps(bool recx) {
  return recx ? reinterpret_cast<const void*>(&k_select_fused<8, true, false, 0, 0, 1, true>)
              : reinterpret_cast<const void*>(&k_select_fused<8, false, false, 0, 0, 1, true>);
}

// The multi-sub-chunk instance of the plain method (several sub-chunks of
// channels per workgroup, screen inside the launch).
const void* fused_kernel_e8_ms() {
  return reinterpret_cast<const void*>(&k_select_fused<8, false, false, 0, 0, 1, false, true>);
}

}  // namespace cfm
