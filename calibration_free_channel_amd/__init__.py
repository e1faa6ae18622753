"""Channel-selected routed-expert SwiGLU FFN for MoE decoding on MI355X (gfx950).

The computation lives in libcfm.so (hand-written HIP, C ABI in include/cfm.h);
this package is its ctypes binding. Importing it without the built library
raises ImportError: there is no CPU fallback.
"""
from ._lib import (  # noqa: F401
    FORWARD_AUTO, FORWARD_GROUPED, FORWARD_PER_PAIR, FORWARD_PER_PAIR_GENERAL, FORWARD_PER_PAIR_SINGLE,
    RECOVER_CANDIDATES_EXACT, RECOVER_SKETCH, CfmError,
    EXPORTED, STATS_BYTES, decode_stats,
    dense_workspace, forward_path, last_error, lowrank_build, lowrank_workspace, moe_dense_forward,
    moe_layer_dense_forward, moe_layer_forward,
    moe_select_forward, moe_select_forward_noalloc, moe_select_forward_threshold, new_workspace, phase_trace, select_workspace,
    set_forward_path, set_resident_limit, set_wait_limit, workspace_status,
    rotation_signs, sketch_build, sketch_build_seeded, sketch_bytes, timing_enable,
    timing_report, version,
)
