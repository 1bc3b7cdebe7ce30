"""StateKV streaming video prefill on MI355X (gfx950).

The compute path is libstatekv.so: hand-written HIP kernels behind a C ABI
(include/statekv.h).  This package holds the ctypes binding with the same
entry-point names (``_binding``), a torch-facing ``Layer`` wrapper and the
build script.  Importing it loads the library and fails if it is missing.
"""

from ._binding import (  # noqa: F401
    STATEKV_FLAG_C_IN_D,
    STATEKV_FLAG_D_RING,
    STATEKV_FLAG_NONCAUSAL_FRAME,
    STATEKV_FLAG_SELECT_RECENT,
    STATEKV_FLAG_SELECT_SHARED,
    STATEKV_FLAG_SLOT_STABLE,
    STATEKV_FLAG_OUT_BF16,
    STATEKV_KERNELS,
    StateKVError,
    load_library,
    make_config,
    statekv_attention_mass,
    statekv_decode_attention,
    statekv_decode_attention_noalloc,
    statekv_detailed_cache,
    statekv_free_layer,
    statekv_full_attention_frame,
    statekv_init_layer,
    statekv_mass_set_words,
    statekv_launch_plan_for,
    statekv_prefill_frame,
    statekv_profile_start,
    statekv_profile_stop,
    statekv_qkv_rope,
    statekv_qkv_rope_workspace_size,
    statekv_reset_layer,
    statekv_restore_layer,
    statekv_rope,
    statekv_select_topb,
    statekv_state,
    statekv_status_string,
    statekv_workspace_bytes,
)
from .layer import Layer, qkv_rope, qkv_rope_workspace_bytes, select_topb  # noqa: F401

load_library()
