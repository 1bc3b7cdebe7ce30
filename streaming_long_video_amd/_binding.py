"""ctypes binding of libstatekv.so: the C entry points under the same names.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of the library; there is no Python or CPU fallback, and loading fails
loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libstatekv.so")

STATEKV_OK = 0
STATEKV_ERR_INVALID_ARGUMENT = -1
STATEKV_ERR_UNSUPPORTED = -2
STATEKV_ERR_WORKSPACE = -3
STATEKV_ERR_CAPACITY = -4
STATEKV_ERR_HIP = -5

STATEKV_KERNELS = ("attn_stats", "attn_out", "split_sum", "select", "gather", "decode",
                   "rope", "mass")

STATEKV_FLAG_SELECT_SHARED = 1 << 0
STATEKV_FLAG_D_RING = 1 << 1
STATEKV_FLAG_NONCAUSAL_FRAME = 1 << 2
STATEKV_FLAG_C_IN_D = 1 << 3
STATEKV_FLAG_SELECT_RECENT = 1 << 4
STATEKV_FLAG_SLOT_STABLE = 1 << 5
STATEKV_FLAG_OUT_BF16 = 1 << 6


class StateKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {statekv_status_string(status)} ({status})")


class statekv_layer_config(ctypes.Structure):
    _fields_ = [
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("frame_tokens", ctypes.c_int32),
        ("state_budget", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("detailed_capacity", ctypes.c_int64),
        ("position_offset", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("rope_theta", ctypes.c_float),
        ("rope_scaling", ctypes.c_float),
    ]


class statekv_state_view(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("pos", ctypes.c_void_p),
        ("last_scores", ctypes.c_void_p),
        ("count", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("last_pool", ctypes.c_int32),
        ("scores_stride", ctypes.c_int32),
        ("frames_seen", ctypes.c_int64),
    ]


class statekv_cache_view(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("length", ctypes.c_int64),
        ("capacity", ctypes.c_int64),
        ("start", ctypes.c_int64),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


class statekv_launch_plan(ctypes.Structure):
    _fields_ = [
        ("out_splits", ctypes.c_int32),
        ("stat_splits", ctypes.c_int32),
        ("row_tiles", ctypes.c_int32),
        ("key_tiles", ctypes.c_int32),
    ]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libstatekv.so (once).  Raises ImportError if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing; build it with `python streaming_long_video_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(statekv_layer_config)
    sig = {
        "statekv_workspace_bytes": (ctypes.c_int, [cfgp, ctypes.POINTER(ctypes.c_size_t)]),
        "statekv_init_layer": (ctypes.c_int, [cfgp, P, ctypes.c_size_t, ctypes.POINTER(P)]),
        "statekv_prefill_frame": (ctypes.c_int, [P, P, P, P, P, P]),
        "statekv_full_attention_frame": (ctypes.c_int, [P, P, P, P, P, P]),
        "statekv_decode_attention": (ctypes.c_int, [P, P, ctypes.c_int32, P, P]),
        "statekv_decode_attention_noalloc": (ctypes.c_int, [P, P, ctypes.c_int32, P, P]),
        "statekv_rope": (ctypes.c_int, [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P]),
        "statekv_qkv_rope": (ctypes.c_int, [P, P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                            ctypes.c_double, ctypes.c_double, P, P, P, P,
                                            ctypes.c_uint64, P]),
        "statekv_qkv_rope_workspace_size": (ctypes.c_int, [ctypes.c_int32] * 5
                                            + [ctypes.POINTER(ctypes.c_uint64)]),
        "statekv_state": (ctypes.c_int, [P, ctypes.POINTER(statekv_state_view)]),
        "statekv_detailed_cache": (ctypes.c_int, [P, ctypes.POINTER(statekv_cache_view)]),
        "statekv_reset_layer": (ctypes.c_int, [P]),
        "statekv_restore_layer": (ctypes.c_int, [P, ctypes.c_int64, ctypes.c_int32]),
        "statekv_free_layer": (ctypes.c_int, [P]),
        "statekv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "statekv_select_topb": (ctypes.c_int, [P, ctypes.c_int32, ctypes.c_int32, P, P]),
        "statekv_attention_mass": (ctypes.c_int, [P, ctypes.POINTER(ctypes.c_int32),
                                                  ctypes.c_int32, P, P, P]),
        "statekv_mass_set_words": (ctypes.c_int, [P, ctypes.POINTER(ctypes.c_int32)]),
        "statekv_launch_plan_for": (ctypes.c_int, [P, ctypes.c_int32,
                                                   ctypes.POINTER(statekv_launch_plan)]),
        "statekv_profile_start": (ctypes.c_int, [P, ctypes.c_uint32, ctypes.c_int32]),
        "statekv_profile_stop": (ctypes.c_int, [P, ctypes.POINTER(ctypes.c_double),
                                                ctypes.POINTER(ctypes.c_int64)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str) -> None:
    if status != STATEKV_OK:
        raise StateKVError(status, what)


def make_config(n_q_heads, n_kv_heads, head_dim, frame_tokens, state_budget,
                detailed_capacity, position_offset=0, softmax_scale=0.0, flags=0,
                num_splits=0, rope_theta=0.0, rope_scaling=0.0) -> statekv_layer_config:
    return statekv_layer_config(int(n_q_heads), int(n_kv_heads), int(head_dim),
                                int(frame_tokens), int(state_budget), int(num_splits),
                                int(detailed_capacity), int(position_offset),
                                float(softmax_scale), int(flags), float(rope_theta),
                                float(rope_scaling))


def statekv_status_string(status: int) -> str:
    return load_library().statekv_status_string(int(status)).decode()


def statekv_workspace_bytes(cfg: statekv_layer_config) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().statekv_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "statekv_workspace_bytes")
    return n.value


def statekv_init_layer(cfg: statekv_layer_config, workspace_ptr: int, nbytes: int) -> int:
    h = ctypes.c_void_p(0)
    _check(load_library().statekv_init_layer(ctypes.byref(cfg), ctypes.c_void_p(workspace_ptr),
                                             ctypes.c_size_t(nbytes), ctypes.byref(h)),
           "statekv_init_layer")
    return h.value


def statekv_prefill_frame(layer: int, q: int, k: int, v: int, o: int, stream: int = 0) -> None:
    _check(load_library().statekv_prefill_frame(layer, q, k, v, o, stream or None),
           "statekv_prefill_frame")


def statekv_full_attention_frame(layer: int, q: int, k: int, v: int, o: int,
                                 stream: int = 0) -> None:
    _check(load_library().statekv_full_attention_frame(layer, q, k, v, o, stream or None),
           "statekv_full_attention_frame")


def statekv_decode_attention(layer: int, q: int, n_queries: int, o: int, stream: int = 0) -> None:
    _check(load_library().statekv_decode_attention(layer, q, n_queries, o, stream or None),
           "statekv_decode_attention")


def statekv_decode_attention_noalloc(layer: int, q: int, n_queries: int, o: int,
                                     stream: int = 0) -> None:
    _check(load_library().statekv_decode_attention_noalloc(layer, q, n_queries, o,
                                                           stream or None),
           "statekv_decode_attention_noalloc")


def statekv_rope(layer: int, x: int, n_tokens: int, n_heads: int, first_position: int,
                 stream: int = 0) -> None:
    _check(load_library().statekv_rope(layer, x, n_tokens, n_heads, first_position,
                                       stream or None), "statekv_rope")


def statekv_qkv_rope(x: int, w: int, n_tokens: int, hidden: int, n_q_heads: int,
                     n_kv_heads: int, head_dim: int, first_position: int, rope_theta: float,
                     rope_scaling: float, q: int, k: int, v: int, workspace: int = 0,
                     workspace_bytes: int = 0, stream: int = 0) -> None:
    _check(load_library().statekv_qkv_rope(x, w, n_tokens, hidden, n_q_heads, n_kv_heads,
                                           head_dim, first_position, rope_theta, rope_scaling,
                                           q, k, v, workspace or None, workspace_bytes,
                                           stream or None), "statekv_qkv_rope")


def statekv_qkv_rope_workspace_size(n_tokens: int, hidden: int, n_q_heads: int,
                                    n_kv_heads: int, head_dim: int) -> int:
    n = ctypes.c_uint64()
    _check(load_library().statekv_qkv_rope_workspace_size(n_tokens, hidden, n_q_heads,
                                                          n_kv_heads, head_dim, ctypes.byref(n)),
           "statekv_qkv_rope_workspace_size")
    return n.value


def statekv_state(layer: int) -> statekv_state_view:
    view = statekv_state_view()
    _check(load_library().statekv_state(layer, ctypes.byref(view)), "statekv_state")
    return view


def statekv_detailed_cache(layer: int) -> statekv_cache_view:
    view = statekv_cache_view()
    _check(load_library().statekv_detailed_cache(layer, ctypes.byref(view)),
           "statekv_detailed_cache")
    return view


def statekv_reset_layer(layer: int) -> None:
    _check(load_library().statekv_reset_layer(layer), "statekv_reset_layer")


def statekv_restore_layer(layer: int, frames_seen: int, count: int) -> None:
    _check(load_library().statekv_restore_layer(layer, int(frames_seen), int(count)),
           "statekv_restore_layer")


def statekv_free_layer(layer: int) -> None:
    _check(load_library().statekv_free_layer(layer), "statekv_free_layer")


def statekv_select_topb(scores: int, n: int, budget: int, out_idx: int, stream: int = 0) -> None:
    _check(load_library().statekv_select_topb(scores, int(n), int(budget), out_idx,
                                              stream or None),
           "statekv_select_topb")


def statekv_attention_mass(layer: int, budgets, sets: int, out: int, stream: int = 0) -> None:
    arr = (ctypes.c_int32 * len(budgets))(*[int(b) for b in budgets])
    _check(load_library().statekv_attention_mass(layer, arr, len(budgets), sets, out,
                                                 stream or None), "statekv_attention_mass")


def statekv_launch_plan_for(layer: int, pool: int) -> dict:
    """The prefill step's launch plan at a pool of `pool` candidates."""
    lp = statekv_launch_plan()
    _check(load_library().statekv_launch_plan_for(layer, int(pool), ctypes.byref(lp)),
           "statekv_launch_plan_for")
    return {f: int(getattr(lp, f)) for f, _ in statekv_launch_plan._fields_}


def statekv_mass_set_words(layer: int) -> int:
    w = ctypes.c_int32(0)
    _check(load_library().statekv_mass_set_words(layer, ctypes.byref(w)),
           "statekv_mass_set_words")
    return w.value


def statekv_profile_start(layer: int, kernel_mask: int, max_records: int) -> None:
    _check(load_library().statekv_profile_start(layer, int(kernel_mask), int(max_records)),
           "statekv_profile_start")


def statekv_profile_stop(layer: int):
    """Returns {kernel name: (total ms, launches)} for the recorded launches."""
    n = len(STATEKV_KERNELS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(load_library().statekv_profile_stop(layer, ms, cnt), "statekv_profile_stop")
    return {name: (ms[i], cnt[i]) for i, name in enumerate(STATEKV_KERNELS)}
