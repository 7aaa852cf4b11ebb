"""ctypes view of the C ABI in include/pod_attn.h (libpod_attn.so, built in-tree).

There is no fallback: if the shared library is missing or does not load, the
import fails loudly.
"""
from __future__ import annotations

import ctypes
import os

LIB_NAME = "libpod_attn.so"
# POD_ATTN_LIB names another build of the same library (the host-only
# sanitizer build of the planner and ABI layer that the CPU tests use)
LIB_PATH = os.environ.get("POD_ATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

POD_OK = 0
POD_ERR_INVALID = 1
POD_ERR_UNSUPPORTED = 2
POD_ERR_NOT_PLANNED = 3
POD_ERR_WORKSPACE = 4
POD_ERR_HIP = 5

POD_DTYPE_F16 = 0
POD_DTYPE_BF16 = 1
POD_DTYPE_FP8_E4M3 = 3

POD_ORDER_INTERLEAVE = 0
POD_ORDER_PREFILL_FIRST = 1
POD_ORDER_DECODE_FIRST = 2
POD_ORDER_LONGEST_FIRST = 3

POD_HDR_WORDS = 24
POD_IMAGE_MAGIC = 0x504F4431

EXPORTED = (
    "pod_create", "pod_destroy", "pod_plan", "pod_plan_stats", "pod_run",
    "pod_last_error", "pod_workspace_bytes", "pod_plan_compute", "pod_merge_states",
    "pod_create_graph", "pod_run_static",
)

_i32p = ctypes.POINTER(ctypes.c_int32)


class PodRoleDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        # host int32 arrays, as addresses (a plain integer or None)
        ("qo_indptr", ctypes.c_void_p),
        ("kv_indptr", ctypes.c_void_p),
        ("last_page_len", ctypes.c_void_p),
        ("causal", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
    ]


class PodPlanDesc(ctypes.Structure):
    _fields_ = [
        ("prefill", PodRoleDesc),
        ("decode", PodRoleDesc),
        ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("has_sinks", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("decode_chunk", ctypes.c_int32),
        ("order", ctypes.c_int32),
        ("decode_kv_dtype", ctypes.c_int32),
    ]


class PodRoleArgs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("q_stride_tok", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("kv_stride_page", ctypes.c_int64),
        ("kv_stride_tok", ctypes.c_int64),
        ("kv_stride_head", ctypes.c_int64),
        ("kv_indices", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("out_stride_tok", ctypes.c_int64),
        ("out_stride_head", ctypes.c_int64),
        ("lse", ctypes.c_void_p),
    ]


class PodRunArgs(ctypes.Structure):
    _fields_ = [
        ("prefill", PodRoleArgs),
        ("decode", PodRoleArgs),
        ("sinks", ctypes.c_void_p),
        ("q_scale_d", ctypes.c_float),
        ("k_scale_d", ctypes.c_float),
        ("v_scale_d", ctypes.c_float),
    ]


class PodPlanInfo(ctypes.Structure):
    _fields_ = [
        ("n_items", ctypes.c_int32),
        ("n_prefill_items", ctypes.c_int32),
        ("n_decode_items", ctypes.c_int32),
        ("n_groups", ctypes.c_int32),
        ("n_slots", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("decode_chunk", ctypes.c_int32),
        ("image_ints", ctypes.c_int32),
        ("float_ws_bytes", ctypes.c_int64),
        ("int_ws_bytes", ctypes.c_int64),
    ]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_LIB = None


def load() -> ctypes.CDLL:
    """Load libpod_attn.so once; raise if it is not built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    vp = ctypes.c_void_p
    lib.pod_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_size_t, vp, ctypes.c_size_t]
    lib.pod_create_graph.argtypes = [ctypes.POINTER(vp), ctypes.c_int, vp, ctypes.c_size_t, vp,
                                     ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32]
    lib.pod_destroy.argtypes = [vp]
    lib.pod_plan.argtypes = [vp, ctypes.POINTER(PodPlanDesc), vp]
    lib.pod_plan_stats.argtypes = [vp, ctypes.POINTER(PodPlanInfo)]
    lib.pod_run.argtypes = [vp, ctypes.POINTER(PodRunArgs), vp]
    lib.pod_last_error.argtypes = []
    lib.pod_last_error.restype = ctypes.c_char_p
    lib.pod_workspace_bytes.argtypes = [ctypes.POINTER(PodPlanDesc), ctypes.POINTER(ctypes.c_size_t),
                                        ctypes.POINTER(ctypes.c_size_t)]
    lib.pod_plan_compute.argtypes = [ctypes.POINTER(PodPlanDesc), _i32p, ctypes.c_size_t,
                                     ctypes.POINTER(PodPlanInfo)]
    fp = ctypes.POINTER(ctypes.c_float)
    lib.pod_merge_states.argtypes = [vp, fp, vp, fp, vp, fp, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, fp, ctypes.c_int, vp]
    lib.pod_run_static.argtypes = [ctypes.POINTER(PodPlanDesc), ctypes.POINTER(PodRunArgs), ctypes.c_int, vp]
    for name in ("pod_create", "pod_destroy", "pod_plan", "pod_plan_stats", "pod_run",
                 "pod_workspace_bytes", "pod_plan_compute", "pod_merge_states", "pod_create_graph",
                 "pod_run_static"):
        getattr(lib, name).restype = ctypes.c_int
    _LIB = lib
    return lib


class PodError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pod error {code}: {msg}")
        self.code = code


def check(code: int) -> None:
    """Map a POD_ERR_* code to an exception (ValueError / NotImplementedError as the pages do)."""
    if code == POD_OK:
        return
    msg = load().pod_last_error().decode(errors="replace")
    if code == POD_ERR_INVALID:
        raise ValueError(msg)
    if code == POD_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise PodError(code, msg)
