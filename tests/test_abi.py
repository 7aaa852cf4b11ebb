"""The C ABI library loads on a host without a GPU and exports every entry
point include/pod_attn.h declares; error paths return their documented codes."""
import ctypes
import os
import re

import pytest

from serving_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pod_attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pod_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_entry_point():
    lib = _lib.load()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_null_arguments_are_rejected():
    lib = _lib.load()
    assert lib.pod_plan_compute(None, None, 0, None) == _lib.POD_ERR_INVALID
    assert b"NULL" in lib.pod_last_error()
    assert lib.pod_workspace_bytes(None, None, None) == _lib.POD_ERR_INVALID
    assert lib.pod_plan(None, None, None) == _lib.POD_ERR_INVALID
    assert lib.pod_run(None, None, None) == _lib.POD_ERR_INVALID
    assert lib.pod_destroy(None) == _lib.POD_OK
    out = ctypes.c_void_p()
    assert lib.pod_create(ctypes.byref(out), 0, None, 0, None, 0) == _lib.POD_ERR_INVALID
    assert lib.pod_plan_stats(None, None) == _lib.POD_ERR_INVALID
    assert lib.pod_create_graph(None, 0, None, 0, None, 0, 1, 1) == _lib.POD_ERR_INVALID
    assert lib.pod_create_graph(ctypes.byref(out), 0, None, 0, None, 0, -1, 1) == _lib.POD_ERR_INVALID
    assert b"batch" in lib.pod_last_error()
    # the merge checks its arguments before touching a device
    bf16 = _lib.POD_DTYPE_BF16
    assert lib.pod_merge_states(None, None, None, None, None, None, 4, 8, 128, bf16, None, 0, None) \
        == _lib.POD_ERR_INVALID
    assert lib.pod_merge_states(None, None, None, None, None, None, 4, 8, 64, bf16, None, 0, None) \
        == _lib.POD_ERR_UNSUPPORTED
    assert lib.pod_merge_states(None, None, None, None, None, None, -1, 8, 128, bf16, None, 0, None) \
        == _lib.POD_ERR_INVALID
    assert lib.pod_merge_states(None, None, None, None, None, None, 0, 8, 128, bf16, None, 0, None) \
        == _lib.POD_OK
    bad = ctypes.c_void_p(0x1008)   # 8-byte aligned only
    fl = ctypes.cast(ctypes.c_void_p(0x2000), ctypes.POINTER(ctypes.c_float))
    assert lib.pod_merge_states(bad, fl, bad, fl, bad, fl, 4, 8, 128, bf16, None, 0, None) \
        == _lib.POD_ERR_INVALID
    assert b"16-byte" in lib.pod_last_error()


def test_error_codes_map_to_python_exceptions():
    lib = _lib.load()
    lib.pod_plan_compute(None, None, 0, None)
    with pytest.raises(ValueError):
        _lib.check(_lib.POD_ERR_INVALID)
    with pytest.raises(NotImplementedError):
        _lib.check(_lib.POD_ERR_UNSUPPORTED)
    with pytest.raises(_lib.PodError):
        _lib.check(_lib.POD_ERR_NOT_PLANNED)


@pytest.mark.parametrize("kind", ["int32", "int64", "list", "torch", "strided"])
def test_plan_descriptor_marshalling(kind):
    """The binding's plan descriptor points at int32 host copies of the length
    arrays, whatever array type the caller hands in, and the planner reads the
    same lengths from it as from a descriptor built directly."""
    import numpy as np
    import torch

    from serving_attention_amd.pod import BatchPOD

    qo = [0, 3, 3, 10]
    kv = [0, 2, 3, 7]
    lpl = [5, 16, 1]
    conv = {
        "int32": lambda a: np.asarray(a, np.int32),
        "int64": lambda a: np.asarray(a, np.int64),
        "list": list,
        "torch": lambda a: torch.tensor(a, dtype=torch.int32),
        "strided": lambda a: np.repeat(np.asarray(a, np.int32), 2)[::2],
    }[kind]
    keep = []
    qo_in = conv(qo)
    d = BatchPOD._role_desc(qo_in, conv(kv), conv(lpl), True, -1, None, keep)
    assert d.batch == 3 and len(keep) == 3
    for arr, want, addr in zip(keep, (qo, kv, lpl), (d.qo_indptr, d.kv_indptr, d.last_page_len)):
        assert arr.dtype == np.int32 and arr.flags.c_contiguous
        assert addr == arr.ctypes.data
        got = np.ctypeslib.as_array(ctypes.cast(addr, ctypes.POINTER(ctypes.c_int32)), (len(want),))
        assert got.tolist() == want
    # an int32 array that is already dense is used in place, anything else copied
    assert (keep[0] is qo_in) == (kind == "int32")
    lib = _lib.load()
    empty = BatchPOD._role_desc(None, None, None, True, -1, None, [])
    desc = _lib.PodPlanDesc(d, empty, 8, 2, 128, 16, _lib.POD_DTYPE_BF16, 0, 256, 0, 0, 0)
    info = _lib.PodPlanInfo()
    assert lib.pod_plan_compute(ctypes.byref(desc), None, 0, ctypes.byref(info)) in (
        _lib.POD_OK, _lib.POD_ERR_WORKSPACE)
    assert info.n_prefill_items > 0 and info.n_decode_items == 0
