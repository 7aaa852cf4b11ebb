"""Host-side helpers for driving the planner through the C ABI (no GPU needed)."""
import ctypes

import numpy as np

from serving_attention_amd import _lib


def role_desc(qo_lens, kv_lens, page_size, causal=True, window_left=-1, keep=None,
              qo_indptr=None, kv_indptr=None, last_page_len=None, sm_scale=0.0):
    if qo_lens is None:
        return _lib.PodRoleDesc(0, None, None, None, int(causal), window_left, 0.0)
    qo = np.asarray(qo_indptr if qo_indptr is not None else np.concatenate([[0], np.cumsum(qo_lens)]), np.int32)
    if kv_indptr is None:
        pages = [-(-k // page_size) for k in kv_lens]
        kv_indptr = np.concatenate([[0], np.cumsum(pages)])
    kv = np.asarray(kv_indptr, np.int32)
    lpl = np.asarray(last_page_len if last_page_len is not None else [(k - 1) % page_size + 1 for k in kv_lens], np.int32)
    keep.extend([qo, kv, lpl])
    p = lambda a: a.ctypes.data
    return _lib.PodRoleDesc(len(qo) - 1, p(qo), p(kv), p(lpl), int(causal), window_left, float(sm_scale))


def plan_desc(prefill=None, decode=None, hqo=8, hkv=2, page_size=16, head_dim=128, dtype=1,
              sinks=0, num_cus=256, decode_chunk=0, order=0, keep=None):
    """prefill / decode: dicts of role_desc keyword arguments (or None)."""
    keep = [] if keep is None else keep
    rp = role_desc(page_size=page_size, keep=keep, **prefill) if prefill else role_desc(None, None, page_size)
    rd = role_desc(page_size=page_size, keep=keep, **decode) if decode else role_desc(None, None, page_size)
    d = _lib.PodPlanDesc(rp, rd, hqo, hkv, head_dim, page_size, dtype, sinks, num_cus,
                         decode_chunk, order)
    return d, keep


def compute(desc):
    lib = _lib.load()
    info = _lib.PodPlanInfo()
    rc = lib.pod_plan_compute(ctypes.byref(desc), None, 0, ctypes.byref(info))
    if rc not in (_lib.POD_OK, _lib.POD_ERR_WORKSPACE):
        return rc, None, None
    img = np.zeros(max(info.image_ints, 1), np.int32)
    rc = lib.pod_plan_compute(ctypes.byref(desc), img.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                              img.size, ctypes.byref(info))
    return rc, img, info


def decode_image(img):
    h = img[:_lib.POD_HDR_WORDS]
    assert h[0] == _lib.POD_IMAGE_MAGIC
    n_items, grid, n_reqs, n_groups = int(h[1]), int(h[2]), int(h[3]), int(h[4])
    n_blocks = int(h[14])
    reqs = img[h[5]:h[5] + 4 * n_reqs].reshape(n_reqs, 4)
    items = img[h[6]:h[6] + 8 * n_items].reshape(n_items, 8)
    wgs = img[h[12]:h[12] + 8 * grid].reshape(grid, 8)
    blocks = img[h[13]:h[13] + 4 * n_blocks].reshape(n_blocks, 4)
    groups = img[h[7]:h[7] + 4 * n_groups].reshape(n_groups, 4)
    counters = img[h[8]:h[8] + n_groups]
    wg_of_item = np.full(n_items, -1, np.int64)
    for w, wg in enumerate(wgs):
        first, nt, nc = int(wg[0]), int(wg[1]), int(wg[2])
        wg_of_item[first:first + nt + nc] = w
    pool_first, pool_count = int(h[15]), int(h[16])
    queue = img[h[17]:h[17] + 2]
    tdesc = img[h[18]:h[18] + 8 * n_items].reshape(n_items, 8)
    return dict(n_items=n_items, grid=grid, reqs=reqs, items=items, wgs=wgs, blocks=blocks,
                wg_of_item=wg_of_item, groups=groups, counters=counters, n_slots=int(h[9]),
                slot_floats=int(h[10]), chunk=int(h[11]), pool_first=pool_first,
                pool_count=pool_count, queue=queue, tdesc=tdesc)
