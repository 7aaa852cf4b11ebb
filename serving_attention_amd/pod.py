"""Python binding of the POD attention library: argument marshalling only.

Mirrors the batch wrapper of the POD article (www.dpshk.com/news/5405057,
"批量 POD" and "BatchPOD 的 run 差异"): plan() once from host length arrays,
run() per layer, returning (out_p, out_d) or ((out_p, lse_p), (out_d, lse_d)).
PyTorch supplies device memory and the current stream; every step of the
attention itself runs in the HIP library.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional, Sequence, Tuple, Union

import numpy as np
import torch

from . import _lib

_DT = {torch.float16: _lib.POD_DTYPE_F16, torch.bfloat16: _lib.POD_DTYPE_BF16}
KVCache = Union[torch.Tensor, Tuple[torch.Tensor, torch.Tensor]]


def _host_i32(x) -> np.ndarray:
    if type(x) is np.ndarray and x.dtype == np.int32 and x.flags.c_contiguous:
        return x
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu")
        x = x.numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: Optional[np.ndarray]):
    """Address of a host array's data (the plan descriptor's pointer fields)."""
    if a is None:
        return None
    return a.__array_interface__["data"][0]


def _dtype_code(dtype) -> int:
    if isinstance(dtype, str):
        dtype = {"f16": torch.float16, "float16": torch.float16, "half": torch.float16,
                 "bf16": torch.bfloat16, "bfloat16": torch.bfloat16}[dtype]
    if dtype not in _DT:
        raise NotImplementedError(f"dtype {dtype} is not supported (float16 / bfloat16)")
    return _DT[dtype]


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def kv_views(cache: KVCache, kv_layout: str):
    """(k, v, page_stride, token_stride, head_stride) in elements for a paged cache.

    cache: combined [P, 2, page_size, H_kv, D] (NHD) / [P, 2, H_kv, page_size, D]
    (HND), or a (k_cache, v_cache) pair of [P, page_size, H_kv, D] / [P, H_kv,
    page_size, D] tensors with equal strides.
    """
    if isinstance(cache, (tuple, list)):
        k, v = cache
    else:
        if cache.dim() != 5 or cache.shape[1] != 2:
            raise ValueError("combined paged cache must be [pages, 2, ...]")
        k, v = cache[:, 0], cache[:, 1]
    if k.dim() != 4 or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("k and v caches must be 4-D with equal shapes and strides")
    if k.stride(-1) != 1:
        raise ValueError("head_dim must be the innermost, dense dimension")
    if kv_layout == "NHD":
        return k, v, k.stride(0), k.stride(1), k.stride(2)
    if kv_layout == "HND":
        return k, v, k.stride(0), k.stride(2), k.stride(1)
    raise ValueError(f"unknown kv_layout {kv_layout!r}")


def _kv_geometry(cache: KVCache, kv_layout: str):
    """What a launch needs of a paged cache, read from the tensor metadata
    without building views: (k address, v address, dtype, device, pages,
    page_size, kv heads, head_dim, page / token / head strides in elements).
    The same checks as kv_views."""
    if isinstance(cache, (tuple, list)):
        k, v = cache
        if k.dim() != 4 or k.shape != v.shape or k.stride() != v.stride():
            raise ValueError("k and v caches must be 4-D with equal shapes and strides")
        shape, st = k.shape, k.stride()
        kp, vp, dt, dev = k.data_ptr(), v.data_ptr(), k.dtype, k.device
    else:
        if cache.dim() != 5 or cache.shape[1] != 2:
            raise ValueError("combined paged cache must be [pages, 2, ...]")
        cs = cache.stride()
        shape = (cache.shape[0],) + tuple(cache.shape[2:])
        st = (cs[0],) + tuple(cs[2:])
        kp, dt, dev = cache.data_ptr(), cache.dtype, cache.device
        vp = kp + cs[1] * cache.element_size()
    if st[3] != 1:
        raise ValueError("head_dim must be the innermost, dense dimension")
    if kv_layout == "NHD":
        return kp, vp, dt, dev, shape[0], shape[1], shape[2], shape[3], st[0], st[1], st[2]
    if kv_layout == "HND":
        return kp, vp, dt, dev, shape[0], shape[2], shape[1], shape[3], st[0], st[2], st[1]
    raise ValueError(f"unknown kv_layout {kv_layout!r}")


def _plan_record(keep, present, num_qo_heads, num_kv_heads, head_dim, page_size, dtype, sinks,
                 kv_dtype_d) -> dict:
    """What run() checks its tensors against. keep holds (qo, kv, lpl) of each
    present role, prefill first."""
    nnz, rows = [], []
    k = 0
    for here in present:
        if not here:
            rows.append(0)
            nnz.append(0)
        else:
            rows.append(int(keep[k][-1]))
            nnz.append(int(keep[k + 1][-1]))
            k += 3
    return dict(rows=tuple(rows), nnz=tuple(nnz), num_qo_heads=int(num_qo_heads),
                num_kv_heads=int(num_kv_heads), head_dim=int(head_dim), page_size=int(page_size),
                dtype=_dtype_code(dtype), sinks=bool(sinks), fp8_d=kv_dtype_d == torch.float8_e4m3fn)


def _role_args(pl, kv_layout, graph, idx, q, cache, kv_indices, out, lse):
    """One role's pod_role_args, checked against the plan record."""
    rows = pl["rows"][idx]
    if rows == 0 or q is None:
        return _lib.PodRoleArgs()
    hq, d = pl["num_qo_heads"], pl["head_dim"]
    # graph mode: buffers sized for the largest plan
    short = q.shape[0] < rows if graph else q.shape[0] != rows
    if q.dim() != 3 or short or q.shape[1] != hq or q.shape[2] != d:
        raise ValueError(f"q must be [{rows}, {hq}, {d}], got {tuple(q.shape)}")
    if _DT.get(q.dtype) != pl["dtype"]:
        raise _lib.PodError(_lib.POD_ERR_NOT_PLANNED, "q dtype differs from the planned dtype")
    if q.stride(-1) != 1:
        raise ValueError("q: head_dim must be dense")
    kp, vp, kdt, kdev, pages, ps, hk, kd, sp, st, sh = _kv_geometry(cache, kv_layout)
    want = torch.float8_e4m3fn if (idx == 1 and pl["fp8_d"]) else q.dtype
    if kdt != want:
        raise _lib.PodError(_lib.POD_ERR_NOT_PLANNED, f"kv dtype {kdt} differs from the planned {want}")
    if ps != pl["page_size"] or hk != pl["num_kv_heads"] or kd != d:
        raise ValueError("paged cache shape differs from the plan")
    if kdev != q.device:
        raise ValueError("the paged cache must be on q's device")
    nnz = pl["nnz"][idx]
    if kv_indices is not None:
        if kv_indices.dtype != torch.int32 or not kv_indices.is_cuda or kv_indices.dim() != 1:
            raise ValueError("kv_indices must be a 1-D int32 device tensor")
        if kv_indices.numel() < nnz:
            raise ValueError(f"kv_indices holds {kv_indices.numel()} pages, the plan needs {nnz}")
    elif pages < nnz:
        raise ValueError(f"identity page table needs {nnz} pages, the cache has {pages}")
    # outputs: the kernel writes 16-byte vectors of a dense head_dim and the
    # LSE at row * num_qo_heads + head
    if not isinstance(out, torch.Tensor) or out.dim() != 3 or out.shape[0] < q.shape[0] \
            or out.shape[1] != hq or out.shape[2] != d:
        raise ValueError(f"out must be [{q.shape[0]}, {hq}, {d}]")
    if out.dtype != q.dtype or out.device != q.device or out.stride(-1) != 1:
        raise ValueError("out must have q's dtype and device and a dense head_dim")
    if lse is not None:
        if lse.dim() != 2 or lse.shape[0] < q.shape[0] or lse.shape[1] != hq:
            raise ValueError(f"lse must be [{q.shape[0]}, {hq}]")
        if lse.dtype != torch.float32 or lse.device != q.device or lse.stride() != (hq, 1):
            raise ValueError("lse must be a contiguous float32 tensor on q's device")
    return _lib.PodRoleArgs(
        q.data_ptr(), q.stride(0), q.stride(1), kp, vp, sp, st, sh,
        kv_indices.data_ptr() if kv_indices is not None else None,
        out.data_ptr(), out.stride(0), out.stride(1),
        lse.data_ptr() if lse is not None else None)


def _run_args(pl, kv_layout, graph, q_p, paged_kv_cache_p, kv_indices_p, q_d, paged_kv_cache_d,
              kv_indices_d, sinks, return_lse, out_p, out_d, lse_p, lse_d, q_scale_d, k_scale_d,
              v_scale_d):
    """pod_run_args for one launch, with the outputs it writes (allocated here
    when not given)."""
    hq, d = pl["num_qo_heads"], pl["head_dim"]
    outs, lses = [], []
    for idx, q, o, l in ((0, q_p, out_p, lse_p), (1, q_d, out_d, lse_d)):
        rows = pl["rows"][idx]
        if q is None:
            if rows:
                raise ValueError("a planned role needs its q tensor")
            outs.append(None)
            lses.append(None)
            continue
        n = q.shape[0] if graph else rows
        if o is None:
            o = torch.empty((n, hq, d), dtype=q.dtype, device=q.device)
        if l is None and return_lse:
            l = torch.empty((n, hq), dtype=torch.float32, device=q.device)
        outs.append(o)
        lses.append(l)
    if pl["sinks"]:
        if sinks is None or sinks.dtype != torch.float32 or sinks.numel() != hq or not sinks.is_cuda:
            raise ValueError("plan has sinks: pass an fp32 [num_qo_heads] device tensor")
    elif sinks is not None:
        raise ValueError("plan has no sinks")
    args = _lib.PodRunArgs(
        _role_args(pl, kv_layout, graph, 0, q_p, paged_kv_cache_p, kv_indices_p, outs[0], lses[0]),
        _role_args(pl, kv_layout, graph, 1, q_d, paged_kv_cache_d, kv_indices_d, outs[1], lses[1]),
        sinks.data_ptr() if sinks is not None else None,
        float(q_scale_d or 0.0), float(k_scale_d or 0.0), float(v_scale_d or 0.0))
    return args, outs, lses


class BatchPOD:
    """Batch prefill + batch decode paged attention in one launch per run()."""

    def __init__(self, float_workspace_buffer: torch.Tensor, kv_layout: str = "NHD",
                 int_workspace_bytes: int = 8 << 20, use_cuda_graph: bool = False,
                 prefill_batch_size: Optional[int] = None, decode_batch_size: Optional[int] = None):
        """``use_cuda_graph`` fixes both batch sizes (POD article, "CUDAGraph 模式的运行时
        约束"): every plan must keep them, run() may be captured into a graph and
        the graph replays correctly after later plans. The caller then passes
        q, out and lse buffers sized for the largest plan and keeps them."""
        self._lib = _lib.load()
        if not float_workspace_buffer.is_cuda:
            raise ValueError("the float workspace must be a device tensor")
        if kv_layout not in ("NHD", "HND"):
            raise ValueError(f"unknown kv_layout {kv_layout!r}")
        self.kv_layout = kv_layout
        self.device = float_workspace_buffer.device
        self._float_ws = float_workspace_buffer
        # every plan copies a whole image (its counters zeroed) into the half it uses
        self._int_ws = torch.empty(int_workspace_bytes // 4, dtype=torch.int32, device=self.device)
        ctx = ctypes.c_void_p()
        dev = self.device.index if self.device.index is not None else 0
        fws = (ctypes.c_void_p(self._float_ws.data_ptr()), self._float_ws.numel() * self._float_ws.element_size())
        iws = (ctypes.c_void_p(self._int_ws.data_ptr()), self._int_ws.numel() * 4)
        self.use_cuda_graph = bool(use_cuda_graph)
        if self.use_cuda_graph:
            if prefill_batch_size is None or decode_batch_size is None:
                raise ValueError("use_cuda_graph needs prefill_batch_size and decode_batch_size")
            _lib.check(self._lib.pod_create_graph(ctypes.byref(ctx), dev, *fws, *iws,
                                                  int(prefill_batch_size), int(decode_batch_size)))
        else:
            _lib.check(self._lib.pod_create(ctypes.byref(ctx), dev, *fws, *iws))
        self._ctx = ctx
        self._planned = None

    def __del__(self):
        ctx = getattr(self, "_ctx", None)
        if ctx is not None and ctx.value:
            self._lib.pod_destroy(ctx)
            self._ctx = None

    @staticmethod
    def _role_desc(qo_indptr, kv_indptr, last_page_len, causal, window_left, sm_scale, keep):
        if qo_indptr is None:
            return _lib.PodRoleDesc(0, None, None, None, int(bool(causal)), int(window_left), 0.0)
        qo = _host_i32(qo_indptr)
        kv = _host_i32(kv_indptr)
        lpl = _host_i32(last_page_len)
        if qo.ndim != 1 or kv.shape != qo.shape or lpl.shape != (qo.shape[0] - 1,):
            raise ValueError("indptr arrays must be [batch+1] and last_page_len [batch]")
        keep.extend([qo, kv, lpl])
        return _lib.PodRoleDesc(int(qo.shape[0] - 1), _ptr(qo), _ptr(kv), _ptr(lpl),
                                int(bool(causal)), int(window_left),
                                float(sm_scale) if sm_scale is not None else 0.0)

    @classmethod
    def _plan_desc(cls, qo_indptr_p, kv_indptr_p, last_page_len_p,
                   qo_indptr_d, kv_indptr_d, last_page_len_d, *,
                   num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                   dtype=torch.bfloat16, causal_p: bool = True, causal_d: bool = True,
                   window_left_p: int = -1, window_left_d: int = -1,
                   sm_scale_p: Optional[float] = None, sm_scale_d: Optional[float] = None,
                   sinks: bool = False, decode_chunk: int = 0, order: int = 0,
                   kv_dtype_d=None, num_cus: int = 0):
        """The C plan descriptor and the host arrays it points into (kept alive
        by the caller while the descriptor is used)."""
        keep = []
        desc = _lib.PodPlanDesc(
            cls._role_desc(qo_indptr_p, kv_indptr_p, last_page_len_p, causal_p, window_left_p,
                           sm_scale_p, keep),
            cls._role_desc(qo_indptr_d, kv_indptr_d, last_page_len_d, causal_d, window_left_d,
                           sm_scale_d, keep),
            int(num_qo_heads), int(num_kv_heads), int(head_dim), int(page_size),
            _dtype_code(dtype), int(bool(sinks)), int(num_cus), int(decode_chunk), int(order),
            _lib.POD_DTYPE_FP8_E4M3 if kv_dtype_d == torch.float8_e4m3fn else 0)
        if kv_dtype_d not in (None, torch.float8_e4m3fn) and _DT.get(kv_dtype_d) != _dtype_code(dtype):
            raise NotImplementedError(f"decode K/V dtype {kv_dtype_d} is not supported")
        return desc, keep

    @classmethod
    def workspace_bytes(cls, *args, **kwargs) -> Tuple[int, int]:
        """(float, int) workspace bytes the plan with these arguments (those of
        plan(), plus ``num_cus``, default 256) needs. Host only."""
        desc, keep = cls._plan_desc(*args, **kwargs)
        fb, ib = ctypes.c_size_t(), ctypes.c_size_t()
        lib = _lib.load()
        _lib.check(lib.pod_workspace_bytes(ctypes.byref(desc), ctypes.byref(fb), ctypes.byref(ib)))
        del keep
        return int(fb.value), int(ib.value)

    def plan(self, qo_indptr_p, kv_indptr_p, last_page_len_p,
             qo_indptr_d, kv_indptr_d, last_page_len_d, *,
             num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
             dtype=torch.bfloat16, causal_p: bool = True, causal_d: bool = True,
             window_left_p: int = -1, window_left_d: int = -1,
             sm_scale_p: Optional[float] = None, sm_scale_d: Optional[float] = None,
             sinks: bool = False, decode_chunk: int = 0, order: int = 0, stream=None,
             kv_dtype_d=None):
        """Build and upload the work list. Either role may be None (empty).

        ``kv_dtype_d=torch.float8_e4m3fn`` plans the decode role over an FP8 KV
        cache (POD article, "Decode 侧参数与'plan 覆盖'行为": the calibration scales are decode
        run parameters); q and outputs keep ``dtype``.
        """
        desc, keep = self._plan_desc(
            qo_indptr_p, kv_indptr_p, last_page_len_p, qo_indptr_d, kv_indptr_d, last_page_len_d,
            num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
            page_size=page_size, dtype=dtype, causal_p=causal_p, causal_d=causal_d,
            window_left_p=window_left_p, window_left_d=window_left_d, sm_scale_p=sm_scale_p,
            sm_scale_d=sm_scale_d, sinks=sinks, decode_chunk=decode_chunk, order=order,
            kv_dtype_d=kv_dtype_d)
        s = _stream_handle(self.device) if stream is None else ctypes.c_void_p(stream)
        _lib.check(self._lib.pod_plan(self._ctx, ctypes.byref(desc), s))
        self._planned = _plan_record(keep, (qo_indptr_p is not None, qo_indptr_d is not None),
                                     num_qo_heads, num_kv_heads, head_dim, page_size, dtype, sinks,
                                     kv_dtype_d)
        return self

    def plan_info(self) -> dict:
        info = _lib.PodPlanInfo()
        _lib.check(self._lib.pod_plan_stats(self._ctx, ctypes.byref(info)))
        return info.as_dict()

    def run(self, q_p, paged_kv_cache_p, kv_indices_p, q_d, paged_kv_cache_d, kv_indices_d, *,
            sinks: Optional[torch.Tensor] = None, return_lse: bool = False,
            out_p=None, out_d=None, lse_p=None, lse_d=None,
            q_scale_d: Optional[float] = None, k_scale_d: Optional[float] = None,
            v_scale_d: Optional[float] = None):
        """One fused launch. Returns (out_p, out_d) or ((out_p, lse_p), (out_d, lse_d)).

        q_scale_d * k_scale_d multiply the decode sm_scale and v_scale_d the decode
        output (POD article, "Decode 侧参数与'plan 覆盖'行为"; here v_scale is folded into the
        launch's final normalisation). None means 1.
        """
        if self._planned is None:
            raise _lib.PodError(_lib.POD_ERR_NOT_PLANNED, "run() before plan()")
        args, outs, lses = _run_args(self._planned, self.kv_layout, self.use_cuda_graph, q_p,
                                     paged_kv_cache_p, kv_indices_p, q_d, paged_kv_cache_d, kv_indices_d,
                                     sinks, return_lse, out_p, out_d, lse_p, lse_d,
                                     q_scale_d, k_scale_d, v_scale_d)
        _lib.check(self._lib.pod_run(self._ctx, ctypes.byref(args), _stream_handle(self.device)))
        if return_lse:
            return (outs[0], lses[0]), (outs[1], lses[1])
        return outs[0], outs[1]


def single_decode_with_kv_cache(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                kv_layout: str = "NHD", window_left: int = -1,
                                sm_scale: Optional[float] = None, return_lse: bool = False,
                                workspace: Optional[torch.Tensor] = None):
    """Single-request decode (README tour, "快速上手单请求 Decode 注意力").

    q [num_qo_heads, head_dim]; k, v [kv_len, num_kv_heads, head_dim] (NHD) or
    [num_kv_heads, kv_len, head_dim] (HND). Runs the fused grid with only the
    decode role, treating the dense K/V as pages of one token.
    """
    if q.dim() != 2 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [H_qo, D] and k, v [kv_len, H_kv, D]")
    if kv_layout == "NHD":
        kv_len, hk, d = k.shape
        sp, sh = k.stride(0), k.stride(1)
    elif kv_layout == "HND":
        hk, kv_len, d = k.shape
        sp, sh = k.stride(1), k.stride(0)
    else:
        raise ValueError(f"unknown kv_layout {kv_layout!r}")
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    hq = q.shape[0]
    plan_args = dict(num_qo_heads=hq, num_kv_heads=hk, head_dim=d, page_size=1, dtype=q.dtype,
                     causal_d=False, window_left_d=window_left, sm_scale_d=sm_scale)
    dev = q.device.index if q.device.index is not None else torch.cuda.current_device()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    # the workspaces this plan needs (split-KV partial states grow with kv_len)
    fbytes, ibytes = BatchPOD.workspace_bytes(None, None, None, [0, 1], [0, kv_len], [1],
                                              num_cus=cus, **plan_args)
    if workspace is None:
        workspace = torch.empty(max(fbytes, 1 << 16), dtype=torch.uint8, device=q.device)
    w = BatchPOD(workspace, "NHD", int_workspace_bytes=max(ibytes, 1 << 16))
    w.plan(None, None, None, [0, 1], [0, kv_len], [1], **plan_args)
    # page_size 1 view: [kv_len, 1, H_kv, D] with the caller's strides
    kp = torch.as_strided(k, (kv_len, 1, hk, d), (sp, sp, sh, 1))
    vp = torch.as_strided(v, (kv_len, 1, hk, d), (sp, sp, sh, 1))
    res = w.run(None, None, None, q.view(1, hq, d), (kp, vp), None, return_lse=return_lse)
    if return_lse:
        (_, _), (o, lse) = res
        return o.view(hq, d), lse.view(hq)
    return res[1].view(hq, d)


def merge_states(o_a: torch.Tensor, lse_a: torch.Tensor, o_b: torch.Tensor, lse_b: torch.Tensor,
                 sinks: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                 lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Cascade merge of two states of the same rows over disjoint key sets.

    README tour, core operator list ("Cascade Attention": a shared-prefix level
    and a per-request level); the base-2 LSE of the cuDNN article ("LSE 契约")
    is what the merge consumes. o_* [rows, H, 128] float16 / bfloat16, lse_*
    [rows, H] float32, all on one GPU. ``sinks`` [H] float32 is applied once to
    the merged state (inputs must be sink-free). ``out`` / ``lse_out`` may be
    an input tensor itself. Returns (out, lse_out).
    """
    for name, t in (("o_a", o_a), ("o_b", o_b)):
        if t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [rows, heads, head_dim] tensor")
    if o_b.shape != o_a.shape or o_b.dtype != o_a.dtype or o_b.device != o_a.device:
        raise ValueError("o_a and o_b must match in shape, dtype and device")
    rows, heads, d = o_a.shape
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        if t.shape != (rows, heads) or t.dtype != torch.float32 or not t.is_contiguous() \
                or t.device != o_a.device:
            raise ValueError(f"{name} must be a contiguous float32 [rows, heads] tensor on o_a's device")
    if sinks is not None and (sinks.shape != (heads,) or sinks.dtype != torch.float32
                              or not sinks.is_contiguous() or sinks.device != o_a.device):
        raise ValueError("sinks must be a contiguous float32 [heads] tensor on o_a's device")
    out = torch.empty_like(o_a) if out is None else out
    lse_out = torch.empty_like(lse_a) if lse_out is None else lse_out
    if out.shape != o_a.shape or out.dtype != o_a.dtype or not out.is_contiguous() or out.device != o_a.device:
        raise ValueError("out must be a contiguous tensor like o_a")
    if lse_out.shape != lse_a.shape or lse_out.dtype != torch.float32 or not lse_out.is_contiguous() \
            or lse_out.device != o_a.device:
        raise ValueError("lse_out must be a contiguous tensor like lse_a")
    fp = ctypes.POINTER(ctypes.c_float)
    f = lambda t: ctypes.cast(t.data_ptr(), fp) if t is not None else None
    lib = _lib.load()
    _lib.check(lib.pod_merge_states(o_a.data_ptr(), f(lse_a), o_b.data_ptr(), f(lse_b), out.data_ptr(),
                                    f(lse_out), rows, heads, d, _dtype_code(o_a.dtype), f(sinks),
                                    o_a.device.index if o_a.device.index is not None else 0,
                                    _stream_handle(o_a.device)))
    return out, lse_out


def run_static(qo_indptr_p, kv_indptr_p, last_page_len_p, qo_indptr_d, kv_indptr_d, last_page_len_d,
               q_p, paged_kv_cache_p, kv_indices_p, q_d, paged_kv_cache_d, kv_indices_d, *,
               num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
               dtype=torch.bfloat16, kv_layout: str = "NHD", causal_p: bool = True, causal_d: bool = True,
               window_left_p: int = -1, window_left_d: int = -1, sm_scale_p: Optional[float] = None,
               sm_scale_d: Optional[float] = None, decode_chunk: int = 0, order: int = 0,
               kv_dtype_d=None, sinks: Optional[torch.Tensor] = None, return_lse: bool = False,
               out_p=None, out_d=None, lse_p=None, lse_d=None, q_scale_d: Optional[float] = None,
               k_scale_d: Optional[float] = None, v_scale_d: Optional[float] = None):
    """BatchPOD(...).plan(...) and .run(...) in one call of pod_run_static: no
    context and no workspace; the work list and split-KV partial states use the
    library's static device scratch (for callers that cannot allocate device
    memory; pass out/lse tensors to allocate nothing here either). Same
    arguments and results as plan() and run(); the plan's `sinks` flag follows
    from whether a sinks tensor is passed."""
    if kv_layout not in ("NHD", "HND"):
        raise ValueError(f"unknown kv_layout {kv_layout!r}")
    has_sinks = sinks is not None
    desc, keep = BatchPOD._plan_desc(
        qo_indptr_p, kv_indptr_p, last_page_len_p, qo_indptr_d, kv_indptr_d, last_page_len_d,
        num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
        dtype=dtype, causal_p=causal_p, causal_d=causal_d, window_left_p=window_left_p,
        window_left_d=window_left_d, sm_scale_p=sm_scale_p, sm_scale_d=sm_scale_d, sinks=has_sinks,
        decode_chunk=decode_chunk, order=order, kv_dtype_d=kv_dtype_d)
    pl = _plan_record(keep, (qo_indptr_p is not None, qo_indptr_d is not None), num_qo_heads,
                      num_kv_heads, head_dim, page_size, dtype, has_sinks, kv_dtype_d)
    args, outs, lses = _run_args(pl, kv_layout, False, q_p, paged_kv_cache_p, kv_indices_p, q_d,
                                 paged_kv_cache_d, kv_indices_d, sinks, return_lse, out_p, out_d, lse_p,
                                 lse_d, q_scale_d, k_scale_d, v_scale_d)
    ref = q_p if q_p is not None else q_d
    if ref is None or not ref.is_cuda:
        raise ValueError("run_static needs device query tensors")
    dev = ref.device.index if ref.device.index is not None else torch.cuda.current_device()
    lib = _lib.load()
    _lib.check(lib.pod_run_static(ctypes.byref(desc), ctypes.byref(args), dev, _stream_handle(ref.device)))
    del keep
    if return_lse:
        return (outs[0], lses[0]), (outs[1], lses[1])
    return outs[0], outs[1]
