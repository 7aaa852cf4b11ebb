"""Seeded workload builder: request lengths, CSR page tables and N(0,1) values.

Shapes and structure follow the examples on the FlashInfer pages:

* the single-request decode example of the README tour (www.gsyq.cn/news/442943,
  section "快速上手单请求 Decode 注意力"): q [32,128], K/V [2048,32,128] fp16;
* the PODWithPagedKVCacheWrapper docstring example of the POD article
  (www.dpshk.com/news/5405057, section "单请求 POD"): 7 requests, 64/8 heads,
  page_size 16, kv_indptr [0,17,29,44,48,66,100,128], last_page_len
  [1,7,14,4,3,1,16];
* the BatchPODWithPagedKVCacheWrapper example of the POD article (section
  "批量 POD"): 2 x 2048-token prefill plus 128 one-token decodes, page_size 1;
* the multi-token decode, left window and sink options of the cuDNN backend
  article (www.gsyq.cn/news/452757, section "Decode 能力矩阵与参数").

Metadata (lengths, page permutations) comes from ``numpy.random.default_rng(meta_seed)``.
Values come from a ``torch.Generator`` seeded with ``value_seed`` on the target
device: fp32 ``randn`` rounded to the storage dtype (round-to-nearest-even).
Consumers read the materialised dtype tensors; nothing here is regenerated
elsewhere.

The only integer relation used here is the inverse page bookkeeping a caller
does when it lays requests into pages: ``pages = ceil(kv_len / page_size)``
and ``last_page_len = (kv_len - 1) % page_size + 1``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

_TORCH_DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class RoleSpec:
    qo_lens: List[int]
    kv_lens: List[int]
    causal: bool = True
    window_left: int = -1


@dataclass
class WorkloadSpec:
    name: str
    prefill: Optional[RoleSpec]
    decode: Optional[RoleSpec]
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int = 128
    page_size: int = 16
    dtype: str = "bf16"
    sinks: bool = False
    # "separate": each role has a pool of its own; "shared": one pool for both
    pool: str = "separate"
    shuffle_pages: bool = False
    # unreferenced pages appended to every pool (poison targets)
    spare_pages: int = 0
    kv_layout: str = "NHD"
    sm_scale: Optional[float] = None
    meta_seed: int = 0
    value_seed: int = 1000
    # FP8 E4M3 decode K/V ("fp8_e4m3"; needs separate pools) and the decode
    # role's calibration scales (q_scale, k_scale, v_scale) of the POD article
    decode_kv_dtype: Optional[str] = None
    fp8_scales: tuple = (1.0, 1.0, 1.0)


@dataclass
class RoleTensors:
    q: torch.Tensor                 # [rows, H_qo, D]
    k_pool: torch.Tensor            # NHD [P, ps, H_kv, D] or HND [P, H_kv, ps, D] view
    v_pool: torch.Tensor
    kv_cache: torch.Tensor          # the tensor the pools are views of
    qo_indptr: np.ndarray           # int32 [B+1], tokens
    kv_indptr: np.ndarray           # int32 [B+1], pages
    kv_indices: np.ndarray          # int32 [nnz_pages], physical page ids
    last_page_len: np.ndarray       # int32 [B]
    kv_indices_dev: torch.Tensor    # int32 copy of kv_indices on the workload device
    causal: bool
    window_left: int
    sm_scale: float
    qo_lens: List[int]
    kv_lens: List[int]

    @property
    def batch(self) -> int:
        return len(self.qo_lens)

    @property
    def rows(self) -> int:
        return int(self.qo_indptr[-1])


@dataclass
class Workload:
    spec: WorkloadSpec
    prefill: Optional[RoleTensors]
    decode: Optional[RoleTensors]
    sinks: Optional[torch.Tensor]   # fp32 [H_qo] or None
    pools: List[torch.Tensor] = field(default_factory=list)

    def roles(self):
        out = []
        if self.prefill is not None:
            out.append(("prefill", self.prefill))
        if self.decode is not None:
            out.append(("decode", self.decode))
        return out


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _fill_randn_(t: torch.Tensor, gen: torch.Generator, chunk: int = 1 << 27) -> None:
    """Fill ``t`` (any float dtype, contiguous) with fp32 N(0,1) rounded to its dtype."""
    flat = t.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        tmp = torch.randn(e - s, generator=gen, dtype=torch.float32, device=t.device)
        flat[s:e].copy_(tmp)
        del tmp


def named_spec(name: str) -> WorkloadSpec:
    """The five named workloads plus small variants used by tests."""
    scale = 1.0 / math.sqrt(128.0)
    if name == "single_decode":
        # README tour: q [32,128], K/V [2048,32,128] fp16, NHD; dense K/V as page_size 1.
        return WorkloadSpec(
            name=name, prefill=None,
            decode=RoleSpec(qo_lens=[1], kv_lens=[2048], causal=False),
            num_qo_heads=32, num_kv_heads=32, page_size=1, dtype="f16",
            sm_scale=scale, meta_seed=1, value_seed=1001)
    if name == "batch_decode":
        # POD article docstring example: kv_indptr [0,17,29,44,48,66,100,128],
        # last_page_len [1,7,14,4,3,1,16], page_size 16 (kv_lens follow from them).
        pages = [17, 12, 15, 4, 18, 34, 28]
        lpl = [1, 7, 14, 4, 3, 1, 16]
        kv = [(p - 1) * 16 + l for p, l in zip(pages, lpl)]
        return WorkloadSpec(
            name=name, prefill=None,
            decode=RoleSpec(qo_lens=[1] * 7, kv_lens=kv, causal=False),
            num_qo_heads=64, num_kv_heads=8, page_size=16, dtype="f16",
            sm_scale=scale, meta_seed=2, value_seed=1002)
    if name == "batch_prefill":
        rng = np.random.default_rng(3)
        lens = [int(x) for x in rng.integers(256, 2049, 4)]
        return WorkloadSpec(
            name=name, prefill=RoleSpec(qo_lens=lens, kv_lens=lens, causal=True),
            decode=None, num_qo_heads=32, num_kv_heads=8, page_size=16, dtype="bf16",
            shuffle_pages=True, sm_scale=scale, meta_seed=3, value_seed=1003)
    if name == "pod":
        # POD article BatchPOD example: 2 x 2048 prefill + 128 x (1 token, kv 2048), page_size 1.
        return WorkloadSpec(
            name=name,
            prefill=RoleSpec(qo_lens=[2048] * 2, kv_lens=[2048] * 2, causal=True),
            decode=RoleSpec(qo_lens=[1] * 128, kv_lens=[2048] * 128, causal=True),
            num_qo_heads=64, num_kv_heads=8, page_size=1, dtype="bf16",
            sm_scale=scale, meta_seed=4, value_seed=1004)
    if name == "pod_fp8":
        # the pod workload with the decode role over an FP8 E4M3 KV cache and
        # calibration scales (q, k, v) of the POD article's decode parameters
        s = named_spec("pod")
        s.name = name
        s.decode_kv_dtype = "fp8_e4m3"
        s.fp8_scales = (1.0, 0.75, 1.25)
        return s
    if name == "pod_chunked":
        # 4096-token prefill chunk on a 16384-token prefix plus 256 four-token decodes.
        rng = np.random.default_rng(5)
        kv_d = [int(x) for x in rng.integers(1024, 32769, 256)]
        return WorkloadSpec(
            name=name,
            prefill=RoleSpec(qo_lens=[4096], kv_lens=[16384 + 4096], causal=True, window_left=4096),
            decode=RoleSpec(qo_lens=[4] * 256, kv_lens=kv_d, causal=True, window_left=4096),
            num_qo_heads=64, num_kv_heads=8, page_size=16, dtype="bf16", sinks=True,
            pool="shared", shuffle_pages=True, sm_scale=scale, meta_seed=5, value_seed=1005)
    raise KeyError(name)


NAMED = ("single_decode", "batch_decode", "batch_prefill", "pod", "pod_chunked", "pod_fp8")


def _role_pages(role: RoleSpec, ps: int):
    pages = [_ceil_div(k, ps) for k in role.kv_lens]
    lpl = [(k - 1) % ps + 1 for k in role.kv_lens]
    return pages, lpl


def build(spec: WorkloadSpec, device="cpu", poison: bool = False) -> Workload:
    """Materialise ``spec`` on ``device``.

    ``poison`` fills every pool slot no request references (tail slots of last
    pages and spare pages) with NaN, so a kernel that reads them shows it.
    """
    device = torch.device(device)
    dt = _TORCH_DTYPES[spec.dtype]
    ps, hkv, hqo, d = spec.page_size, spec.num_kv_heads, spec.num_qo_heads, spec.head_dim
    rng = np.random.default_rng(spec.meta_seed)
    # consume the stream the same way the length draws in named_spec did
    if spec.name == "batch_prefill":
        rng.integers(256, 2049, 4)
    elif spec.name == "pod_chunked":
        rng.integers(1024, 32769, 256)

    roles = [(n, r) for n, r in (("prefill", spec.prefill), ("decode", spec.decode)) if r is not None]
    for _, r in roles:
        assert len(r.qo_lens) == len(r.kv_lens)
    role_pages = {n: _role_pages(r, ps) for n, r in roles}

    # logical page numbering: prefill requests first, then decode
    if spec.pool == "shared":
        total = sum(sum(p) for p, _ in role_pages.values()) + spec.spare_pages
        perm = rng.permutation(total).astype(np.int32) if spec.shuffle_pages else np.arange(total, dtype=np.int32)
        pool_sizes = {"shared": total}
    else:
        perm = None
        pool_sizes = {n: sum(role_pages[n][0]) + spec.spare_pages for n, _ in roles}

    gen = torch.Generator(device=device)
    gen.manual_seed(spec.value_seed)

    def alloc_pool(npages, tdt):
        shape = (npages, 2, ps, hkv, d) if spec.kv_layout == "NHD" else (npages, 2, hkv, ps, d)
        t = torch.empty(shape, dtype=tdt, device=device)
        _fill_randn_(t, gen)
        return t

    assert spec.decode_kv_dtype in (None, "fp8_e4m3")
    assert spec.decode_kv_dtype is None or spec.pool == "separate", "FP8 decode K/V needs its own pool"
    pools = {}
    for key in pool_sizes:
        fp8 = key == "decode" and spec.decode_kv_dtype == "fp8_e4m3"
        pools[key] = alloc_pool(pool_sizes[key], torch.float8_e4m3fn if fp8 else dt)

    out = {}
    logical_base = 0
    for name, r in roles:
        pages, lpl = role_pages[name]
        kv_indptr = np.zeros(len(pages) + 1, dtype=np.int32)
        kv_indptr[1:] = np.cumsum(pages)
        qo_indptr = np.zeros(len(r.qo_lens) + 1, dtype=np.int32)
        qo_indptr[1:] = np.cumsum(r.qo_lens)
        nnz = int(kv_indptr[-1])
        if spec.pool == "shared":
            logical = np.arange(logical_base, logical_base + nnz, dtype=np.int64)
            kv_indices = perm[logical].astype(np.int32)
            logical_base += nnz
            cache = pools["shared"]
        else:
            if spec.shuffle_pages:
                kv_indices = rng.permutation(pool_sizes[name])[:nnz].astype(np.int32)
            else:
                kv_indices = np.arange(nnz, dtype=np.int32)
            cache = pools[name]
        k_pool, v_pool = cache.unbind(1)
        out[name] = dict(
            kv_cache=cache, k_pool=k_pool, v_pool=v_pool,
            qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
            last_page_len=np.asarray(lpl, dtype=np.int32),
            kv_indices_dev=torch.from_numpy(kv_indices.copy()).to(device),
            causal=r.causal, window_left=r.window_left,
            sm_scale=spec.sm_scale if spec.sm_scale is not None else 1.0 / math.sqrt(d),
            qo_lens=list(r.qo_lens), kv_lens=list(r.kv_lens))

    for name, r in roles:
        rows = int(sum(r.qo_lens))
        q = torch.empty((rows, hqo, d), dtype=dt, device=device)
        _fill_randn_(q, gen)
        out[name]["q"] = q

    sinks = None
    if spec.sinks:
        sinks = torch.randn(hqo, generator=gen, dtype=torch.float32, device=device)

    if poison:
        for name, _ in roles:
            o = out[name]
            cache = o["kv_cache"]
            used = np.zeros(cache.shape[0], dtype=bool)
            used[o["kv_indices"]] = True
            for b in range(len(o["last_page_len"])):
                last = int(o["kv_indices"][o["kv_indptr"][b + 1] - 1])
                l = int(o["last_page_len"][b])
                if l < ps:
                    if spec.kv_layout == "NHD":
                        cache[last, :, l:, :, :] = float("nan")
                    else:
                        cache[last, :, :, l:, :] = float("nan")
            if spec.pool == "shared":
                continue
            unused = np.nonzero(~used)[0]
            if len(unused):
                cache[torch.from_numpy(unused).to(device)] = float("nan")
        if spec.pool == "shared":
            used = np.zeros(pools["shared"].shape[0], dtype=bool)
            for name, _ in roles:
                used[out[name]["kv_indices"]] = True
            unused = np.nonzero(~used)[0]
            if len(unused):
                pools["shared"][torch.from_numpy(unused).to(device)] = float("nan")

    rt = {n: RoleTensors(**out[n]) for n, _ in roles}
    return Workload(spec=spec, prefill=rt.get("prefill"), decode=rt.get("decode"),
                    sinks=sinks, pools=list(pools.values()))


@dataclass
class CascadeWorkload:
    """A shared-prefix decode batch (README tour, core operator list: "Cascade
    Attention", a hierarchical KV cache whose shared prefix is stored once).

    Every request's keys are the shared prefix followed by its own suffix; the
    pool holds the prefix pages once. ``flat_*`` describes the same keys as one
    page list per request (prefix pages, then its own), for the one-level
    decode over the same data.
    """
    k_pool: torch.Tensor            # NHD [P, ps, H_kv, D]
    v_pool: torch.Tensor
    q: torch.Tensor                 # [rows, H_qo, D], rows of request b consecutive
    sinks: Optional[torch.Tensor]
    prefix_len: int
    prefix_indices: np.ndarray      # int32 physical pages of the prefix
    prefix_last_page_len: int
    qo_indptr: np.ndarray           # int32 [B+1] decode rows
    suffix_kv_indptr: np.ndarray    # int32 [B+1] pages of the suffixes
    suffix_indices: np.ndarray
    suffix_last_page_len: np.ndarray
    flat_kv_indptr: np.ndarray      # int32 [B+1] pages of prefix + suffix
    flat_indices: np.ndarray
    flat_last_page_len: np.ndarray
    num_qo_heads: int
    num_kv_heads: int
    page_size: int


def build_cascade(prefix_len: int, suffix_lens: List[int], q_len: int = 1, num_qo_heads: int = 64,
                  num_kv_heads: int = 8, page_size: int = 16, dtype: str = "bf16", sinks: bool = False,
                  meta_seed: int = 7, value_seed: int = 1007, device="cpu") -> CascadeWorkload:
    """Materialise a shared-prefix batch; the prefix fills whole pages, so the
    flat page lists describe exactly the same keys."""
    assert prefix_len % page_size == 0, "the prefix must fill whole pages"
    assert all(s >= q_len for s in suffix_lens)
    device = torch.device(device)
    dt = _TORCH_DTYPES[dtype]
    rng = np.random.default_rng(meta_seed)
    n_pre = prefix_len // page_size
    suf_pages = [_ceil_div(s, page_size) for s in suffix_lens]
    total = n_pre + sum(suf_pages)
    perm = rng.permutation(total).astype(np.int32)
    pre_idx = perm[:n_pre]
    suf_idx = perm[n_pre:]
    suf_indptr = np.zeros(len(suffix_lens) + 1, dtype=np.int32)
    suf_indptr[1:] = np.cumsum(suf_pages)
    flat = [np.concatenate([pre_idx, suf_idx[suf_indptr[b]:suf_indptr[b + 1]]])
            for b in range(len(suffix_lens))]
    flat_indptr = np.zeros(len(suffix_lens) + 1, dtype=np.int32)
    flat_indptr[1:] = np.cumsum([len(f) for f in flat])
    lpl = np.array([(s - 1) % page_size + 1 for s in suffix_lens], dtype=np.int32)
    gen = torch.Generator(device=device)
    gen.manual_seed(value_seed)
    cache = torch.empty((total, 2, page_size, num_kv_heads, 128), dtype=dt, device=device)
    _fill_randn_(cache, gen)
    rows = q_len * len(suffix_lens)
    q = torch.empty((rows, num_qo_heads, 128), dtype=dt, device=device)
    _fill_randn_(q, gen)
    sk = torch.randn(num_qo_heads, generator=gen, dtype=torch.float32, device=device) if sinks else None
    k_pool, v_pool = cache.unbind(1)
    return CascadeWorkload(
        k_pool=k_pool, v_pool=v_pool, q=q, sinks=sk, prefix_len=prefix_len,
        prefix_indices=pre_idx, prefix_last_page_len=page_size,
        qo_indptr=np.arange(len(suffix_lens) + 1, dtype=np.int32) * q_len,
        suffix_kv_indptr=suf_indptr, suffix_indices=suf_idx, suffix_last_page_len=lpl,
        flat_kv_indptr=flat_indptr, flat_indices=np.concatenate(flat).astype(np.int32),
        flat_last_page_len=lpl.copy(), num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
        page_size=page_size)
