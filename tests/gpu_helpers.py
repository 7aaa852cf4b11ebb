"""Shared helpers of the GPU parity tests: run the fused launch through the
Python binding (C ABI) and compare against the fp64 oracle request by request."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from serving_attention_amd import BatchPOD

TOL_O = {"f16": 5e-3, "bf16": 2e-2}
TOL_LSE = 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def plan_and_run(w, roles=("prefill", "decode"), decode_chunk=0, order=0, ws_mb=256,
                 return_lse=True, pod=None, poison_out=False, identity_pages_d=False):
    spec = w.spec
    p = w.prefill if "prefill" in roles else None
    d = w.decode if "decode" in roles else None
    if pod is None:
        ws = torch.empty(ws_mb << 20, dtype=torch.uint8, device="cuda")
        pod = BatchPOD(ws, spec.kv_layout, int_workspace_bytes=16 << 20)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[spec.dtype]
    pod.plan(p.qo_indptr if p else None, p.kv_indptr if p else None, p.last_page_len if p else None,
             d.qo_indptr if d else None, d.kv_indptr if d else None, d.last_page_len if d else None,
             num_qo_heads=spec.num_qo_heads, num_kv_heads=spec.num_kv_heads,
             head_dim=spec.head_dim, page_size=spec.page_size, dtype=dt,
             causal_p=p.causal if p else True, causal_d=d.causal if d else True,
             window_left_p=p.window_left if p else -1, window_left_d=d.window_left if d else -1,
             sm_scale_p=p.sm_scale if p else None, sm_scale_d=d.sm_scale if d else None,
             sinks=spec.sinks, decode_chunk=decode_chunk, order=order,
             kv_dtype_d=torch.float8_e4m3fn if spec.decode_kv_dtype == "fp8_e4m3" else None)
    outs = {}
    for name, r in (("p", p), ("d", d)):
        if r is None:
            outs[name] = (None, None)
            continue
        o = torch.empty_like(r.q)
        l = torch.empty(r.q.shape[:2], dtype=torch.float32, device=r.q.device)
        if poison_out:
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        outs[name] = (o, l)
    res = pod.run(p.q if p else None, p.kv_cache if p else None, p.kv_indices_dev if p else None,
                  d.q if d else None, d.kv_cache if d else None,
                  d.kv_indices_dev if d is not None and not identity_pages_d else None,
                  sinks=w.sinks if spec.sinks else None, return_lse=return_lse,
                  out_p=outs["p"][0], out_d=outs["d"][0],
                  lse_p=outs["p"][1] if return_lse else None, lse_d=outs["d"][1] if return_lse else None,
                  **fp8_scale_args(spec))
    torch.cuda.synchronize()
    return res, pod


def fp8_scale_args(spec):
    if spec.decode_kv_dtype != "fp8_e4m3":
        return {}
    qs, ks, vs = spec.fp8_scales
    return dict(q_scale_d=qs, k_scale_d=ks, v_scale_d=vs)


def oracle_request(w, role, b, rows=None):
    """fp64 oracle for request b of a role (optionally some of its rows).

    Copies only the request's own pages to the host and renumbers them, which
    leaves the result unchanged (page-permutation invariance of the oracle).
    With a window it also leaves out the whole pages before the earliest key
    any of the rows sees, shortening kv_len by as much: each row keeps its
    diagonal key, and the dropped keys weigh exactly zero (pinned on the CPU
    by the oracle tests)."""
    spec = w.spec
    p0, p1 = int(role.kv_indptr[b]), int(role.kv_indptr[b + 1])
    q0, q1 = int(role.qo_indptr[b]), int(role.qo_indptr[b + 1])
    if role.window_left >= 0 and q1 > q0:
        kv_len = (p1 - p0 - 1) * spec.page_size + int(role.last_page_len[b])
        # earliest key of the request's first row (kv_len' >= q_len + window_left
        # stays, so every row keeps its whole window)
        lo = max(0, kv_len - (q1 - q0) - role.window_left)
        p0 += min(lo // spec.page_size, p1 - p0 - 1)
    pages = torch.from_numpy(role.kv_indices[p0:p1].astype(np.int64)).to(role.k_pool.device)
    fp8 = role is w.decode and spec.decode_kv_dtype == "fp8_e4m3"
    qs, ks, vs = spec.fp8_scales if fp8 else (1.0, 1.0, 1.0)
    if fp8:   # the oracle's own E4M3 decoding of the stored bytes
        kp = oracle.e4m3_to_float(role.k_pool.view(torch.uint8).index_select(0, pages).cpu().numpy())
        vp = oracle.e4m3_to_float(role.v_pool.view(torch.uint8).index_select(0, pages).cpu().numpy())
    else:
        kp = role.k_pool.index_select(0, pages).float().cpu().numpy()
        vp = role.v_pool.index_select(0, pages).float().cpu().numpy()
    q = role.q[q0:q1].float().cpu().numpy()
    sinks = w.sinks.cpu().numpy() if spec.sinks else None
    res = oracle.attend_role(
        q, kp, vp, np.array([0, q1 - q0]), np.array([0, p1 - p0]), None,
        role.last_page_len[b:b + 1], spec.page_size, spec.num_qo_heads, spec.num_kv_heads,
        role.causal, role.window_left, role.sm_scale * qs * ks, sinks, layout=spec.kv_layout,
        rows_of=(lambda _: rows) if rows is not None else None)
    ids, ro, rl = res[0]
    # attend_rows_fp8_scaled's definition: q_scale * k_scale on the scores,
    # v_scale on the output
    return ids, ro * vs, rl


def compare_role(w, role, out, lse, requests=None, rows_of=None, tag=""):
    """Max errors of out / lse against the oracle over the given requests and rows."""
    spec = w.spec
    reqs = range(role.batch) if requests is None else requests
    worst_o, worst_l = 0.0, 0.0
    out_h = out.float().cpu().numpy()
    lse_h = lse.cpu().numpy() if lse is not None else None
    for b in reqs:
        q0, q1 = int(role.qo_indptr[b]), int(role.qo_indptr[b + 1])
        if q1 == q0:
            continue
        rows = rows_of(b) if rows_of is not None else None
        ids, ro, rl = oracle_request(w, role, b, rows)
        go = out_h[q0 + ids]
        assert np.all(np.isfinite(go)), f"{tag} request {b}: non-finite output"
        worst_o = max(worst_o, float(np.abs(go - ro).max()))
        if lse_h is not None:
            gl = lse_h[q0 + ids]
            worst_l = max(worst_l, float(np.abs(gl - rl).max()))
    return worst_o, worst_l


def assert_close(w, errs, tag=""):
    eo, el = errs
    log(f"{tag}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O[w.spec.dtype], f"{tag}: O error {eo} > {TOL_O[w.spec.dtype]}"
    assert el <= TOL_LSE, f"{tag}: LSE error {el} > {TOL_LSE}"
