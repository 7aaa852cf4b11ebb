"""GPU: graph-mode contexts (POD article, "CUDAGraph 模式的运行时约束").

A run() captured once into a HIP graph (torch.cuda.CUDAGraph) is replayed after
new plans with other lengths (same batch sizes) and new page tables and queries
written into the captured buffers. Every replay must equal, bit for bit, an
ordinary context's eager launch on the same inputs, and one replay is also
compared with the fp64 oracle. Eager work and synchronisations sit between the
replays. Plans that change the fixed batch or the plan-time policy are refused."""
import numpy as np
import pytest
import torch

import oracle
from serving_attention_amd import BatchPOD

from gpu_helpers import TOL_LSE, TOL_O, log

pytestmark = pytest.mark.gpu

H_QO, H_KV, D, PS = 16, 4, 128, 16
P_BATCH, D_BATCH = 2, 6
CAP_P_ROWS, CAP_D_ROWS = 320, 12
POOL_PAGES = 400


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")


def step_inputs(seed):
    """Lengths and page tables of one step (fixed batch sizes)."""
    rng = np.random.default_rng(seed)
    p_q = rng.integers(1, 150, P_BATCH)
    p_kv = p_q + rng.integers(0, 400, P_BATCH)
    d_q = rng.integers(1, 3, D_BATCH)
    d_kv = d_q + rng.integers(0, 700, D_BATCH)
    pages = lambda kv: [-(-int(k) // PS) for k in kv]
    lpl = lambda kv: [(int(k) - 1) % PS + 1 for k in kv]
    pp, dp = pages(p_kv), pages(d_kv)
    perm = rng.permutation(POOL_PAGES)[:sum(pp) + sum(dp)].astype(np.int32)
    return dict(
        p=dict(qo=np.concatenate([[0], np.cumsum(p_q)]).astype(np.int32),
               kv=np.concatenate([[0], np.cumsum(pp)]).astype(np.int32),
               lpl=np.array(lpl(p_kv), np.int32), idx=perm[:sum(pp)], q_lens=p_q, kv_lens=p_kv),
        d=dict(qo=np.concatenate([[0], np.cumsum(d_q)]).astype(np.int32),
               kv=np.concatenate([[0], np.cumsum(dp)]).astype(np.int32),
               lpl=np.array(lpl(d_kv), np.int32), idx=perm[sum(pp):], q_lens=d_q, kv_lens=d_kv))


def plan(pod, s, **over):
    kw = dict(num_qo_heads=H_QO, num_kv_heads=H_KV, head_dim=D, page_size=PS, dtype=torch.bfloat16,
              causal_p=True, causal_d=True)
    kw.update(over)
    pod.plan(s["p"]["qo"], s["p"]["kv"], s["p"]["lpl"], s["d"]["qo"], s["d"]["kv"], s["d"]["lpl"], **kw)


def test_graph_replay_across_plans():
    dev = "cuda"
    gen = torch.Generator(device=dev).manual_seed(5)
    pool = torch.randn(POOL_PAGES, 2, PS, H_KV, D, generator=gen, device=dev).to(torch.bfloat16)
    kv = (pool[:, 0], pool[:, 1])
    q_p = torch.zeros(CAP_P_ROWS, H_QO, D, dtype=torch.bfloat16, device=dev)
    q_d = torch.zeros(CAP_D_ROWS, H_QO, D, dtype=torch.bfloat16, device=dev)
    idx_p = torch.zeros(POOL_PAGES, dtype=torch.int32, device=dev)
    idx_d = torch.zeros(POOL_PAGES, dtype=torch.int32, device=dev)
    o_p, l_p = torch.zeros_like(q_p), torch.zeros(CAP_P_ROWS, H_QO, device=dev)
    o_d, l_d = torch.zeros_like(q_d), torch.zeros(CAP_D_ROWS, H_QO, device=dev)

    def load(s, seed):
        g2 = torch.Generator(device=dev).manual_seed(seed)
        q_p.copy_(torch.randn(q_p.shape, generator=g2, device=dev).to(torch.bfloat16))
        q_d.copy_(torch.randn(q_d.shape, generator=g2, device=dev).to(torch.bfloat16))
        idx_p[:len(s["p"]["idx"])].copy_(torch.from_numpy(s["p"]["idx"]))
        idx_d[:len(s["d"]["idx"])].copy_(torch.from_numpy(s["d"]["idx"]))

    gpod = BatchPOD(torch.empty(32 << 20, dtype=torch.uint8, device=dev), "NHD", int_workspace_bytes=4 << 20,
                    use_cuda_graph=True, prefill_batch_size=P_BATCH, decode_batch_size=D_BATCH)
    epod = BatchPOD(torch.empty(32 << 20, dtype=torch.uint8, device=dev), "NHD", int_workspace_bytes=4 << 20)

    def run_graph_ctx():
        gpod.run(q_p, kv, idx_p, q_d, kv, idx_d, return_lse=True, out_p=o_p, lse_p=l_p, out_d=o_d, lse_d=l_d)

    s0 = step_inputs(0)
    load(s0, 100)
    plan(gpod, s0)
    run_graph_ctx()                     # eager warm-up
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_graph_ctx()
    torch.cuda.synchronize()

    for step in range(4):
        s = step_inputs(step)
        load(s, 100 + step)
        plan(gpod, s)
        for rep in range(2):
            o_p.fill_(float("nan"))
            o_d.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            _ = (q_p.float() * 2).sum().item()   # eager work between replays
            rows_p, rows_d = int(s["p"]["qo"][-1]), int(s["d"]["qo"][-1])
            plan(epod, s)
            (eo_p, el_p), (eo_d, el_d) = epod.run(q_p[:rows_p], kv, idx_p, q_d[:rows_d], kv, idx_d,
                                                  return_lse=True)
            torch.cuda.synchronize()
            log(f"step {step} replay {rep}: prefill rows {rows_p}, decode rows {rows_d}")
            assert torch.equal(o_p[:rows_p], eo_p) and torch.equal(l_p[:rows_p], el_p)
            assert torch.equal(o_d[:rows_d], eo_d) and torch.equal(l_d[:rows_d], el_d)

    # the last replay against the oracle, request by request
    kp = pool[:, 0].double().cpu().numpy()
    vp = pool[:, 1].double().cpu().numpy()
    worst_o = worst_l = 0.0
    for name, out, lse, q in (("p", o_p, l_p, q_p), ("d", o_d, l_d, q_d)):
        r = s[name]
        qh = q.double().cpu().numpy()
        go, gl = out.double().cpu().numpy(), lse.double().cpu().numpy()
        for b in range(len(r["q_lens"])):
            q0, q1 = int(r["qo"][b]), int(r["qo"][b + 1])
            pg = r["idx"][r["kv"][b]:r["kv"][b + 1]]
            n = int(r["kv_lens"][b])
            k = kp[pg].reshape(-1, H_KV, D)[:n]
            v = vp[pg].reshape(-1, H_KV, D)[:n]
            keep = oracle.valid_key_mask(q1 - q0, n, True, -1)
            ro, rl = oracle.attend_rows(qh[q0:q1], k, v, keep, 1.0 / np.sqrt(D))
            worst_o = max(worst_o, float(np.abs(go[q0:q1] - ro).max()))
            worst_l = max(worst_l, float(np.abs(gl[q0:q1] - rl).max()))
    log(f"graph replay vs oracle: max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}")
    assert worst_o <= TOL_O["bf16"] and worst_l <= TOL_LSE


def test_graph_mode_plan_checks():
    dev = "cuda"
    gpod = BatchPOD(torch.empty(8 << 20, dtype=torch.uint8, device=dev), "NHD", int_workspace_bytes=1 << 20,
                    use_cuda_graph=True, prefill_batch_size=P_BATCH, decode_batch_size=D_BATCH)
    s = step_inputs(1)
    plan(gpod, s)
    bad = step_inputs(2)
    bad["d"] = dict(bad["d"], qo=bad["d"]["qo"][:-1], kv=bad["d"]["kv"][:-1], lpl=bad["d"]["lpl"][:-1])
    with pytest.raises(ValueError, match="batch"):
        plan(gpod, bad)
    with pytest.raises(ValueError, match="first plan"):
        plan(gpod, s, causal_d=False)
    with pytest.raises(ValueError, match="first plan"):
        plan(gpod, s, window_left_p=8)
    plan(gpod, step_inputs(3))   # same batch and policy: accepted
