"""GPU parity of the cascade merge (C ABI pod_merge_states) and of a two-level
shared-prefix cascade built from one fused launch plus the merge.

The merge is checked against the oracle's merge_states / apply_sink on random
states (rows with one or both sides empty, in-place output, ragged sizes). The
cascade runs the shared prefix as the prefill role (one request holding every
query row, non-causal: the whole prefix precedes each row's diagonal) and each
request's own suffix as the decode role (bottom-right causal), merges the two
states with the sink applied once, and is compared with the oracle's plain
attention over prefix + suffix. Tolerances as for the fused launch."""
import numpy as np
import pytest
import torch

import oracle
from serving_attention_amd import BatchPOD, merge_states

from gpu_helpers import TOL_LSE, TOL_O, log

pytestmark = pytest.mark.gpu

DT = {"f16": torch.float16, "bf16": torch.bfloat16}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")


def random_states(rows, heads, dtype, gen, empty_frac=0.1):
    o = torch.randn(rows, heads, 128, generator=gen, device="cuda").to(dtype)
    lse = torch.empty(rows, heads, device="cuda").uniform_(-6.0, 24.0, generator=gen)
    drop = torch.rand(rows, heads, generator=gen, device="cuda") < empty_frac
    lse[drop] = -float("inf")
    return o, lse


@pytest.mark.parametrize("dt,rows,heads,sinks,inplace", [
    ("bf16", 1, 1, False, False),
    ("bf16", 37, 8, True, False),
    ("f16", 333, 64, False, True),
    ("bf16", 1024, 64, True, True),
])
def test_merge_states_against_oracle(dt, rows, heads, sinks, inplace):
    log(f"case: merge {dt} rows={rows} heads={heads} sinks={sinks} inplace={inplace}")
    gen = torch.Generator(device="cuda").manual_seed(rows * 7 + heads)
    oa, la = random_states(rows, heads, DT[dt], gen)
    ob, lb = random_states(rows, heads, DT[dt], gen)
    if rows > 1:
        la[0, :] = -float("inf")      # a row with both sides empty
        lb[0, :] = -float("inf")
    sk = torch.randn(heads, generator=gen, device="cuda") if sinks else None
    ref_o, ref_l = oracle.merge_states([(oa.double().cpu().numpy(), la.double().cpu().numpy()),
                                        (ob.double().cpu().numpy(), lb.double().cpu().numpy())])
    if sinks:
        ref_o = oracle.apply_sink(ref_o, ref_l, sk.double().cpu().numpy()[None, :])
    oa_h = oa.clone()
    out, lse = merge_states(oa, la, ob, lb, sinks=sk, out=oa if inplace else None,
                            lse_out=la if inplace else None)
    torch.cuda.synchronize()
    go = out.double().cpu().numpy()
    gl = lse.double().cpu().numpy()
    assert np.all(np.isfinite(go))
    eo = float(np.abs(go - ref_o).max())
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(gl), fin)
    el = float(np.abs(gl[fin] - ref_l[fin]).max()) if fin.any() else 0.0
    log(f"merge: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O[dt] and el <= TOL_LSE
    if rows > 1:
        assert np.all(go[0] == 0.0)
    if not inplace:
        assert torch.equal(oa, oa_h)


def pages_of(n_keys, ps):
    return -(-n_keys // ps), (n_keys - 1) % ps + 1


def cascade_case(dt, prefix, q_lens, suffixes, hqo, hkv, ps, sinks, seed):
    """Run the two-level cascade and return what the test compares."""
    dev = "cuda"
    rng = np.random.default_rng(seed)
    gen = torch.Generator(device=dev).manual_seed(1000 + seed)
    n_pre, lpl_pre = pages_of(prefix, ps)
    suf = [pages_of(s, ps) for s in suffixes]
    total = n_pre + sum(n for n, _ in suf) + 3
    perm = rng.permutation(total)                       # physical page of each logical page
    pre_idx = perm[:n_pre]
    suf_idx, at = [], n_pre
    for n, _ in suf:
        suf_idx.append(perm[at:at + n])
        at += n
    k_pool = torch.randn(total, ps, hkv, 128, generator=gen, device=dev).to(DT[dt])
    v_pool = torch.randn(total, ps, hkv, 128, generator=gen, device=dev).to(DT[dt])
    rows = int(sum(q_lens))
    q = torch.randn(rows, hqo, 128, generator=gen, device=dev).to(DT[dt])
    sk = torch.randn(hqo, generator=gen, device=dev) if sinks else None

    ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)
    pod = BatchPOD(ws, "NHD", int_workspace_bytes=8 << 20)
    qo_d = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    kv_d = np.concatenate([[0], np.cumsum([n for n, _ in suf])]).astype(np.int32)
    lpl_d = np.array([l for _, l in suf], np.int32)
    pod.plan([0, rows], [0, n_pre], [lpl_pre], qo_d, kv_d, lpl_d,
             num_qo_heads=hqo, num_kv_heads=hkv, head_dim=128, page_size=ps, dtype=DT[dt],
             causal_p=False, causal_d=True)
    idx_p = torch.from_numpy(pre_idx.astype(np.int32)).to(dev)
    idx_d = torch.from_numpy(np.concatenate(suf_idx).astype(np.int32)).to(dev)
    (op, lp), (od, ld) = pod.run(q, (k_pool, v_pool), idx_p, q, (k_pool, v_pool), idx_d,
                                 return_lse=True)
    o, lse = merge_states(op, lp, od, ld, sinks=sk)
    torch.cuda.synchronize()
    return dict(k_pool=k_pool, v_pool=v_pool, q=q, sinks=sk, pre_idx=pre_idx, suf_idx=suf_idx,
                o=o, lse=lse)


@pytest.mark.parametrize("dt,prefix,q_lens,suffixes,hqo,hkv,ps,sinks", [
    ("bf16", 1000, [1, 3, 1, 4, 2], [17, 40, 1, 100, 2], 16, 4, 16, False),
    ("f16", 333, [2, 1, 1], [5, 70, 1], 8, 2, 5, True),
    ("bf16", 4096, [1] * 64, list(range(16, 16 + 64 * 9, 9)), 64, 8, 16, True),
])
def test_shared_prefix_cascade_against_oracle(dt, prefix, q_lens, suffixes, hqo, hkv, ps, sinks):
    log(f"case: cascade {dt} prefix={prefix} requests={len(q_lens)} heads={hqo}/{hkv} ps={ps} sinks={sinks}")
    c = cascade_case(dt, prefix, q_lens, suffixes, hqo, hkv, ps, sinks, seed=len(q_lens) + prefix)
    kp = c["k_pool"].double().cpu().numpy()
    vp = c["v_pool"].double().cpu().numpy()
    q = c["q"].double().cpu().numpy()
    go = c["o"].double().cpu().numpy()
    gl = c["lse"].double().cpu().numpy()
    sk = c["sinks"].double().cpu().numpy() if sinks else None
    assert np.all(np.isfinite(go))
    flat = lambda pool, idx, n: pool[idx].reshape(-1, hkv, 128)[:n]
    k_pre = flat(kp, c["pre_idx"], prefix)
    v_pre = flat(vp, c["pre_idx"], prefix)
    worst_o = worst_l = 0.0
    r0 = 0
    for b, (ql, s) in enumerate(zip(q_lens, suffixes)):
        k = np.concatenate([k_pre, flat(kp, c["suf_idx"][b], s)])
        v = np.concatenate([v_pre, flat(vp, c["suf_idx"][b], s)])
        keep = oracle.valid_key_mask(ql, prefix + s, True, -1)
        ro, rl = oracle.attend_rows(q[r0:r0 + ql], k, v, keep, 1.0 / np.sqrt(128.0), sk)
        worst_o = max(worst_o, float(np.abs(go[r0:r0 + ql] - ro).max()))
        worst_l = max(worst_l, float(np.abs(gl[r0:r0 + ql] - rl).max()))
        r0 += ql
    log(f"cascade: max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}")
    assert worst_o <= TOL_O[dt] and worst_l <= TOL_LSE
