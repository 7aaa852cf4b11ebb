"""pod_run_static, the entry point for callers that cannot allocate (its work
list and split-KV partial states live in the library's static device scratch),
against pod_plan + pod_run on the same inputs: the same kernel over the same
plan, so the outputs must agree bit for bit (stricter than the parity
tolerances). Two calls in a row, the second with a smaller input, so the second
call finds the first one's contents in the scratch; both are also checked
against the fp64 oracle."""
import numpy as np
import pytest
import torch

from serving_attention_amd import _lib, run_static
from workloads import RoleSpec, WorkloadSpec, build

from gpu_helpers import assert_close, compare_role, log, plan_and_run

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")


def spec(name, p_q, p_kv, d_q, d_kv, seed):
    return WorkloadSpec(
        name=name, prefill=RoleSpec(list(p_q), list(p_kv), causal=True, window_left=300),
        decode=RoleSpec(list(d_q), list(d_kv), causal=True, window_left=300),
        num_qo_heads=16, num_kv_heads=4, page_size=16, dtype="bf16", sinks=True, pool="shared",
        shuffle_pages=True, spare_pages=3, meta_seed=700 + seed, value_seed=800 + seed)


def static_call(w, decode_chunk):
    p, d = w.prefill, w.decode
    outs = [torch.full_like(r.q, float("nan")) for r in (p, d)]
    lses = [torch.full(r.q.shape[:2], float("nan"), device="cuda") for r in (p, d)]
    res = run_static(p.qo_indptr, p.kv_indptr, p.last_page_len, d.qo_indptr, d.kv_indptr, d.last_page_len,
                     p.q, p.kv_cache, p.kv_indices_dev, d.q, d.kv_cache, d.kv_indices_dev,
                     num_qo_heads=16, num_kv_heads=4, head_dim=128, page_size=16, dtype=torch.bfloat16,
                     window_left_p=300, window_left_d=300, decode_chunk=decode_chunk, sinks=w.sinks,
                     return_lse=True, out_p=outs[0], lse_p=lses[0], out_d=outs[1], lse_d=lses[1])
    torch.cuda.synchronize()
    return res


def test_static_entry_matches_plan_and_run():
    big = build(spec("static_big", (300, 77, 1), (900, 77, 40), (1, 3, 2, 4, 1, 1), (2049, 700, 65, 3000, 1, 513), 1),
                device="cuda")
    small = build(spec("static_small", (40,), (130,), (2, 1), (300, 90), 2), device="cuda")
    for tag, w, chunk in (("first call", big, 128), ("second call, smaller", small, 64)):
        log(f"case: pod_run_static {tag}")
        ref, pod = plan_and_run(w, decode_chunk=chunk)
        info = pod.plan_info()
        assert info["n_groups"] > 0          # split chunks use the partial states
        got = static_call(w, chunk)
        for (a, la), (b, lb) in zip(ref, got):
            assert torch.equal(a, b) and torch.equal(la, lb), tag
        (op, lp), (od, ld) = got
        assert_close(w, compare_role(w, w.prefill, op, lp, tag=tag + "/prefill"), tag + "/prefill")
        assert_close(w, compare_role(w, w.decode, od, ld, tag=tag + "/decode"), tag + "/decode")


def test_static_entry_refuses_plans_above_its_limits():
    # 8 kv heads x 262144 keys in 64-key splits: 32768 partial states (541 MB)
    log("case: pod_run_static above the static limits")
    q = torch.zeros(1, 8, 128, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(262144, 2, 1, 8, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(_lib.PodError) as ex:
        run_static(None, None, None, [0, 1], [0, 262144], [1], None, None, None, q, kv, None,
                   num_qo_heads=8, num_kv_heads=8, head_dim=128, page_size=1, causal_d=False,
                   decode_chunk=64, out_d=out)
    assert ex.value.code == _lib.POD_ERR_WORKSPACE and "static limit" in str(ex.value)
