"""The correctness grid of the POD article ("正确性验证：测试如何对标参考实现"):
a prefill of 127 or 12288 tokens fused with a decode batch of 1, 17 or 127
requests, page_size 1 or 16, 8 or 32 query heads, each fused result compared
element by element with an independent reference (here the fp64 oracle, per
role).

Readings where the passage leaves values open: the prefill is one causal
request with kv_len = qo_len (the single-request prefill of that test); the
decode requests hold one query token each with kv lengths drawn uniformly from
[1, 4096] (seeded); "8/32 heads" is the number of query heads, over 8 kv heads
(groups 1 and 4); values are fp16 N(0,1). Every decode row is checked; the
12288-token prefill is checked on rows at tile edges plus random rows, the
127-token prefill on every row."""
import itertools

import numpy as np
import pytest
import torch

from workloads import RoleSpec, WorkloadSpec, build

from gpu_helpers import assert_close, compare_role, log, plan_and_run

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")


GRID = list(itertools.product((127, 12288), (1, 17, 127), (1, 16), (8, 32)))


def edge_rows(n, rng):
    rows = {0, 1, 31, 32, 33, 63, 64, 255, 256, n // 2, n - 33, n - 32, n - 2, n - 1}
    rows |= set(rng.integers(0, n, 24).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n))


@pytest.mark.parametrize("p_len,d_batch,ps,hqo", GRID,
                         ids=[f"p{a}-d{b}-ps{c}-h{d}" for a, b, c, d in GRID])
def test_pages_grid(p_len, d_batch, ps, hqo):
    seed = GRID.index((p_len, d_batch, ps, hqo))
    rng = np.random.default_rng(900 + seed)
    kv_d = [int(x) for x in rng.integers(1, 4097, d_batch)]
    spec = WorkloadSpec(
        name="pages_grid", prefill=RoleSpec([p_len], [p_len], causal=True),
        decode=RoleSpec([1] * d_batch, kv_d, causal=True),
        num_qo_heads=hqo, num_kv_heads=8, page_size=ps, dtype="f16", pool="separate",
        shuffle_pages=True, spare_pages=2, meta_seed=1900 + seed, value_seed=2900 + seed)
    log(f"case: pages grid prefill {p_len}, decode batch {d_batch}, page_size {ps}, {hqo}/8 heads")
    w = build(spec, device="cuda")
    res, pod = plan_and_run(w)
    log(f"plan: {pod.plan_info()}")
    (op, lp), (od, ld) = res
    rows_of = (lambda b: edge_rows(p_len, rng)) if p_len > 1024 else None
    assert_close(w, compare_role(w, w.prefill, op, lp, rows_of=rows_of, tag="grid/prefill"), "grid/prefill")
    assert_close(w, compare_role(w, w.decode, od, ld, tag="grid/decode"), "grid/decode")
    del w
    torch.cuda.empty_cache()
