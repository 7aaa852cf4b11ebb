"""GPU parity over a fixed list of mixed configurations drawn once from a seeded
generator: group sizes 1-128, page sizes 1-64 (powers of two and not), both
layouts, windows, causal and non-causal roles, sinks, FP8 decode caches, split
sizes and item orders in combinations the hand-written cases do not reach.
Every row of every request is compared with the fp64 oracle."""
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


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 3, 8, 16, 64, 128]))
        if hkv * g > 512:
            hkv = max(1, 512 // g)
        ps = int(rng.choice([1, 5, 16, 48, 64]))
        fp8 = bool(rng.random() < 0.3)
        dtype = str(rng.choice(["bf16", "f16"]))
        roles = {}
        for role in ("prefill", "decode"):
            if rng.random() < 0.15:
                roles[role] = None
                continue
            causal = bool(rng.random() < 0.7)
            w = int(rng.choice([-1, -1, 0, 9, 150]))
            n_req = int(rng.integers(1, 5))
            if role == "prefill":
                q = rng.integers(0, 160, n_req).tolist()
            else:
                q = rng.integers(1, 6, n_req).tolist()
            kv = [int(max(k, qq if causal else 1)) for k, qq in zip(rng.integers(1, 900, n_req), q)]
            roles[role] = RoleSpec([int(x) for x in q], kv, causal=causal, window_left=w)
        if roles["prefill"] is None and roles["decode"] is None:
            roles["decode"] = RoleSpec([1], [300], causal=True, window_left=-1)
        if fp8 and roles["decode"] is None:
            fp8 = False
        out.append(dict(
            spec=WorkloadSpec(
                name=f"mixed{i}", prefill=roles["prefill"], decode=roles["decode"],
                num_qo_heads=hkv * g, num_kv_heads=hkv, page_size=ps, dtype=dtype,
                sinks=bool(rng.random() < 0.4), pool="separate" if fp8 else str(rng.choice(["shared", "separate"])),
                shuffle_pages=True, spare_pages=2, kv_layout=str(rng.choice(["NHD", "HND"])),
                meta_seed=500 + i, value_seed=600 + i,
                decode_kv_dtype="fp8_e4m3" if fp8 else None,
                fp8_scales=(float(rng.choice([0.5, 1.0])), float(rng.choice([0.75, 1.0])), float(rng.choice([1.0, 1.25])))
                if fp8 else (1.0, 1.0, 1.0)),
            chunk=int(rng.choice([0, 0, 64, 192, -1])), order=int(rng.integers(0, 4))))
    return out


CASES = _cases()


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[str(i) for i in range(len(CASES))])
def test_mixed_case(idx):
    c = CASES[idx]
    spec = c["spec"]
    log(f"case: mixed {idx}: heads {spec.num_qo_heads}/{spec.num_kv_heads} ps {spec.page_size} "
        f"{spec.dtype} {spec.kv_layout} sinks {spec.sinks} fp8 {spec.decode_kv_dtype} "
        f"prefill {spec.prefill} decode {spec.decode} chunk {c['chunk']} order {c['order']}")
    w = build(spec, device="cuda")
    roles = tuple(n for n, r in (("prefill", w.prefill), ("decode", w.decode)) if r is not None)
    res, pod = plan_and_run(w, roles=roles, decode_chunk=c["chunk"], order=c["order"])
    log(f"plan: {pod.plan_info()}")
    (op, lp), (od, ld) = res
    if w.prefill is not None:
        assert_close(w, compare_role(w, w.prefill, op, lp, tag=f"mixed{idx}/prefill"), f"mixed{idx}/prefill")
    if w.decode is not None:
        assert_close(w, compare_role(w, w.decode, od, ld, tag=f"mixed{idx}/decode"), f"mixed{idx}/decode")
