"""GPU parity of the FP8 (E4M3) decode KV cache against the fp64 oracle.

The decode role reads K/V stored as FP8 E4M3 bytes, with the calibration scales
of the POD article ("Decode 侧参数与'plan 覆盖'行为": q_scale * k_scale multiply the decode
sm_scale, v_scale the decode output); q, the prefill K/V and the outputs keep
the query dtype. The oracle decodes the stored bytes itself (pinned against
torch's float8_e4m3fn) and applies the scales by their definition. Tolerances
as for the query dtype: the FP8 values are widened exactly, so only the
attention arithmetic differs."""
import dataclasses

import numpy as np
import pytest
import torch

from serving_attention_amd import BatchPOD
from workloads import RoleSpec, WorkloadSpec, build, named_spec

from gpu_helpers import assert_close, compare_role, log, plan_and_run

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")


def fp8_spec(dtype="bf16", ps=16, hqo=16, hkv=4, w=-1, sinks=False, dq=1, scales=(1.0, 0.75, 1.25),
             d_kv=(1, 16, 17, 100, 513, 1000, 2049), p_q=(127, 33), p_kv=(127, 300), seed=0, layout="NHD"):
    return WorkloadSpec(
        name="fp8", prefill=RoleSpec(list(p_q), list(p_kv), causal=True, window_left=w) if p_q else None,
        decode=RoleSpec([dq] * len(d_kv), [max(k, dq) for k in d_kv], causal=True, window_left=w),
        num_qo_heads=hqo, num_kv_heads=hkv, page_size=ps, dtype=dtype, sinks=sinks, pool="separate",
        shuffle_pages=True, spare_pages=2, kv_layout=layout, meta_seed=300 + seed, value_seed=400 + seed,
        decode_kv_dtype="fp8_e4m3", fp8_scales=scales)


CASES = [
    dict(),
    dict(dtype="f16", ps=1, scales=(0.5, 2.0, 0.25)),
    dict(ps=5, hqo=8, hkv=8, sinks=True),
    dict(hqo=32, hkv=4, dq=4, w=37, sinks=True),          # 32 rows per item, window, sinks
    dict(layout="HND", scales=(1.0, 1.0, 1.0), p_q=()),
    # more than 32 rows per (request, kv head): key chunks in 32-row slices
    dict(hqo=64, hkv=1, dq=1),                              # group 64: two slices
    dict(hqo=16, hkv=2, dq=5, w=300, sinks=True),           # 8 x 5 = 40 rows: 32 + 8
    dict(hqo=128, hkv=2, dq=2, ps=1, scales=(0.5, 2.0, 1.5)),  # 64 x 2 = 128 rows: four slices
    dict(hqo=64, hkv=2, dq=1, layout="HND", w=100, sinks=True, p_q=()),  # slices over HND pools
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[str(i) for i in range(len(CASES))])
@pytest.mark.parametrize("decode_chunk", [0, 64, -1])
def test_fp8_decode_small(idx, decode_chunk):
    spec = fp8_spec(seed=idx, **CASES[idx])
    log(f"case: fp8 decode #{idx} {CASES[idx]} decode_chunk={decode_chunk}")
    w = build(spec, device="cuda")
    res, _ = plan_and_run(w, decode_chunk=decode_chunk)
    (op, lp), (od, ld) = res
    if w.prefill is not None:
        assert_close(w, compare_role(w, w.prefill, op, lp, tag="fp8/prefill"), "fp8/prefill")
    assert_close(w, compare_role(w, w.decode, od, ld, tag="fp8/decode"), "fp8/decode")


def test_fp8_unit_scales_equal_bf16_of_same_values():
    # FP8 values widened exactly: with unit scales the FP8 launch equals a bf16
    # launch over the same (widened) pool bit for bit
    spec = fp8_spec(scales=(1.0, 1.0, 1.0), p_q=(), d_kv=(40, 300, 2049))
    w = build(spec, device="cuda")
    res8, _ = plan_and_run(w, roles=("decode",))
    wb = dataclasses.replace(w, spec=dataclasses.replace(spec, decode_kv_dtype=None))
    d = w.decode
    kb = d.kv_cache.to(torch.bfloat16)
    wb.decode = dataclasses.replace(d, kv_cache=kb, k_pool=kb.unbind(1)[0], v_pool=kb.unbind(1)[1])
    resb, _ = plan_and_run(wb, roles=("decode",))
    assert torch.equal(res8[1][0], resb[1][0]) and torch.equal(res8[1][1], resb[1][1])


def test_fp8_plan_checks():
    ws = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    pod = BatchPOD(ws, "NHD", int_workspace_bytes=1 << 20)
    # 64 rows per decode request (group 64): planned as two 32-row key-chunk slices
    pod.plan(None, None, None, [0, 1], [0, 4], [16], num_qo_heads=64, num_kv_heads=1, head_dim=128,
             page_size=16, dtype=torch.bfloat16, kv_dtype_d=torch.float8_e4m3fn)
    assert pod.plan_info()["n_decode_items"] == 2
    # no page table
    pod.plan(None, None, None, [0, 1], [0, 4], [16], num_qo_heads=8, num_kv_heads=1, head_dim=128,
             page_size=16, dtype=torch.bfloat16, kv_dtype_d=torch.float8_e4m3fn)
    kv = torch.zeros(4, 2, 16, 1, 128, device="cuda").to(torch.float8_e4m3fn)
    q = torch.zeros(1, 8, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="kv_indices"):
        pod.run(None, None, None, q, kv, None)


def test_named_pod_fp8():
    log("case: named workload pod_fp8 (full size)")
    w = build(named_spec("pod_fp8"), device="cuda")
    res, pod = plan_and_run(w)
    (op, lp), (od, ld) = res
    rng = np.random.default_rng(9)
    # the bf16 prefill role on sampled rows (tile edges plus random rows), every
    # FP8 decode request
    rows = lambda b: np.array(sorted({0, 1, 31, 32, 63, 64, 1023, 1024, 2046, 2047} |
                                     set(rng.integers(0, 2048, 30).tolist())))
    assert_close(w, compare_role(w, w.prefill, op, lp, rows_of=rows, tag="pod_fp8/prefill"), "pod_fp8/prefill")
    assert_close(w, compare_role(w, w.decode, od, ld, tag="pod_fp8/decode"), "pod_fp8/decode")
    del w
    torch.cuda.empty_cache()
