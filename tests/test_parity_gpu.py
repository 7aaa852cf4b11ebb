"""GPU parity: the fused HIP launch (through the C ABI) against the fp64 oracle.

Tolerances: max-abs error on O <= 5e-3 (fp16) / 2e-2 (bf16), on the base-2 LSE
<= 1e-3. Small ragged cases compare every element; the five named workloads
run at full size in the launch configuration the benchmark times and compare
sampled rows (every row for the decode roles)."""
import ctypes

import numpy as np
import pytest
import torch

from serving_attention_amd import BatchPOD, single_decode_with_kv_cache, _lib
from workloads import RoleSpec, WorkloadSpec, build, named_spec

from gpu_helpers import TOL_LSE, TOL_O, assert_close, compare_role, log, oracle_request, plan_and_run

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")


def small_spec(name="small", dtype="bf16", ps=16, hqo=16, hkv=4, w=-1, sinks=False, dq=1,
               p_q=(127, 33, 300), p_kv=(127, 60, 700), d_kv=(1, 16, 17, 100, 513, 1000, 2049),
               seed=0, pool="shared", layout="NHD", spare=3):
    return WorkloadSpec(
        name=name,
        prefill=RoleSpec(list(p_q), list(p_kv), causal=True, window_left=w) if p_q else None,
        decode=RoleSpec([dq] * len(d_kv), [max(k, dq) for k in d_kv], causal=True, window_left=w) if d_kv else None,
        num_qo_heads=hqo, num_kv_heads=hkv, page_size=ps, dtype=dtype, sinks=sinks, pool=pool,
        shuffle_pages=True, spare_pages=spare, kv_layout=layout, meta_seed=100 + seed,
        value_seed=200 + seed)


def check_all(w, res, tag):
    (op, lp), (od, ld) = res
    if w.prefill is not None:
        assert_close(w, compare_role(w, w.prefill, op, lp, tag=tag + "/prefill"), tag + "/prefill")
    if w.decode is not None:
        assert_close(w, compare_role(w, w.decode, od, ld, tag=tag + "/decode"), tag + "/decode")


def test_tiny_key_chunk():
    log("case: tiny key chunk (1 request, 1 token, 50 keys, f16)")
    w = build(small_spec(dtype="f16", p_q=(), d_kv=(50,), hqo=8, hkv=2), device="cuda")
    res, _ = plan_and_run(w, roles=("decode",))
    check_all(w, res, "tiny-chunk")


def test_tiny_query_tile():
    log("case: tiny query tile (1 request, 70 tokens, bf16)")
    w = build(small_spec(p_q=(70,), p_kv=(70,), d_kv=(), hqo=8, hkv=2), device="cuda")
    res, _ = plan_and_run(w, roles=("prefill",))
    check_all(w, res, "tiny-tile")


GRID = [
    dict(dtype="f16", ps=16, hqo=16, hkv=4),
    dict(dtype="bf16", ps=1, hqo=16, hkv=4),
    dict(dtype="bf16", ps=16, hqo=8, hkv=8),
    dict(dtype="bf16", ps=16, hqo=32, hkv=4, w=37),
    dict(dtype="f16", ps=5, hqo=16, hkv=2, sinks=True),
    dict(dtype="bf16", ps=16, hqo=16, hkv=2, w=100, sinks=True, dq=4),
    dict(dtype="bf16", ps=16, hqo=8, hkv=1, dq=3),
    dict(dtype="f16", ps=16, hqo=64, hkv=2, dq=1),       # group 32: a full MFMA column block
    dict(dtype="bf16", ps=16, hqo=64, hkv=1, dq=2),      # group 64: decode runs as query tiles
    dict(dtype="bf16", ps=16, hqo=12, hkv=4, w=0),       # group 3, diagonal-only window
    dict(dtype="bf16", ps=16, hqo=16, hkv=4, layout="HND"),
    # limits: the most sink heads the query tiles stage (1024 query heads, group 128)
    dict(dtype="bf16", ps=16, hqo=1024, hkv=8, sinks=True, dq=1, p_q=(40, 3), p_kv=(40, 300),
         d_kv=(1, 300, 1100)),
    dict(dtype="bf16", ps=64, hqo=16, hkv=4, w=200, sinks=True, dq=2),   # large power-of-two pages
    dict(dtype="f16", ps=48, hqo=16, hkv=4, dq=3),                       # large other pages
]


@pytest.mark.parametrize("idx", range(len(GRID)), ids=[str(i) for i in range(len(GRID))])
def test_small_grid(idx):
    cfg = GRID[idx]
    log(f"case: small grid {idx} {cfg}")
    w = build(small_spec(seed=idx, **cfg), device="cuda")
    res, _ = plan_and_run(w)
    check_all(w, res, f"grid{cfg}")


@pytest.mark.parametrize("chunk", [64, 128, 192, 256])
def test_split_kv_merge(chunk):
    log(f"case: split-KV merge, decode_chunk={chunk}")
    w = build(small_spec(dq=2, w=300, sinks=True, d_kv=(1, 63, 64, 65, 700, 2000)), device="cuda")
    res, pod = plan_and_run(w, decode_chunk=chunk)
    assert pod.plan_info()["n_groups"] > 0
    check_all(w, res, f"split{chunk}")


MANY = [
    dict(dtype="bf16", ps=16, w=-1, sinks=False, chunk=0, identity=False),
    dict(dtype="f16", ps=5, w=90, sinks=True, chunk=0, identity=True),
    dict(dtype="bf16", ps=16, w=-1, sinks=True, chunk=128, identity=False),
]


@pytest.mark.parametrize("idx", range(len(MANY)), ids=[str(i) for i in range(len(MANY))])
def test_many_chunks_per_workgroup(idx):
    """More key-chunk items than workgroups, so each workgroup runs a list of
    them back to back and issues a chunk's first loads in the previous one's
    tail. Ragged lengths leave waves without keys in some chunks; requests of
    one and of three rows (group 8: 8 and 24 rows) put chunks of both widths
    in one list; split groups and an identity page table (no kv_indices) are
    covered too."""
    cfg = MANY[idx]
    rng = np.random.default_rng(40 + idx)
    n = 640
    q_lens = rng.choice([1, 1, 1, 3], n).tolist()
    kv_lens = [int(max(k, q)) for k, q in zip(rng.integers(1, 700, n), q_lens)]
    spec = WorkloadSpec(
        name="many_chunks", prefill=None,
        decode=RoleSpec(q_lens, kv_lens, causal=True, window_left=cfg["w"]),
        num_qo_heads=16, num_kv_heads=2, page_size=cfg["ps"], dtype=cfg["dtype"], sinks=cfg["sinks"],
        pool="separate", shuffle_pages=not cfg["identity"], spare_pages=0, meta_seed=300 + idx,
        value_seed=400 + idx)
    log(f"case: many chunks per workgroup {idx} {cfg}")
    w = build(spec, device="cuda")
    if cfg["identity"]:
        assert np.array_equal(w.decode.kv_indices, np.arange(len(w.decode.kv_indices)))
    res, pod = plan_and_run(w, roles=("decode",), decode_chunk=cfg["chunk"],
                            identity_pages_d=cfg["identity"])
    info = pod.plan_info()
    log(f"plan: {info}")
    assert info["n_items"] > 2 * info["grid"]
    if cfg["chunk"]:
        assert info["n_groups"] > 0
    check_all(w, res, f"many{idx}")


TILES = [
    dict(dtype="bf16", ps=16, w=-1, sinks=True, hqo=16, hkv=8),
    dict(dtype="f16", ps=16, w=40, sinks=False, hqo=32, hkv=4),
    dict(dtype="bf16", ps=5, w=-1, sinks=True, hqo=16, hkv=8),
]


@pytest.mark.parametrize("idx", range(len(TILES)), ids=[str(i) for i in range(len(TILES))])
def test_many_query_tiles_per_workgroup(idx):
    """Hundreds of short prefill requests (chunks on prefixes, 1-150 rows) and a
    decode batch whose q_len x group exceeds 32 rows, so both roles run as query
    tiles: each workgroup streams several tiles per role with an item boundary
    every one to a few key blocks (normalise and store, reset, next query), and
    the loads of later blocks are in flight across those boundaries."""
    cfg = TILES[idx]
    rng = np.random.default_rng(70 + idx)
    n_p, n_d = 400, 60
    pq = rng.integers(1, 151, n_p).tolist()
    pkv = [int(q + x) for q, x in zip(pq, rng.integers(0, 200, n_p))]
    g = cfg["hqo"] // cfg["hkv"]
    dq = rng.integers(32 // g + 1, 32 // g + 9, n_d).tolist()
    dkv = [int(q + x) for q, x in zip(dq, rng.integers(0, 400, n_d))]
    spec = WorkloadSpec(
        name="many_tiles", prefill=RoleSpec(pq, pkv, causal=True, window_left=cfg["w"]),
        decode=RoleSpec(dq, dkv, causal=True, window_left=cfg["w"]),
        num_qo_heads=cfg["hqo"], num_kv_heads=cfg["hkv"], page_size=cfg["ps"], dtype=cfg["dtype"],
        sinks=cfg["sinks"], pool="shared", shuffle_pages=True, spare_pages=2, meta_seed=500 + idx,
        value_seed=600 + idx)
    log(f"case: many query tiles per workgroup {idx} {cfg}")
    w = build(spec, device="cuda")
    res, pod = plan_and_run(w)
    info = pod.plan_info()
    log(f"plan: {info}")
    assert info["n_prefill_items"] > 2 * info["grid"]
    check_all(w, res, f"tiles{idx}")


def test_repeat_runs_are_bitwise_stable_and_counters_reset():
    log("case: repeated runs with split-KV")
    w = build(small_spec(dq=2, sinks=True), device="cuda")
    res1, pod = plan_and_run(w, decode_chunk=64)
    first = [t.clone() for pair in res1 for t in pair]
    for _ in range(3):
        res, _ = plan_and_run(w, decode_chunk=64, pod=pod)
        again = [t for pair in res for t in pair]
        for a, b in zip(first, again):
            assert torch.equal(a, b)
    info = pod.plan_info()
    h = pod._int_ws[:16].cpu().numpy()
    counters = pod._int_ws[int(h[8]):int(h[8]) + info["n_groups"]].cpu().numpy()
    assert np.all(counters == 0)


def test_fused_equals_role_isolated():
    log("case: fused vs role-isolated launches")
    w = build(small_spec(dq=4, w=200, sinks=True), device="cuda")
    fused, _ = plan_and_run(w)
    pre, _ = plan_and_run(w, roles=("prefill",))
    dec, _ = plan_and_run(w, roles=("decode",))
    assert torch.equal(fused[0][0], pre[0][0]) and torch.equal(fused[0][1], pre[0][1])
    assert torch.equal(fused[1][0], dec[1][0]) and torch.equal(fused[1][1], dec[1][1])


def test_item_orders_agree():
    """Every order policy gives the same bits; group 16 puts decode requests of
    one token in key chunks and of three tokens in query tiles, so lists hold
    both roles' tiles and chunks."""
    log("case: item order policies")
    w = build(small_spec(dq=1, hqo=32, hkv=2, d_kv=(1, 16, 17, 100, 513, 1000, 2049)), device="cuda")
    base, _ = plan_and_run(w, order=0)
    for order in (1, 2, 3):
        res, _ = plan_and_run(w, order=order)
        for a, b in zip(base, res):
            assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_poisoned_unreferenced_slots_and_outputs():
    log("case: NaN in unreferenced pool slots and in the output buffers")
    spec = small_spec(dq=3, ps=16, pool="separate", spare=5, d_kv=(5, 17, 33, 300))
    w = build(spec, device="cuda", poison=True)
    res, _ = plan_and_run(w, poison_out=True, decode_chunk=64)
    check_all(w, res, "poison")


def test_empty_requests_and_single_key():
    log("case: zero-length query requests and single-key requests")
    w = build(small_spec(p_q=(0, 1, 5, 0), p_kv=(7, 1, 5, 3), d_kv=(1, 1, 2)), device="cuda")
    res, _ = plan_and_run(w)
    check_all(w, res, "empty")


def test_single_decode_api_matches_oracle():
    log("case: single_decode_with_kv_cache, README example shapes")
    g = torch.Generator(device="cuda").manual_seed(1001)
    q = torch.randn(32, 128, generator=g, device="cuda").half()
    k = torch.randn(2048, 32, 128, generator=g, device="cuda").half()
    v = torch.randn(2048, 32, 128, generator=g, device="cuda").half()
    import oracle
    ro, rl = oracle.attend_rows(q.float().cpu().numpy()[None], k.float().cpu().numpy(),
                                v.float().cpu().numpy(), np.ones((1, 2048), bool), 128 ** -0.5)
    for layout in ("NHD", "HND"):
        kk = k if layout == "NHD" else k.transpose(0, 1).contiguous()
        vv = v if layout == "NHD" else v.transpose(0, 1).contiguous()
        o, lse = single_decode_with_kv_cache(q, kk, vv, kv_layout=layout, return_lse=True)
        torch.cuda.synchronize()
        eo = float(np.abs(o.float().cpu().numpy() - ro[0]).max())
        el = float(np.abs(lse.cpu().numpy() - rl[0]).max())
        log(f"single_decode {layout}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL_O["f16"] and el <= TOL_LSE


@pytest.mark.parametrize("hq,hk,kv_len", [(64, 8, 32768), (32, 32, 32768), (8, 8, 65536), (8, 1, 262144)])
def test_single_decode_long_context(hq, hk, kv_len):
    """Long single-request decodes through single_decode_with_kv_cache: the
    split-KV partial states of these plans need more than 16 MiB of float
    workspace, which the call sizes from the plan itself."""
    log(f"case: single decode {hq}/{hk} heads, {kv_len} keys (bf16)")
    fbytes, _ = BatchPOD.workspace_bytes(None, None, None, [0, 1], [0, kv_len], [1], num_qo_heads=hq,
                                         num_kv_heads=hk, head_dim=128, page_size=1, causal_d=False,
                                         num_cus=torch.cuda.get_device_properties(0).multi_processor_count)
    log(f"float workspace needed: {fbytes} bytes")
    g = torch.Generator(device="cuda").manual_seed(kv_len + hq)
    q = torch.randn(hq, 128, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(kv_len, hk, 128, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(kv_len, hk, 128, generator=g, device="cuda").to(torch.bfloat16)
    o, lse = single_decode_with_kv_cache(q, k, v, return_lse=True)
    torch.cuda.synchronize()
    import oracle
    ro, rl = oracle.attend_rows(q.float().cpu().numpy()[None], k.float().cpu().numpy(),
                                v.float().cpu().numpy(), np.ones((1, kv_len), bool), 128 ** -0.5)
    eo = float(np.abs(o.float().cpu().numpy() - ro[0]).max())
    el = float(np.abs(lse.cpu().numpy() - rl[0]).max())
    log(f"single_decode long: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE


def test_run_errors():
    log("case: run-time error paths")
    w = build(small_spec(p_q=(10,), p_kv=(10,), d_kv=(20,), hqo=8, hkv=2), device="cuda")
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    pod = BatchPOD(ws)
    with pytest.raises(_lib.PodError):
        pod.run(w.prefill.q, w.prefill.kv_cache, w.prefill.kv_indices_dev, None, None, None)
    res, pod = plan_and_run(w, pod=pod)
    with pytest.raises(_lib.PodError):
        pod.run(w.prefill.q.half(), w.prefill.kv_cache, w.prefill.kv_indices_dev,
                w.decode.q, w.decode.kv_cache, w.decode.kv_indices_dev)
    with pytest.raises(ValueError):
        pod.run(w.prefill.q, w.prefill.kv_cache, w.prefill.kv_indices_dev,
                w.decode.q, w.decode.kv_cache, w.decode.kv_indices_dev,
                sinks=torch.zeros(8, device="cuda"))
    with pytest.raises(ValueError):
        pod.run(w.prefill.q[:5], w.prefill.kv_cache, w.prefill.kv_indices_dev,
                w.decode.q, w.decode.kv_cache, w.decode.kv_indices_dev)
    # caller-supplied outputs are checked like q: rows, heads, dtype, dense head_dim,
    # and a contiguous fp32 LSE (the kernel writes lse[row * num_qo_heads + head])
    args = (w.prefill.q, w.prefill.kv_cache, w.prefill.kv_indices_dev,
            w.decode.q, w.decode.kv_cache, w.decode.kv_indices_dev)
    qp = w.prefill.q
    bad_outs = [
        dict(out_p=torch.empty(5, 8, 128, dtype=qp.dtype, device="cuda")),
        dict(out_p=torch.empty(10, 8, 128, dtype=torch.float16, device="cuda")),
        dict(out_p=torch.empty(10, 8, 256, dtype=qp.dtype, device="cuda")[:, :, ::2]),
        dict(out_d=torch.empty(1, 4, 128, dtype=qp.dtype, device="cuda")),
        dict(lse_p=torch.empty(10, 16, device="cuda")[:, :8], return_lse=True),
        dict(lse_p=torch.empty(10, 8, dtype=torch.float16, device="cuda"), return_lse=True),
        dict(lse_d=torch.empty(0, 8, device="cuda"), return_lse=True),
    ]
    for kw in bad_outs:
        with pytest.raises(ValueError):
            pod.run(*args, **kw)
    # the paged caches: on q's device, of the planned dtype and shape (combined
    # [P, 2, ...] cache or a (k, v) pair)
    kc = w.decode.kv_cache
    bad_caches = [kc.cpu(), kc.half(), kc[:, :, :8], (kc[:, 0], kc[:, 1, :, :1]), kc[:, :1]]
    for c in bad_caches:
        with pytest.raises((ValueError, _lib.PodError)):
            pod.run(w.prefill.q, w.prefill.kv_cache, w.prefill.kv_indices_dev,
                    w.decode.q, c, w.decode.kv_indices_dev)
    # the decode scales: finite, q_scale * k_scale > 0, effective scale <= 1e6
    for kw in (dict(q_scale_d=-1.0), dict(k_scale_d=float("nan")), dict(v_scale_d=float("inf")),
               dict(q_scale_d=1e4, k_scale_d=1e4)):
        with pytest.raises(ValueError):
            pod.run(*args, **kw)
    # workspace too small for a split plan: one request of 2000 keys in chunks of 64
    tiny = BatchPOD(torch.empty(4096, dtype=torch.uint8, device="cuda"))
    with pytest.raises(_lib.PodError):
        tiny.plan(None, None, None, [0, 1], [0, 125], [16], num_qo_heads=8, num_kv_heads=2,
                  head_dim=128, page_size=16, decode_chunk=64)


# ------------------------------------------------------------ named workloads, full size


def sample_rows(qo_len, rng, extra=24):
    base = {0, 1, 15, 16, 17, 31, 63, 64, 127, 128, qo_len // 2, qo_len - 17, qo_len - 16,
            qo_len - 2, qo_len - 1}
    base |= set(rng.integers(0, qo_len, extra).tolist())
    return np.array(sorted(r for r in base if 0 <= r < qo_len))


@pytest.mark.parametrize("name", ["single_decode", "batch_decode", "batch_prefill", "pod"])
def test_named_workload(name):
    log(f"case: named workload {name} (full size)")
    w = build(named_spec(name), device="cuda")
    res, pod = plan_and_run(w)
    log(f"plan: {pod.plan_info()}")
    (op, lp), (od, ld) = res
    rng = np.random.default_rng(7)
    if w.prefill is not None:
        errs = compare_role(w, w.prefill, op, lp,
                            rows_of=lambda b: sample_rows(int(w.prefill.qo_lens[b]), rng),
                            tag=name + "/prefill")
        assert_close(w, errs, name + "/prefill")
    if w.decode is not None:
        assert_close(w, compare_role(w, w.decode, od, ld, tag=name + "/decode"), name + "/decode")
    del w
    torch.cuda.empty_cache()


def test_named_pod_chunked():
    log("case: named workload pod_chunked (full size, 17.8 GB pool)")
    w = build(named_spec("pod_chunked"), device="cuda")
    res, pod = plan_and_run(w)
    log(f"plan: {pod.plan_info()}")
    (op, lp), (od, ld) = res
    rng = np.random.default_rng(5)
    errs = compare_role(w, w.prefill, op, lp, rows_of=lambda b: sample_rows(4096, rng, 150),
                        tag="pod_chunked/prefill")
    assert_close(w, errs, "pod_chunked/prefill")
    # every decode request (the oracle reads each one's window of keys)
    errs = compare_role(w, w.decode, od, ld, tag="pod_chunked/decode")
    assert_close(w, errs, "pod_chunked/decode")
    del w
    torch.cuda.empty_cache()


@pytest.mark.parametrize("w,dq,hqo", [(-1, 1, 16), (50, 3, 16), (0, 2, 16), (200, 5, 64)])
def test_non_causal_roles(w, dq, hqo):
    """Both roles without the causal mask: every row sees keys up to kv_len - 1,
    and a window bounds them on the left at (diagonal - window_left), the
    reading taken where the pages give the window only for causal rows. Prefill
    chunks sit on prefixes (qo_len < kv_len); with hqo 64 / 4 kv heads the
    multi-token decode rows (group 16 x q_len 5 > 32) run as query tiles."""
    log(f"case: non-causal roles (window_left={w}, q_len_d={dq}, hqo={hqo})")
    d_kv = (5, 40, 300, 1000)
    spec = WorkloadSpec(
        name="noncausal",
        prefill=RoleSpec([60, 130, 1], [60, 400, 90], causal=False, window_left=w),
        decode=RoleSpec([dq] * len(d_kv), [max(k, dq) for k in d_kv], causal=False, window_left=w),
        num_qo_heads=hqo, num_kv_heads=4, page_size=16, dtype="bf16", sinks=False, pool="shared",
        shuffle_pages=True, spare_pages=3, meta_seed=311, value_seed=411)
    wl = build(spec, device="cuda")
    res, _ = plan_and_run(wl)
    check_all(wl, res, f"noncausal-w{w}-q{dq}")


@pytest.mark.parametrize("w", [-1, 10])
def test_non_causal_more_queries_than_keys(w):
    """Non-causal requests may hold more query rows than keys: the diagonal
    kv_len - q_len + i is negative for the first rows, every row sees all keys
    (up to its window's left bound, which then lies before key 0)."""
    log(f"case: non-causal, q_len > kv_len (window_left={w})")
    spec = WorkloadSpec(
        name="noncausal_short_kv",
        prefill=RoleSpec([200, 70, 33], [50, 20, 1], causal=False, window_left=w),
        decode=RoleSpec([5, 5, 3], [3, 40, 1], causal=False, window_left=w),
        num_qo_heads=16, num_kv_heads=4, page_size=16, dtype="bf16", sinks=True, pool="shared",
        shuffle_pages=True, spare_pages=3, meta_seed=312, value_seed=412)
    wl = build(spec, device="cuda")
    res, _ = plan_and_run(wl)
    check_all(wl, res, f"noncausal-short-w{w}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_group_128(dtype):
    """The largest supported group (128 query heads per kv head): query tiles of
    two tokens, decode requests of one and two tokens (128 and 256 rows), with a
    window and sinks."""
    log(f"case: group 128 ({dtype})")
    spec = WorkloadSpec(
        name="group128", prefill=RoleSpec([40, 7, 130], [40, 300, 130], causal=True, window_left=90),
        decode=RoleSpec([1, 2, 1, 2], [1, 70, 600, 1500], causal=True, window_left=90),
        num_qo_heads=128, num_kv_heads=1, page_size=16, dtype=dtype, sinks=True, pool="shared",
        shuffle_pages=True, spare_pages=3, meta_seed=128, value_seed=228)
    w = build(spec, device="cuda")
    res, pod = plan_and_run(w)
    log(f"plan: {pod.plan_info()}")
    check_all(w, res, f"group128-{dtype}")


def test_first_plan_waits_for_work_queued_on_the_stream():
    """A new context planned right behind a few milliseconds of queued work on
    the caller's stream: the first image copy of each workspace half is
    ordered after that work (a caller may still be initialising or using that
    memory there), so the launch reads the plan. Outputs start as NaN, so a
    launch that found no work would show."""
    log("case: first plans behind queued work on the stream")
    w = build(small_spec(p_q=(70,), p_kv=(300,), d_kv=(1, 700, 2049), dq=2), device="cuda")
    ref = None
    busy = torch.empty(1 << 29, dtype=torch.float32, device="cuda")
    for trial in range(3):
        for _ in range(4):
            busy.fill_(float(trial))          # ~2 GB of writes queued ahead
        ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
        pod = BatchPOD(ws, "NHD", int_workspace_bytes=4 << 20)
        p, d = w.prefill, w.decode
        outs = [torch.full_like(r.q, float("nan")) for r in (p, d)]
        lses = [torch.full(r.q.shape[:2], float("nan"), device="cuda") for r in (p, d)]
        for rep in range(2):                  # both workspace halves
            pod.plan(p.qo_indptr, p.kv_indptr, p.last_page_len, d.qo_indptr, d.kv_indptr,
                     d.last_page_len, num_qo_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                     dtype=torch.bfloat16, decode_chunk=256)
            res = pod.run(p.q, p.kv_cache, p.kv_indices_dev, d.q, d.kv_cache, d.kv_indices_dev,
                          return_lse=True, out_p=outs[0], lse_p=lses[0], out_d=outs[1], lse_d=lses[1])
            torch.cuda.synchronize()
            if ref is None:
                check_all(w, res, "first-plan")
                ref = [t.clone() for t in outs + lses]
            for a, b in zip(ref, outs + lses):
                assert torch.equal(a, b), f"trial {trial} plan {rep}: outputs differ"
        del pod


def test_plan_and_run_on_other_streams():
    """Plans on one stream and runs on another, alternating plans made while
    the previous launch is still queued (the host then waits for the work-list
    copy) with plans made on an idle GPU (the launch then waits for the copy on
    the device): every run reads its own plan. Two workloads alternate, so a
    launch that read the other plan's list would not match."""
    log("case: plans and runs on different streams, GPU busy and idle")
    wls = [build(small_spec(p_q=(70,), p_kv=(300,), d_kv=(1, 700, 2049), dq=2), device="cuda"),
           build(small_spec(p_q=(33, 5), p_kv=(33, 400), d_kv=(900, 17), dq=1, seed=7), device="cuda")]
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    pod = BatchPOD(ws, "NHD", int_workspace_bytes=4 << 20)
    busy = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    s_plan, s_run = torch.cuda.Stream(), torch.cuda.Stream()
    kept = []
    for it in range(8):
        w = wls[it % 2]
        p, d = w.prefill, w.decode
        idle = it % 4 >= 2
        if idle:
            torch.cuda.synchronize()
        with torch.cuda.stream(s_plan):
            pod.plan(p.qo_indptr, p.kv_indptr, p.last_page_len, d.qo_indptr, d.kv_indptr,
                     d.last_page_len, num_qo_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                     dtype=torch.bfloat16, decode_chunk=256)
        outs = [torch.full_like(r.q, float("nan")) for r in (p, d)]
        lses = [torch.full(r.q.shape[:2], float("nan"), device="cuda") for r in (p, d)]
        s_run.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_run):
            if not idle:
                busy.fill_(float(it))         # the launch queues behind ~1 GB of writes
            res = pod.run(p.q, p.kv_cache, p.kv_indices_dev, d.q, d.kv_cache, d.kv_indices_dev,
                          return_lse=True, out_p=outs[0], lse_p=lses[0], out_d=outs[1], lse_d=lses[1])
        kept.append((it % 2, res, outs + lses))
    torch.cuda.synchronize()
    first = {}
    for it, (k, res, ts) in enumerate(kept):
        if k not in first:
            check_all(wls[k], res, f"streams-{k}")
            first[k] = ts
            continue
        for a, b in zip(first[k], ts):
            assert torch.equal(a, b), f"iteration {it}: outputs differ from the first run of this plan"


@pytest.mark.parametrize("ps", [16, 5])
def test_identity_pages_for_query_tiles(ps):
    """Roles run without a page table (identity pages: page i of a request's
    range is pool page i): the query tiles' own code for identity pages
    (power-of-two page sizes) and the code that decides it per launch (other
    page sizes), for the prefill role and for decode rows that run as query
    tiles (group 16 x q_len 3 = 48 rows)."""
    log(f"case: identity pages through query tiles (page_size={ps})")
    spec = WorkloadSpec(
        name="identity_tiles", prefill=RoleSpec([70, 1, 130], [200, 1, 130], causal=True, window_left=-1),
        decode=RoleSpec([3, 1, 3], [3, 90, 700], causal=True, window_left=40),
        num_qo_heads=32, num_kv_heads=2, page_size=ps, dtype="bf16", sinks=True, pool="separate",
        shuffle_pages=False, spare_pages=0, meta_seed=321, value_seed=421)
    w = build(spec, device="cuda")
    for r in (w.prefill, w.decode):
        assert np.array_equal(r.kv_indices, np.arange(len(r.kv_indices)))
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    pod = BatchPOD(ws, "NHD", int_workspace_bytes=4 << 20)
    p, d = w.prefill, w.decode
    pod.plan(p.qo_indptr, p.kv_indptr, p.last_page_len, d.qo_indptr, d.kv_indptr, d.last_page_len,
             num_qo_heads=32, num_kv_heads=2, head_dim=128, page_size=ps, dtype=torch.bfloat16,
             window_left_d=40, sinks=True)
    res = pod.run(p.q, p.kv_cache, None, d.q, d.kv_cache, None, sinks=w.sinks, return_lse=True)
    torch.cuda.synchronize()
    check_all(w, res, f"identity-tiles-ps{ps}")
