"""Pins for the fp64 oracle: closed forms, invariants, library special cases and
the worked examples the pages print. None of these re-derives the oracle's own
formula; each would fail under a plausible slip in it (a dropped sink or
denominator, a flipped mask, a wrong GQA or page index, a natural-log LSE).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import attend_role, attend_rows, merge_states, apply_sink, valid_key_mask

LOG2E = 1.0 / math.log(2.0)


def paged_inputs(rng, kv_lens, qo_lens, page_size, hqo, hkv, d, shuffle=True, spare=2):
    """Tiny fp64 paged inputs: pool [P, ps, H_kv, D] with a random page order."""
    pages = [-(-k // page_size) for k in kv_lens]
    lpl = [(k - 1) % page_size + 1 for k in kv_lens]
    kv_indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int64)
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int64)
    total = int(kv_indptr[-1]) + spare
    perm = rng.permutation(total) if shuffle else np.arange(total)
    kv_indices = perm[: int(kv_indptr[-1])]
    kp = rng.standard_normal((total, page_size, hkv, d))
    vp = rng.standard_normal((total, page_size, hkv, d))
    q = rng.standard_normal((int(qo_indptr[-1]), hqo, d))
    return dict(q=q, k_pool=kp, v_pool=vp, qo_indptr=qo_indptr, kv_indptr=kv_indptr,
                kv_indices=kv_indices, last_page_len=np.array(lpl), page_size=page_size,
                num_qo_heads=hqo, num_kv_heads=hkv)


def run(inp, **kw):
    args = dict(inp)
    args.update(kw)
    return oracle.attend_role_dense(**args)


# ---------------------------------------------------------------- worked examples


def test_seq_lens_docstring_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "pod_docstring_example.json")))
    got = oracle.seq_lens(g["kv_indptr"], g["last_page_len"], g["page_size"])
    assert got.tolist() == g["kv_len_hand_derived"]


def test_batch_pod_example_shapes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "batch_pod_example.json")))
    # down-scaled lengths, the example's head layout and page_size 1; shapes must follow
    rng = np.random.default_rng(0)
    inp = paged_inputs(rng, [40, 40], [40, 40], 1, g["num_qo_heads"] // 8, g["num_kv_heads"] // 8, 8)
    o, lse = run(inp, causal=True)
    assert o.shape == (80, g["num_qo_heads"] // 8, 8) and lse.shape == (80, g["num_qo_heads"] // 8)
    assert g["printed_out_p_shape"] == [sum(g["p_qo_lens"]), g["num_qo_heads"], g["head_dim"]]
    assert g["printed_out_d_shape"] == [g["d_qo_lens_repeat"][1], g["num_qo_heads"], g["head_dim"]]
    lpl = [(k - 1) % g["page_size"] + 1 for k in g["p_kv_lens"]]
    assert lpl == [1, 1]


def test_single_decode_example_shapes(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "single_decode_example.json")))
    rng = np.random.default_rng(1)
    hq, d = g["q_shape"]
    kv, hk, _ = g["kv_shape"]
    q = rng.standard_normal((1, hq, d))
    k = rng.standard_normal((64, hk, d))
    v = rng.standard_normal((64, hk, d))
    o, lse = attend_rows(q, k, v, np.ones((1, 64), bool), 1 / math.sqrt(d))
    assert o[0].shape == tuple(g["output_shape"]) and lse[0].shape == tuple(g["lse_shape"])


# ---------------------------------------------------------------- library special cases


@pytest.mark.parametrize("hqo,hkv", [(4, 4), (8, 2), (6, 3)])
def test_dense_causal_matches_torch_sdpa(hqo, hkv):
    """qo_len == kv_len causal (configs with prefill = prefix) equals torch SDPA is_causal
    with enable_gqa (kv head h // g), in float64 on the CPU."""
    rng = np.random.default_rng(10 + hqo)
    L, d, scale = 37, 16, 0.31
    inp = paged_inputs(rng, [L], [L], 4, hqo, hkv, d)
    o, lse = run(inp, causal=True, sm_scale=scale)
    k, v = oracle.logical_kv(inp["k_pool"], inp["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                             inp["last_page_len"], 4, 0)
    qt = torch.from_numpy(inp["q"]).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale, enable_gqa=True)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_lse_matches_scipy_logsumexp():
    rng = np.random.default_rng(3)
    inp = paged_inputs(rng, [23], [5], 3, 2, 1, 8)
    o, lse = run(inp, causal=True, sm_scale=0.7)
    k, _ = oracle.logical_kv(inp["k_pool"], inp["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                             inp["last_page_len"], 3, 0)
    for i in range(5):
        nkeys = 23 - 5 + i + 1
        for h in range(2):
            s = 0.7 * np.einsum("d,kd->k", inp["q"][i, h], k[:nkeys, 0])
            assert abs(lse[i, h] - scipy.special.logsumexp(s) / math.log(2)) < 1e-12


def test_sink_is_extra_logit_with_zero_value_row():
    """Sink semantics via scipy's softmax over [scores, sink] with a zero value row."""
    rng = np.random.default_rng(4)
    inp = paged_inputs(rng, [19], [3], 4, 4, 2, 8)
    sinks = rng.standard_normal(4) * 2
    o, lse = run(inp, causal=True, sm_scale=0.5, sinks=sinks)
    o0, lse0 = run(inp, causal=True, sm_scale=0.5)
    k, v = oracle.logical_kv(inp["k_pool"], inp["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                             inp["last_page_len"], 4, 0)
    for i in range(3):
        n = 19 - 3 + i + 1
        for h in range(4):
            s = 0.5 * (k[:n, h // 2] @ inp["q"][i, h])
            p = scipy.special.softmax(np.concatenate([s, [sinks[h]]]))
            vv = np.concatenate([v[:n, h // 2], np.zeros((1, 8))])
            np.testing.assert_allclose(o[i, h], p @ vv, atol=1e-12)
    np.testing.assert_array_equal(lse, lse0)   # the returned lse excludes the sink


# ---------------------------------------------------------------- closed forms


def test_values_all_one_give_one():
    rng = np.random.default_rng(5)
    inp = paged_inputs(rng, [30, 9], [30, 4], 4, 4, 2, 8)
    inp["v_pool"] = np.ones_like(inp["v_pool"])
    for causal, w in [(True, -1), (True, 3), (False, -1), (False, 5)]:
        o, _ = run(inp, causal=causal, window_left=w)
        np.testing.assert_allclose(o, 1.0, atol=1e-13)


def test_zero_query_gives_mean_and_log2_count():
    rng = np.random.default_rng(6)
    inp = paged_inputs(rng, [17], [4], 5, 2, 2, 8)
    inp["q"] = np.zeros_like(inp["q"])
    o, lse = run(inp, causal=True, window_left=6)
    k, v = oracle.logical_kv(inp["k_pool"], inp["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                             inp["last_page_len"], 5, 0)
    for i in range(4):
        p = 17 - 4 + i
        J = list(range(max(0, p - 6), p + 1))
        np.testing.assert_allclose(lse[i], math.log2(len(J)), atol=1e-13)
        np.testing.assert_allclose(o[i], v[J].mean(axis=0), atol=1e-13)


def test_identical_keys_give_mean_values():
    rng = np.random.default_rng(7)
    inp = paged_inputs(rng, [12], [2], 4, 2, 1, 8)
    inp["k_pool"][:] = rng.standard_normal((1, 1, 1, 8))
    o, lse = run(inp, causal=True, sm_scale=0.9)
    k, v = oracle.logical_kv(inp["k_pool"], inp["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                             inp["last_page_len"], 4, 0)
    for i in range(2):
        n = 12 - 2 + i + 1
        for h in range(2):
            s = 0.9 * float(inp["q"][i, h] @ k[0, 0])
            np.testing.assert_allclose(lse[i, h], math.log2(n) + s * LOG2E, atol=1e-12)
            np.testing.assert_allclose(o[i, h], v[:n, 0].mean(axis=0), atol=1e-12)


def test_single_key_gives_its_value():
    rng = np.random.default_rng(8)
    inp = paged_inputs(rng, [1], [1], 16, 4, 4, 8)
    o, lse = run(inp, causal=True, sm_scale=0.25)
    page = inp["kv_indices"][0]
    np.testing.assert_allclose(o[0], inp["v_pool"][page, 0], atol=1e-14)
    s = 0.25 * np.einsum("hd,hd->h", inp["q"][0], inp["k_pool"][page, 0])
    np.testing.assert_allclose(lse[0], s * LOG2E, atol=1e-13)


def test_window_zero_keeps_only_the_diagonal():
    rng = np.random.default_rng(9)
    inp = paged_inputs(rng, [21], [6], 4, 2, 2, 8)
    o, lse = run(inp, causal=True, window_left=0, sm_scale=0.4)
    k, v = oracle.logical_kv(inp["k_pool"], inp["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                             inp["last_page_len"], 4, 0)
    for i in range(6):
        p = 21 - 6 + i
        np.testing.assert_allclose(o[i], v[p], atol=1e-14)
        np.testing.assert_allclose(lse[i], 0.4 * np.einsum("hd,hd->h", inp["q"][i], k[p]) * LOG2E,
                                   atol=1e-13)


def test_wide_window_equals_no_window():
    rng = np.random.default_rng(11)
    inp = paged_inputs(rng, [21, 8], [6, 8], 4, 2, 1, 8)
    a = run(inp, causal=True, window_left=21)
    b = run(inp, causal=True, window_left=-1)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_single_row_causal_equals_non_causal():
    rng = np.random.default_rng(12)
    inp = paged_inputs(rng, [33, 7, 1], [1, 1, 1], 4, 4, 2, 8)
    a = run(inp, causal=True)
    b = run(inp, causal=False)
    np.testing.assert_array_equal(a[0], b[0])


def test_bottom_right_alignment_first_and_last_rows():
    """Row 0 of a q_len < kv_len request sees exactly the first kv_len - q_len + 1
    keys; its last row sees every key."""
    rng = np.random.default_rng(13)
    kv, ql = 29, 5
    inp = paged_inputs(rng, [kv], [ql], 4, 2, 1, 8)
    o, lse = run(inp, causal=True)
    k, v = oracle.logical_kv(inp["k_pool"], inp["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                             inp["last_page_len"], 4, 0)
    n0 = kv - ql + 1
    o_first, l_first = attend_rows(inp["q"][:1], k[:n0], v[:n0], np.ones((1, n0), bool),
                                   1 / math.sqrt(8))
    o_last, l_last = attend_rows(inp["q"][ql - 1:], k, v, np.ones((1, kv), bool), 1 / math.sqrt(8))
    np.testing.assert_allclose(o[0], o_first[0], atol=1e-13)
    np.testing.assert_allclose(lse[0], l_first[0], atol=1e-13)
    np.testing.assert_allclose(o[-1], o_last[0], atol=1e-13)


def test_mask_matches_enumerated_rule():
    """The visible set equals an enumeration of the stated rule: row i sees keys
    0 .. kv_len - q_len + i, and a window keeps window_left keys before the
    diagonal plus the diagonal."""
    for kv in range(1, 12):
        for ql in range(1, kv + 1):
            for w in (-1, 0, 1, 3, 20):
                m = valid_key_mask(ql, kv, True, w)
                for i in range(ql):
                    diag = kv - ql + i
                    allowed = set(range(0, diag + 1))
                    if w >= 0:
                        allowed = {j for j in allowed if diag - j <= w}
                    assert set(np.nonzero(m[i])[0].tolist()) == allowed


def test_empty_valid_set_gives_zero_and_neg_inf():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((2, 2, 4))
    k = rng.standard_normal((5, 1, 4))
    keep = np.zeros((2, 5), bool)
    o, lse = attend_rows(q, k, k, keep, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- sinks


def test_sink_minus_infinity_is_no_sink():
    rng = np.random.default_rng(15)
    inp = paged_inputs(rng, [14], [3], 4, 4, 2, 8)
    a = run(inp, causal=True, sinks=np.full(4, -1e30))
    b = run(inp, causal=True)
    np.testing.assert_allclose(a[0], b[0], atol=1e-15)


def test_apply_sink_to_sink_free_state():
    rng = np.random.default_rng(16)
    inp = paged_inputs(rng, [14, 40], [3, 4], 4, 4, 2, 8)
    sinks = rng.standard_normal(4)
    a = run(inp, causal=True, window_left=7, sinks=sinks)
    b = run(inp, causal=True, window_left=7)
    np.testing.assert_allclose(a[0], apply_sink(b[0], b[1], sinks[None, :]), atol=1e-13)


# ---------------------------------------------------------------- invariants


def test_merge_of_key_halves_equals_full():
    rng = np.random.default_rng(17)
    n, kv, d = 4, 31, 8
    q = rng.standard_normal((n, 2, d))
    k = rng.standard_normal((kv, 1, d))
    v = rng.standard_normal((kv, 1, d))
    keep = valid_key_mask(n, kv, True, 9)
    full = attend_rows(q, k, v, keep, 0.6)
    for cut in (5, 16, 29):
        lo = keep.copy(); lo[:, cut:] = False
        hi = keep.copy(); hi[:, :cut] = False
        a = attend_rows(q, k, v, lo, 0.6)
        b = attend_rows(q, k, v, hi, 0.6)
        o, lse = merge_states([a, b])
        np.testing.assert_allclose(o, full[0], atol=1e-13)
        np.testing.assert_allclose(lse, full[1], atol=1e-13)
    # three-way split with one empty part
    parts = []
    for lo_, hi_ in ((0, 10), (10, 10), (10, kv)):
        m = keep.copy(); m[:, :lo_] = False; m[:, hi_:] = False
        parts.append(attend_rows(q, k, v, m, 0.6))
    o, lse = merge_states(parts)
    np.testing.assert_allclose(o, full[0], atol=1e-13)


def test_page_permutation_invariance():
    rng = np.random.default_rng(18)
    inp = paged_inputs(rng, [45, 3, 16], [45, 3, 2], 4, 4, 2, 8, shuffle=False, spare=3)
    a = run(inp, causal=True)
    perm = rng.permutation(inp["k_pool"].shape[0])
    inv = np.argsort(perm)
    inp2 = dict(inp)
    inp2["k_pool"] = inp["k_pool"][perm]
    inp2["v_pool"] = inp["v_pool"][perm]
    inp2["kv_indices"] = inv[inp["kv_indices"]]
    b = run(inp2, causal=True)
    np.testing.assert_array_equal(a[0], b[0])


def test_paged_equals_contiguous():
    """The same logical keys laid out with page_size 5 (shuffled) and page_size 1."""
    rng = np.random.default_rng(19)
    inp = paged_inputs(rng, [23, 11], [4, 11], 5, 4, 2, 8)
    a = run(inp, causal=True, window_left=6)
    ks, vs = [], []
    for b in range(2):
        k, v = oracle.logical_kv(inp["k_pool"], inp["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                                 inp["last_page_len"], 5, b)
        ks.append(k); vs.append(v)
    kc = np.concatenate(ks)[:, None]
    vc = np.concatenate(vs)[:, None]
    dense = dict(inp, k_pool=kc, v_pool=vc, page_size=1, kv_indices=None,
                 kv_indptr=np.array([0, 23, 34]), last_page_len=np.array([1, 1]))
    b_ = run(dense, causal=True, window_left=6)
    np.testing.assert_array_equal(a[0], b_[0])


def test_unreferenced_slots_are_never_read():
    rng = np.random.default_rng(20)
    inp = paged_inputs(rng, [13, 6], [2, 6], 4, 2, 1, 8, spare=3)
    a = run(inp, causal=True)
    poisoned = dict(inp)
    kp = inp["k_pool"].copy(); vp = inp["v_pool"].copy()
    used = np.zeros(kp.shape[0], bool); used[inp["kv_indices"]] = True
    kp[~used] = np.nan; vp[~used] = np.nan
    for b in range(2):
        last = inp["kv_indices"][inp["kv_indptr"][b + 1] - 1]
        l = inp["last_page_len"][b]
        kp[last, l:] = np.nan; vp[last, l:] = np.nan
    poisoned["k_pool"], poisoned["v_pool"] = kp, vp
    b = run(poisoned, causal=True)
    assert np.all(np.isfinite(b[0]))
    np.testing.assert_array_equal(a[0], b[0])


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(21)
    inp = paged_inputs(rng, [15], [4], 4, 8, 2, 8)
    a = run(inp, causal=True)
    mha = dict(inp, k_pool=np.repeat(inp["k_pool"], 4, axis=2),
               v_pool=np.repeat(inp["v_pool"], 4, axis=2), num_kv_heads=8)
    b = run(mha, causal=True)
    np.testing.assert_array_equal(a[0], b[0])


def test_validation_rejects_bad_page_tables():
    rng = np.random.default_rng(22)
    inp = paged_inputs(rng, [10], [4], 4, 4, 2, 8)
    with pytest.raises(oracle.OracleInputError):
        run(dict(inp, num_kv_heads=3), causal=True)
    with pytest.raises(oracle.OracleInputError):
        run(dict(inp, last_page_len=np.array([5])), causal=True)
    with pytest.raises(oracle.OracleInputError):
        run(dict(inp, last_page_len=np.array([0])), causal=True)
    with pytest.raises(oracle.OracleInputError):
        run(dict(inp, qo_indptr=np.array([0, 11])), causal=True)   # q_len > kv_len


def test_e4m3_decoding_matches_torch_float8_e4m3fn():
    # every one of the 256 codes against torch's own float8_e4m3fn -> float32
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_float(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.isnan(ours).sum() == 2                      # 0x7F and 0xFF only


def test_e4m3_closed_form_values():
    v = oracle.e4m3_to_float(np.array([0x38, 0x7E, 0x01, 0x08, 0xB8, 0x00, 0x80, 0x3C], np.uint8))
    assert v[0] == 1.0                                    # exponent field 7, mantissa 0
    assert v[1] == 448.0                                  # largest finite: 1.75 * 2^8
    assert v[2] == 2.0 ** -9                              # smallest subnormal: 1/8 * 2^-6
    assert v[3] == 2.0 ** -6                              # smallest normal
    assert v[4] == -1.0
    assert v[5] == 0.0 and v[6] == 0.0 and np.signbit(v[6])
    assert v[7] == 1.5


def test_fp8_scales_fold_into_scale_and_output():
    # q_scale * k_scale act as a factor on the scores, v_scale on the output:
    # the same as scaling K and V themselves
    rng = np.random.default_rng(8)
    q = rng.standard_normal((3, 4, 128))
    k = rng.standard_normal((50, 2, 128))
    v = rng.standard_normal((50, 2, 128))
    keep = oracle.valid_key_mask(3, 50, True, -1)
    o1, l1 = oracle.attend_rows_fp8_scaled(q, k, v, keep, 0.09, 0.5, 3.0, 1.75)
    o2, l2 = attend_rows(q, k * 1.5, v * 1.75, keep, 0.09)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    o3, l3 = oracle.attend_rows_fp8_scaled(q, k, v, keep, 0.09, 1.0, 1.0, 1.0)
    o4, l4 = attend_rows(q, k, v, keep, 0.09)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


# ---------------------------------------------------------------- layouts, non-causal rows, brute force


def _direct_kv(pool, kv_indptr, kv_indices, kv_len, page_size, b, layout="NHD"):
    """Keys of request b read straight from the pool with the page-table rule
    (logical key j = physical page kv_indices[kv_indptr[b] + j // page_size],
    slot j % page_size), one key at a time: [kv_len, H_kv, D]."""
    rows = []
    for j in range(kv_len):
        page = int(kv_indices[int(kv_indptr[b]) + j // page_size])
        slot = j % page_size
        rows.append(pool[page, slot] if layout == "NHD" else pool[page, :, slot])
    return np.stack(rows).astype(np.float64)


@pytest.mark.parametrize("ps,hkv", [(3, 2), (2, 2), (5, 1)])
def test_hnd_layout_equals_nhd(ps, hkv):
    """The same pool stored head-major ([P, H_kv, page_size, D]) gives the
    identical result; page_size == H_kv is included, where an index mix-up of
    the two axes keeps the shapes."""
    rng = np.random.default_rng(30 + ps)
    inp = paged_inputs(rng, [17, 6], [4, 6], ps, 2 * hkv, hkv, 8)
    a = run(inp, causal=True, window_left=5)
    hnd = dict(inp, k_pool=np.ascontiguousarray(inp["k_pool"].transpose(0, 2, 1, 3)),
               v_pool=np.ascontiguousarray(inp["v_pool"].transpose(0, 2, 1, 3)), layout="HND")
    b = run(hnd, causal=True, window_left=5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    # and the head-major keys themselves, read key by key from the pool
    kv_len = int(oracle.seq_lens(inp["kv_indptr"], inp["last_page_len"], ps)[0])
    k, _ = oracle.logical_kv(hnd["k_pool"], hnd["v_pool"], inp["kv_indptr"], inp["kv_indices"],
                             inp["last_page_len"], ps, 0, layout="HND")
    np.testing.assert_array_equal(k, _direct_kv(hnd["k_pool"], inp["kv_indptr"], inp["kv_indices"],
                                                kv_len, ps, 0, layout="HND"))


@pytest.mark.parametrize("hqo,hkv", [(4, 4), (6, 2)])
def test_non_causal_multi_row_matches_torch_sdpa(hqo, hkv):
    """Without the causal mask every row of a q_len < kv_len request sees every
    key: torch SDPA (fp64, no mask, enable_gqa) over keys read straight from the
    pool."""
    rng = np.random.default_rng(40 + hqo)
    kv, ql, d, scale = 29, 7, 16, 0.27
    inp = paged_inputs(rng, [kv], [ql], 4, hqo, hkv, d)
    o, lse = run(inp, causal=False, sm_scale=scale)
    k = _direct_kv(inp["k_pool"], inp["kv_indptr"], inp["kv_indices"], kv, 4, 0)
    v = _direct_kv(inp["v_pool"], inp["kv_indptr"], inp["kv_indices"], kv, 4, 0)
    qt = torch.from_numpy(inp["q"]).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=False, scale=scale, enable_gqa=True)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    # every row's lse is the log-sum-exp over all kv keys
    g = hqo // hkv
    for i in range(ql):
        for h in range(hqo):
            s = scale * (k[:, h // g] @ inp["q"][i, h])
            assert abs(lse[i, h] - scipy.special.logsumexp(s) / math.log(2)) < 1e-12


def test_window_without_causal_matches_enumeration():
    """Window without the causal mask: row i sees keys p_i - window_left ..
    kv_len - 1 (clipped at 0), p_i = kv_len - q_len + i."""
    for kv in range(1, 13):
        for ql in range(1, kv + 1):
            for w in (0, 1, 2, 5, 30):
                m = valid_key_mask(ql, kv, False, w)
                for i in range(ql):
                    diag = kv - ql + i
                    allowed = set(range(max(0, diag - w), kv))
                    assert set(np.nonzero(m[i])[0].tolist()) == allowed
    # and the attention itself over those keys
    rng = np.random.default_rng(43)
    kv, ql, w = 19, 6, 4
    inp = paged_inputs(rng, [kv], [ql], 3, 2, 1, 8)
    o, lse = run(inp, causal=False, window_left=w, sm_scale=0.5)
    k = _direct_kv(inp["k_pool"], inp["kv_indptr"], inp["kv_indices"], kv, 3, 0)
    v = _direct_kv(inp["v_pool"], inp["kv_indptr"], inp["kv_indices"], kv, 3, 0)
    for i in range(ql):
        J = list(range(max(0, kv - ql + i - w), kv))
        for h in range(2):
            s = 0.5 * (k[J, 0] @ inp["q"][i, h])
            p = scipy.special.softmax(s)
            np.testing.assert_allclose(o[i, h], p @ v[J, 0], atol=1e-12)
            assert abs(lse[i, h] - scipy.special.logsumexp(s) / math.log(2)) < 1e-12


def _brute_force(inp, causal, window_left, sm_scale, sinks=None):
    """Scalar pure-Python evaluation of the definition: each key read from the
    pool by the page-table rule, every sum taken with math.fsum."""
    q, kp, vp = inp["q"], inp["k_pool"], inp["v_pool"]
    ps, hqo, hkv = inp["page_size"], inp["num_qo_heads"], inp["num_kv_heads"]
    g = hqo // hkv
    d = q.shape[-1]
    out = np.zeros_like(q)
    lse = np.zeros(q.shape[:2])
    nreq = len(inp["qo_indptr"]) - 1
    for b in range(nreq):
        npages = int(inp["kv_indptr"][b + 1] - inp["kv_indptr"][b])
        kv_len = (npages - 1) * ps + int(inp["last_page_len"][b])
        q0, q1 = int(inp["qo_indptr"][b]), int(inp["qo_indptr"][b + 1])
        ql = q1 - q0
        for i in range(ql):
            diag = kv_len - ql + i
            for h in range(hqo):
                kh = h // g
                keys = [j for j in range(kv_len)
                        if (not causal or j <= diag) and (window_left < 0 or j >= diag - window_left)]
                s = {}
                for j in keys:
                    page = int(inp["kv_indices"][int(inp["kv_indptr"][b]) + j // ps])
                    kvec = kp[page, j % ps, kh]
                    s[j] = sm_scale * math.fsum(float(q[q0 + i, h, t]) * float(kvec[t]) for t in range(d))
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                z = math.fsum(e.values())
                den = z + (math.exp(float(sinks[h]) - m) if sinks is not None else 0.0)
                for t in range(d):
                    num = math.fsum(e[j] * float(vp[int(inp["kv_indices"][int(inp["kv_indptr"][b]) + j // ps]),
                                                    j % ps, kh, t]) for j in keys)
                    out[q0 + i, h, t] = num / den
                lse[q0 + i, h] = (m + math.log(z)) / math.log(2.0)
    return out, lse


@pytest.mark.parametrize("causal,w,with_sinks", [(True, -1, False), (True, 3, True), (False, -1, False),
                                                  (False, 2, True)])
def test_scalar_brute_force(causal, w, with_sinks):
    """The oracle equals a scalar evaluation that reads every key from the pool
    directly (no shared helper), to 1e-12: paging, GQA, mask, scale, sinks and
    the base-2 lse together."""
    rng = np.random.default_rng(50 + int(causal) + 2 * (w + 1))
    inp = paged_inputs(rng, [11, 5, 8], [3, 5, 1], 3, 4, 2, 6)
    sinks = rng.standard_normal(4) if with_sinks else None
    o, lse = run(inp, causal=causal, window_left=w, sm_scale=0.45, sinks=sinks)
    bo, bl = _brute_force(inp, causal, w, 0.45, sinks)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_dropping_pages_before_the_window_changes_nothing():
    """Keys outside every row's window weigh exactly zero: dropping the whole
    leading pages before the request's earliest visible key (and shortening
    kv_len by as much, which keeps each row's diagonal on the same key) gives
    the identical result. The GPU parity tests use this to bring long windowed
    requests to the host."""
    rng = np.random.default_rng(60)
    ps, kv, ql, w = 4, 57, 5, 9
    inp = paged_inputs(rng, [kv], [ql], ps, 4, 2, 8)
    for causal in (True, False):
        a = run(inp, causal=causal, window_left=w)
        lo = kv - ql - w                       # earliest visible key of row 0
        drop = lo // ps
        cut = dict(inp, kv_indices=inp["kv_indices"][drop:],
                   kv_indptr=np.array([0, int(inp["kv_indptr"][1]) - drop]))
        b = run(cut, causal=causal, window_left=w)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
