"""Host planner, driven through pod_plan_compute (no GPU): the work list covers
every (row, kv head, valid key) exactly once, split groups are consistent, the
per-workgroup lists partition the items and their block tables match the query
tiles, and bad inputs get their error code."""
import ctypes

import numpy as np
import pytest

from serving_attention_amd import _lib

from plan_helpers import compute, decode_image, plan_desc

FLAG_ROLE, FLAG_CHUNK = 1, 2


def check_coverage(img, roles, hqo, hkv):
    """roles: list of (qo_lens, kv_lens, causal, window_left) for prefill then decode.
    Coverage is counted per row (token t, group head j) = t * g + j of each
    (request, kv head): a query tile covers all g rows of its tokens, a key
    chunk the up to 32 rows from its first row (word 3) on."""
    g = hqo // hkv
    im = decode_image(img)
    reqs = im["reqs"]
    items = im["items"]
    # expected request table
    exp = []
    for qo_lens, kv_lens, _, _ in roles:
        qs = 0
        for q, k in zip(qo_lens, kv_lens):
            exp.append((qs, q, k))
            qs += q
    assert [tuple(r[:3]) for r in reqs] == exp
    cover = {}   # (req, kvh) -> count array [qo_len, kv_len]
    role_of_req = []
    for r, (qo_lens, kv_lens, causal, w) in enumerate(roles):
        for q, k in zip(qo_lens, kv_lens):
            role_of_req.append((r, causal, w))
    n_real = 0
    group_members = {}
    for s, it in enumerate(items):
        flags = int(it[0])
        if flags == -1:
            continue
        n_real += 1
        req, kvh, tok0, ntok, kb, ke, grp = [int(x) for x in it[1:]]
        role, causal, w = role_of_req[req]
        assert (flags & FLAG_ROLE) == role
        qo_len, kv_len = int(reqs[req][1]), int(reqs[req][2])
        c = cover.setdefault((req, kvh), np.zeros((qo_len * g, kv_len), np.int32))
        if flags & FLAG_CHUNK:
            # tok0 holds the first row of the item's slice
            assert ntok == qo_len and tok0 % 32 == 0 and 0 <= tok0 < qo_len * g
            rows = range(tok0, min(tok0 + 32, qo_len * g))
            if grp >= 0:
                group_members.setdefault(grp, []).append(flags >> 8)
                assert int(im["groups"][grp][2]) == req and int(im["groups"][grp][3]) == kvh
        else:
            assert ntok * g <= 256 and grp == -1
            rows = range(tok0 * g, (tok0 + ntok) * g)
        assert 0 <= kb < ke <= kv_len
        for r in rows:
            p = kv_len - qo_len + r // g
            lo = max(0, p - w) if w >= 0 else 0
            hi = p if causal else kv_len - 1
            # every valid key of the row inside the item's range is counted once
            c[r, max(kb, lo):min(ke, hi + 1)] += 1
    assert n_real == im["n_items"]
    for (req, kvh), c in cover.items():
        role, causal, w = role_of_req[req]
        kv_len = c.shape[1]
        qo_len = c.shape[0] // g
        for i in range(qo_len * g):
            p = kv_len - qo_len + i // g
            lo = max(0, p - w) if w >= 0 else 0
            hi = p if causal else kv_len - 1
            assert np.all(c[i, lo:hi + 1] == 1), (req, kvh, i)
    expected_units = sum(hkv for qo_lens, _, _, _ in roles for q in qo_lens if q > 0)
    assert len(cover) == expected_units
    # split groups: members 0..n-1, slots disjoint and in range
    slots = set()
    for gi, grp in enumerate(im["groups"]):
        n, first = int(grp[0]), int(grp[1])
        assert sorted(group_members[gi]) == list(range(n))
        for s in range(first, first + n):
            assert s not in slots
            slots.add(s)
    assert slots == set(range(im["n_slots"]))
    assert np.all(im["counters"] == 0)
    assert np.all(im["queue"] == 0)
    return im


@pytest.mark.parametrize("page_size", [1, 16])
def test_pod_example_coverage(page_size):
    roles = [([300, 200], [300, 200], True, -1), ([1] * 17, [700] * 17, True, -1)]
    desc, keep = plan_desc(prefill=dict(qo_lens=roles[0][0], kv_lens=roles[0][1]),
                           decode=dict(qo_lens=roles[1][0], kv_lens=roles[1][1]),
                           hqo=32, hkv=4, page_size=page_size)
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    im = check_coverage(img, roles, 32, 4)
    assert info.n_prefill_items + info.n_decode_items == info.n_items
    assert info.grid % 8 == 0


@pytest.mark.parametrize("w", [-1, 0, 5, 100])
@pytest.mark.parametrize("chunk", [0, 64, 128, -1])
def test_window_and_multi_token_decode_coverage(w, chunk):
    roles = [([64, 1, 0], [500, 77, 20], True, w), ([4, 4, 2, 1], [1053, 90, 4, 33], True, w)]
    desc, keep = plan_desc(prefill=dict(qo_lens=roles[0][0], kv_lens=roles[0][1], window_left=w),
                           decode=dict(qo_lens=roles[1][0], kv_lens=roles[1][1], window_left=w),
                           hqo=16, hkv=2, page_size=16, decode_chunk=chunk)
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    check_coverage(img, roles, 16, 2)


def test_non_causal_and_mha_coverage():
    roles = [([40, 7], [40, 100], False, -1), ([1, 1], [1, 65], False, 3)]
    desc, keep = plan_desc(prefill=dict(qo_lens=roles[0][0], kv_lens=roles[0][1], causal=False),
                           decode=dict(qo_lens=roles[1][0], kv_lens=roles[1][1], causal=False, window_left=3),
                           hqo=4, hkv=4, page_size=3)
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    check_coverage(img, roles, 4, 4)


def test_large_group_uses_tiles_for_decode():
    # group 64: a one-token decode has 64 rows, more than a key chunk holds
    roles = [([], [], True, -1), ([1, 2], [100, 300], True, -1)]
    desc, keep = plan_desc(decode=dict(qo_lens=roles[1][0], kv_lens=roles[1][1]), hqo=64, hkv=1)
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    im = check_coverage(img, roles, 64, 1)
    assert all((int(it[0]) & FLAG_CHUNK) == 0 for it in im["items"] if it[0] != -1)


def test_tiles_of_one_kv_unit_share_a_die():
    desc, keep = plan_desc(prefill=dict(qo_lens=[2048, 2048], kv_lens=[2048, 2048]), hqo=64, hkv=8,
                           page_size=1)
    rc, img, info = compute(desc)
    im = decode_image(img)
    die = {}
    for s, it in enumerate(im["items"]):
        key = (int(it[1]), int(it[2]))
        die.setdefault(key, set()).add(int(im["wg_of_item"][s]) % 8)
    assert all(len(v) == 1 for v in die.values())


def test_auto_split_gives_enough_items_for_single_decode():
    desc, keep = plan_desc(decode=dict(qo_lens=[1], kv_lens=[2048], causal=False), hqo=32, hkv=32,
                           page_size=1)
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    assert info.n_decode_items >= 256 and info.n_groups == 32
    check_coverage(img, [([], [], True, -1), ([1], [2048], False, -1)], 32, 32)


def test_orders_are_permutations_of_the_same_items():
    base = None
    for order in (0, 1, 2, 3):
        desc, keep = plan_desc(prefill=dict(qo_lens=[100, 50], kv_lens=[100, 60]),
                               decode=dict(qo_lens=[1] * 9, kv_lens=list(range(100, 1000, 100))),
                               hqo=8, hkv=2, order=order)
        rc, img, info = compute(desc)
        im = decode_image(img)
        items = sorted(tuple(int(x) for x in it[1:7]) for it in im["items"] if it[0] != -1)
        base = base or items
        assert items == base


def item_cost(it):
    # the planner's estimates (ns of one workgroup): tiles 1500 + 33 per key, chunks 2500 + 20 per key
    keys = int(it[6] - it[5])
    return 2500 + 20 * keys if int(it[0]) & FLAG_CHUNK else 1500 + 33 * keys


WORKLOADS = [
    dict(prefill=dict(qo_lens=[300, 50], kv_lens=[700, 60]),
         decode=dict(qo_lens=[1] * 9, kv_lens=list(range(100, 1000, 100))), hqo=8, hkv=2),
    dict(prefill=dict(qo_lens=[2048, 2048], kv_lens=[2048, 2048]),
         decode=dict(qo_lens=[1] * 128, kv_lens=[2048] * 128), hqo=64, hkv=8, page_size=1),
    dict(prefill=dict(qo_lens=[4096], kv_lens=[20480], window_left=4096),
         decode=dict(qo_lens=[4] * 64, kv_lens=[1024 + 500 * i for i in range(64)], window_left=4096),
         hqo=64, hkv=8),
    dict(decode=dict(qo_lens=[1, 2], kv_lens=[100, 300]), hqo=64, hkv=1),
    # group 16: one-token decodes are key chunks, three-token decodes (48 rows)
    # query tiles, some of them heavier than the prefill tiles
    dict(prefill=dict(qo_lens=[40, 90], kv_lens=[200, 90]),
         decode=dict(qo_lens=[1, 3, 1, 3, 2, 3] * 6, kv_lens=[300, 3000, 900, 500, 4000, 2500] * 6),
         hqo=32, hkv=2),
]


@pytest.mark.parametrize("order", [0, 1, 2, 3])
@pytest.mark.parametrize("wl", range(len(WORKLOADS)))
def test_workgroup_lists(wl, order):
    """Every item sits in exactly one workgroup list: query tiles first (prefill
    role, then decode role), then key chunks, each kind heaviest first; within a
    die the lists are balanced to within one item; the chunks-first flag follows
    the order policy."""
    desc, keep = plan_desc(order=order, **WORKLOADS[wl])
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    im = decode_image(img)
    items, wgs = im["items"], im["wgs"]
    # one workgroup per CU, or, when every die's items fit one workgroup each,
    # as many per die as the busiest die has items (workgroup w runs on die w % 8)
    assert len(wgs) == info.grid and info.grid % 8 == 0 and info.grid <= 256
    pf, pc = im["pool_first"], im["pool_count"]
    if info.grid < 256:
        per_wg = [int(wg[1]) + int(wg[2]) for wg in wgs]
        assert pc == 0 and max(per_wg) <= 1
        busy = [sum(per_wg[x::8]) for x in range(8)]
        assert info.grid == 8 * max(1, max(busy))
    assert pf + pc == im["n_items"]
    assert np.all(im["wg_of_item"][:pf] >= 0) and np.all(im["wg_of_item"][pf:] == -1)
    nxt = 0
    loads = np.zeros(len(wgs))
    for w, wg in enumerate(wgs):
        first, nt, nc, chunks_first, npt = (int(x) for x in (wg[0], wg[1], wg[2], wg[5], wg[6]))
        assert first == nxt
        nxt += nt + nc
        tiles, chunks = items[first:first + nt], items[first + nt:first + nt + nc]
        assert all(int(t[0]) & FLAG_CHUNK == 0 for t in tiles)
        assert all(int(c[0]) & FLAG_CHUNK for c in chunks)
        roles = [int(t[0]) & FLAG_ROLE for t in tiles]
        assert roles == sorted(roles) and roles.count(0) == npt
        for part in (tiles[:npt], tiles[npt:], chunks):
            c = [item_cost(it) for it in part]
            assert c == sorted(c, reverse=True)
        loads[w] = sum(item_cost(it) for it in items[first:first + nt + nc])
        if nt and nc:
            expect = {0: (w // 8) % 2 == 1, 1: False, 2: True,
                      3: item_cost(chunks[0]) > max(item_cost(t) for t in tiles)}[order]
            assert bool(chunks_first) == expect
        else:
            assert chunks_first == 0
    assert nxt == pf
    # the shared pool: key chunks only, heaviest first, at most a tenth of
    # the chunks' estimated cost, and none heavier than a chunk left in a list
    pool = items[pf:]
    assert all(int(c[0]) & FLAG_CHUNK for c in pool)
    pc_cost = [item_cost(c) for c in pool]
    assert pc_cost == sorted(pc_cost, reverse=True)
    chunk_costs = [item_cost(c) for c in items if int(c[0]) & FLAG_CHUNK]
    assert sum(pc_cost) <= 0.10 * sum(chunk_costs) + 1
    listed = [item_cost(c) for c in items[:pf] if int(c[0]) & FLAG_CHUNK]
    if pool.size and listed:
        assert max(pc_cost) <= min(listed)
    biggest = max(item_cost(it) for it in items)
    for x in range(8):
        die = loads[x::8]
        assert die.max() - die.min() <= biggest


@pytest.mark.parametrize("wl", range(len(WORKLOADS)))
def test_block_tables(wl):
    """Each workgroup's block table walks its query tiles in list order, 64 keys
    per block, with the first-block flag, role, kv head and tile index in meta."""
    desc, keep = plan_desc(**WORKLOADS[wl])
    rc, img, info = compute(desc)
    im = decode_image(img)
    items, reqs, blocks = im["items"], im["reqs"], im["blocks"]
    total = 0
    for w, wg in enumerate(im["wgs"]):
        first, nt, fb, nb, npb = int(wg[0]), int(wg[1]), int(wg[3]), int(wg[4]), int(wg[7])
        assert fb == total
        exp = []
        n_pre_blocks = 0
        for j in range(nt):
            it = items[first + j]
            role, kvh, lo, hi = int(it[0]) & FLAG_ROLE, int(it[2]), int(it[5]), int(it[6])
            ps = int(reqs[int(it[1])][3])
            for kb in range(lo, hi, 64):
                meta = (1 << 31 if kb == lo else 0) | (role << 30) | (kvh << 16) | j
                exp.append((kb, hi - 1, ps, meta))
                n_pre_blocks += role == 0
        got = [(int(e[0]), int(e[1]), int(e[2]), int(e[3]) & 0xffffffff) for e in blocks[fb:fb + nb]]
        assert got == exp
        assert npb == n_pre_blocks
        total += nb
    assert total == len(blocks)
    # each query tile's boundary row: first query row, tokens, kv head, diagonal
    # key of its first token, key end, kv_len; a key chunk's row: its request's
    # qo_start, qo_len, kv_len, page_start
    for it, td in zip(items, im["tdesc"]):
        if int(it[0]) & FLAG_CHUNK:
            assert [int(x) for x in td] == [int(x) for x in reqs[int(it[1])]] + [0, 0, 0, 0]
            continue
        qs, ql, kl = (int(x) for x in reqs[int(it[1])][:3])
        assert [int(x) for x in td] == [qs + int(it[3]), int(it[4]), int(it[2]),
                                        kl - ql + int(it[3]), int(it[6]), kl, 0, 0]


@pytest.mark.parametrize("batch", [1, 3, 20, 40])
def test_small_plans_get_one_workgroup_per_item(batch):
    """A plan with fewer items than CUs launches one workgroup per item, rounded
    up to whole dies, and no shared pool; the workspace query reserves the image
    of the full grid, which is larger."""
    desc, keep = plan_desc(decode=dict(qo_lens=[1] * batch, kv_lens=[300] * batch), hqo=16, hkv=2,
                           decode_chunk=-1)
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    n = 2 * batch   # equal items: the dies take turns
    assert info.n_items == n and info.grid == max(8, -(-n // 8) * 8)
    im = decode_image(img)
    assert im["pool_count"] == 0
    assert sorted(int(wg[1]) + int(wg[2]) for wg in im["wgs"]) == [0] * (info.grid - n) + [1] * n
    check_coverage(img, [([], [], True, -1), ([1] * batch, [300] * batch, True, -1)], 16, 2)
    fb, ib = ctypes.c_size_t(), ctypes.c_size_t()
    assert _lib.load().pod_workspace_bytes(ctypes.byref(desc), ctypes.byref(fb), ctypes.byref(ib)) == 0
    assert ib.value == 2 * (-(-(info.image_ints + 8 * (256 - info.grid)) * 4 // 256) * 256)


def test_workspace_sizes():
    desc, keep = plan_desc(decode=dict(qo_lens=[1] * 4, kv_lens=[5000] * 4), hqo=8, hkv=1,
                           decode_chunk=512)
    rc, img, info = compute(desc)
    assert info.n_slots == 4 * 10
    assert info.float_ws_bytes == info.n_slots * (32 * 128 + 32) * 4
    # two plans alternate between the halves of the int workspace
    assert info.int_ws_bytes == 2 * (-(-info.image_ints * 4 // 256) * 256)


@pytest.mark.parametrize("case,code", [
    (dict(hqo=6, hkv=4), _lib.POD_ERR_INVALID),
    (dict(head_dim=64), _lib.POD_ERR_UNSUPPORTED),
    (dict(page_size=0), _lib.POD_ERR_INVALID),
    (dict(dtype=7), _lib.POD_ERR_UNSUPPORTED),
    (dict(hqo=256, hkv=1), _lib.POD_ERR_UNSUPPORTED),
    (dict(order=9), _lib.POD_ERR_INVALID),
    (dict(hqo=2048, hkv=16, sinks=1), _lib.POD_ERR_UNSUPPORTED),
    (dict(hqo=32768, hkv=32768), _lib.POD_ERR_UNSUPPORTED),
])
def test_invalid_plan_parameters(case, code):
    args = dict(prefill=dict(qo_lens=[10], kv_lens=[10]), hqo=8, hkv=2)
    args.update(case)
    if args.get("page_size", 16) == 0:
        args["prefill"] = dict(qo_lens=[10], kv_lens=[10], qo_indptr=[0, 10], kv_indptr=[0, 1],
                               last_page_len=[10])
    desc, keep = plan_desc(**args)
    rc, _, _ = compute(desc)
    assert rc == code


@pytest.mark.parametrize("scale,code", [(1e6, _lib.POD_OK), (2e6, _lib.POD_ERR_INVALID),
                                        (float("nan"), _lib.POD_ERR_INVALID)])
def test_scale_range(scale, code):
    # the query-tile softmax keeps scale * log2(e) * (-1e30) finite in fp32
    desc, keep = plan_desc(prefill=dict(qo_lens=[10], kv_lens=[10], sm_scale=scale), hqo=8, hkv=2)
    rc, _, _ = compute(desc)
    assert rc == code


@pytest.mark.parametrize("role", [dict(qo_indptr=[1, 10]),
                                  dict(qo_indptr=[0, 10], kv_indptr=[0, 0]),
                                  dict(last_page_len=[0]),
                                  dict(last_page_len=[17]),
                                  dict(qo_indptr=[0, 40])])
def test_invalid_page_tables(role):
    base = dict(qo_lens=[10], kv_lens=[20])
    base.update(role)
    desc, keep = plan_desc(prefill=base, hqo=8, hkv=2)
    rc, _, _ = compute(desc)
    assert rc == _lib.POD_ERR_INVALID
    assert _lib.load().pod_last_error()


@pytest.mark.parametrize("hq,hk,kv_len", [(64, 8, 32768), (32, 32, 32768), (8, 8, 65536), (8, 1, 262144)])
def test_workspace_query_of_long_single_decodes(hq, hk, kv_len):
    """The float workspace a plan needs is its split slots times one partial
    state (32 rows x 128 O + 32 LSE, fp32); long single decodes need more than
    the 16 MiB the single-decode call once allocated, and the binding's query
    reports the same sizes as the planner."""
    from serving_attention_amd import BatchPOD
    kw = dict(num_qo_heads=hq, num_kv_heads=hk, head_dim=128, page_size=1, causal_d=False, num_cus=256)
    fb, ib = BatchPOD.workspace_bytes(None, None, None, [0, 1], [0, kv_len], [1], **kw)
    desc, keep = plan_desc(decode=dict(qo_lens=[1], kv_lens=[kv_len], causal=False), hqo=hq, hkv=hk,
                           page_size=1)
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    assert fb == info.float_ws_bytes == info.n_slots * (32 * 128 + 32) * 4
    assert ib == info.int_ws_bytes
    assert info.n_groups > 0 and fb > 16 << 20


@pytest.mark.parametrize("chunk", [0, 64, -1])
@pytest.mark.parametrize("hqo,hkv,q_lens", [(64, 1, [1, 2, 1]), (64, 8, [5, 4, 1]), (128, 1, [1, 3])])
def test_fp8_decode_row_slices(hqo, hkv, q_lens, chunk):
    """An FP8 decode cache puts requests with more than 32 rows (q_len x group)
    into key chunks of 32-row slices: coverage stays exact, each slice of a
    split key range has a split group of its own, and the slices of one key
    range are consecutive items on one die."""
    kv = [300 + 700 * i for i in range(len(q_lens))]
    roles = [([70], [300], True, -1), (q_lens, kv, True, -1)]
    desc, keep = plan_desc(prefill=dict(qo_lens=roles[0][0], kv_lens=roles[0][1]),
                           decode=dict(qo_lens=q_lens, kv_lens=kv), hqo=hqo, hkv=hkv, decode_chunk=chunk)
    desc.decode_kv_dtype = _lib.POD_DTYPE_FP8_E4M3
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    im = check_coverage(img, roles, hqo, hkv)
    g = hqo // hkv
    items = [it for it in im["items"]]
    dec_chunks = [i for i, it in enumerate(items) if int(it[0]) & FLAG_CHUNK and int(it[0]) & FLAG_ROLE]
    assert dec_chunks and all(int(items[i][0]) & FLAG_CHUNK for i in range(len(items))
                              if int(items[i][0]) & FLAG_ROLE)
    assert max(int(items[i][3]) for i in dec_chunks) >= 32
    # slices of one key range share a die (workgroup w runs on die w % 8)
    die = {}
    for i in dec_chunks:
        it = items[i]
        w = int(im["wg_of_item"][i])
        if w < 0:
            continue          # shared pool: any workgroup
        die.setdefault((int(it[1]), int(it[2]), int(it[5])), set()).add(w % 8)
    assert all(len(v) == 1 for v in die.values())


def test_bf16_large_group_decode_still_uses_tiles():
    desc, keep = plan_desc(decode=dict(qo_lens=[1, 2], kv_lens=[100, 300]), hqo=64, hkv=1)
    rc, img, info = compute(desc)
    im = decode_image(img)
    assert not any(int(it[0]) & FLAG_CHUNK for it in im["items"])


# ------------------------------------------------------------ random plans (property test)

from hypothesis import HealthCheck, given, settings, strategies as st  # noqa: E402


@st.composite
def random_plans(draw):
    hkv = draw(st.sampled_from([1, 2, 4, 8]))
    g = draw(st.sampled_from([1, 2, 3, 8, 16, 64, 128]))
    ps = draw(st.sampled_from([1, 5, 16, 64]))
    fp8 = draw(st.booleans())
    roles = []
    for role in ("prefill", "decode"):
        n = draw(st.integers(0, 4))
        if n == 0:
            roles.append(None)
            continue
        causal = draw(st.booleans())
        w = draw(st.sampled_from([-1, 0, 7, 100]))
        max_q = 90 if role == "prefill" else 6
        q_lens = draw(st.lists(st.integers(0 if role == "prefill" else 1, max_q), min_size=n, max_size=n))
        kv_lens = [draw(st.integers(max(1, q if causal else 1), 400)) for q in q_lens]
        roles.append(dict(qo_lens=q_lens, kv_lens=kv_lens, causal=causal, window_left=w))
    return dict(hkv=hkv, g=g, ps=ps, fp8=fp8, roles=roles,
                chunk=draw(st.sampled_from([0, 64, 192, -1])), order=draw(st.integers(0, 3)),
                num_cus=draw(st.sampled_from([4, 8, 40, 256])))


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(random_plans())
def test_random_plans_cover_every_visible_key_once(plan):
    """Random plans of both roles: every (row, kv head, visible key) is covered
    exactly once, split groups are consistent, every item sits in one
    workgroup list or in the shared pool, a grid below the CU count gives each
    workgroup at most one item and no pool, and an FP8 decode cache puts every
    decode item in a key chunk."""
    hkv, g = plan["hkv"], plan["g"]
    if g * hkv > 1024:
        g = max(1, 1024 // hkv)
    roles = plan["roles"]
    desc, keep = plan_desc(prefill=roles[0], decode=roles[1], hqo=hkv * g, hkv=hkv, page_size=plan["ps"],
                           num_cus=plan["num_cus"], decode_chunk=plan["chunk"], order=plan["order"])
    if plan["fp8"]:
        desc.decode_kv_dtype = _lib.POD_DTYPE_FP8_E4M3
    rc, img, info = compute(desc)
    assert rc == _lib.POD_OK
    spec = [(r["qo_lens"], r["kv_lens"], r["causal"], r["window_left"]) if r else ([], [], True, -1)
            for r in roles]
    im = check_coverage(img, spec, hkv * g, hkv)
    grid = info.grid
    assert 0 < grid <= plan["num_cus"]
    pf, pc = im["pool_first"], im["pool_count"]
    assert np.all(im["wg_of_item"][:pf] >= 0) and np.all(im["wg_of_item"][pf:] == -1)
    assert all(int(it[0]) & FLAG_CHUNK for it in im["items"][pf:])
    if grid < plan["num_cus"]:
        assert pc == 0 and all(int(wg[1]) + int(wg[2]) <= 1 for wg in im["wgs"])
    if plan["fp8"]:
        assert all(int(it[0]) & FLAG_CHUNK for it in im["items"] if int(it[0]) & FLAG_ROLE)
