"""The seeded generators: named lengths, page tables and poison placement."""
import numpy as np
import torch

import oracle
from workloads import build, named_spec, RoleSpec, WorkloadSpec


def test_named_lengths():
    s = named_spec("batch_prefill")
    assert s.prefill.qo_lens == [1711, 409, 577, 680]
    s = named_spec("pod_chunked")
    assert min(s.decode.kv_lens) == 1053 and max(s.decode.kv_lens) == 32742
    assert sum(s.decode.kv_lens) == 4325535
    s = named_spec("batch_decode")
    assert s.decode.kv_lens == [257, 183, 238, 52, 275, 529, 448]


def test_page_tables_reproduce_lengths():
    spec = WorkloadSpec(name="t", prefill=RoleSpec([7, 30], [7, 45]),
                        decode=RoleSpec([1, 3, 2], [5, 16, 17]), num_qo_heads=4,
                        num_kv_heads=2, head_dim=16, page_size=4, pool="shared",
                        shuffle_pages=True, spare_pages=3, meta_seed=9, value_seed=9)
    w = build(spec)
    for _, r in w.roles():
        assert oracle.seq_lens(r.kv_indptr, r.last_page_len, 4).tolist() == r.kv_lens
        assert r.q.shape == (sum(r.qo_lens), 4, 16)
    used = np.concatenate([w.prefill.kv_indices, w.decode.kv_indices])
    assert len(set(used.tolist())) == len(used)


def test_poison_marks_only_unreferenced_slots():
    spec = WorkloadSpec(name="t", prefill=None, decode=RoleSpec([1, 1], [5, 9]),
                        num_qo_heads=2, num_kv_heads=1, head_dim=8, page_size=4,
                        spare_pages=2, dtype="bf16", meta_seed=1, value_seed=2)
    w = build(spec, poison=True)
    r = w.decode
    k = r.k_pool.float()
    for b in range(2):
        for j in range(r.kv_lens[b]):
            page = r.kv_indices[r.kv_indptr[b] + j // 4]
            assert torch.isfinite(k[page, j % 4]).all()
    assert torch.isnan(k).any()


def test_values_are_seeded():
    a = build(named_spec("batch_decode"))
    b = build(named_spec("batch_decode"))
    assert torch.equal(a.decode.q, b.decode.q)
    assert torch.equal(a.pools[0], b.pools[0])
