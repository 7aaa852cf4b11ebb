"""Host logic of bench.py (no GPU): the algorithmic work counts behind the
roofline line, pinned to closed forms of the named workloads' shapes; the
traffic file is used only on matching kernel sources; more than one GPU is
refused."""
import json
import os
import subprocess
import sys

import pytest

import bench
from workloads import named_spec

HEADS_QO, HEADS_KV, D = 64, 8, 128


class _Lengths:
    """The part of a built workload that work_counts reads: its spec and roles."""

    def __init__(self, spec):
        self.spec = spec

    def roles(self):
        return [(n, r) for n, r in (("prefill", self.spec.prefill), ("decode", self.spec.decode)) if r is not None]


def _counts(name):
    return bench.work_counts(_Lengths(named_spec(name)))


def test_pod_bytes_and_flops_closed_form():
    c = _counts("pod")
    # decode: 128 one-token requests on 2048 keys, every key of every kv head read once
    assert c["decode"]["kv_bytes"] == 128 * 2048 * HEADS_KV * D * 2 * 2
    # prefill: 2 causal requests of 2048 tokens read their 2048 keys once per kv head
    assert c["prefill"]["kv_bytes"] == 2 * 2048 * HEADS_KV * D * 2 * 2
    # q and O in bf16, LSE in fp32, per (row, qo head)
    rows = 2 * 2048 + 128
    io = sum(c[r]["io_bytes"] for r in ("prefill", "decode"))
    assert io == rows * HEADS_QO * (D * 2 * 2 + 4)
    total = sum(c[r]["kv_bytes"] + c[r]["io_bytes"] for r in ("prefill", "decode"))
    assert total == 1_230_012_416
    # causal prefill: row i of a 2048-token request sees i + 1 keys
    assert c["prefill"]["flops"] == 4.0 * D * HEADS_QO * 2 * (2048 * 2049 // 2)
    assert c["decode"]["flops"] == 4.0 * D * HEADS_QO * 128 * 2048


def test_pod_chunked_window_bounds_the_keys_read():
    spec = named_spec("pod_chunked")
    c = _counts("pod_chunked")
    w = spec.decode.window_left
    assert w == 4096 and spec.decode.causal
    # 4-token decode rows see keys (kv - 4 + i - w) .. (kv - 4 + i): together the
    # last min(kv, w + 4) keys of the request
    tokens = sum(min(kv, w + q) for q, kv in zip(spec.decode.qo_lens, spec.decode.kv_lens))
    assert c["decode"]["kv_bytes"] == tokens * HEADS_KV * D * 2 * 2
    # the 4096-token chunk on a 16384-token prefix reads keys 16384 - 4096 .. 20479
    assert c["prefill"]["kv_bytes"] == (4096 + 4096) * HEADS_KV * D * 2 * 2
    # row i sees min(16384 + i + 1, w + 1) = w + 1 keys (the prefix is longer than the window)
    assert c["prefill"]["flops"] == 4.0 * D * HEADS_QO * 4096 * (w + 1)


def test_pod_fp8_counts_one_byte_decode_rows():
    c8, c16 = _counts("pod_fp8"), _counts("pod")
    assert c8["decode"]["kv_bytes"] * 2 == c16["decode"]["kv_bytes"]
    assert c8["prefill"] == c16["prefill"]


def test_traffic_file_needs_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "pod_grid_pod_traffic.json").write_text(json.dumps({"source_hash": "abc", "hbm_bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda: "abc")
    assert bench.committed_traffic("pod") == 123.0
    monkeypatch.setattr(bench, "source_hash", lambda: "def")
    assert bench.committed_traffic("pod") is None
    assert bench.committed_traffic("pod_chunked") is None


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_source_hash_ignores_comments_only():
    code = 'int f(int x) {\n  // one\n  return x + 1; /* two */\n}\nconst char* s = "a // b /* c */";\n'
    same = 'int f(int x) {\n  // another comment\n\n  return x + 1;   /* changed */\n}\nconst char* s = "a // b /* c */";\n'
    other = 'int f(int x) {\n  return x + 2;\n}\nconst char* s = "a // b /* c */";\n'
    assert bench._code_only(code) == bench._code_only(same)
    assert bench._code_only(code) != bench._code_only(other)
    assert '"a // b /* c */"' in bench._code_only(code)
