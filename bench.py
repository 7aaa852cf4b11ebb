"""POD step benchmark on one MI355X.

A step is one pass of the whole path over one batch: plan() (host work list +
its upload) followed by one fused run() launch. Inputs are synthetic, seeded
and resident in HBM before the timed region. Per layer the KV cache and the
queries differ, as in the per-layer loop of the POD article's examples, so a
step does not find the previous step's KV in the caches.

Prints one JSON line. `value` is the mean step latency in microseconds. The
default workload is the chunked-prefill POD step at serving scale (a 4096-token
chunk on a 16384-token prefix plus 256 four-token decodes, window 4096, sinks);
the other named workloads run with --workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "POD step latency (µs); prefill TFLOP/s + decode KV HBM GB/s vs roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
KERNEL_NAME = "pod_grid_kernel"
# GPU spin ahead of each timed launch (about 100 us at the shader clock)
SPIN_CYCLES = 200_000

DESCR = {
    "single_decode": "single-request decode: q [32,128] fp16, K/V [2048,32,128] fp16, NHD",
    "batch_decode": "batch paged decode: 7 requests, 64/8 heads, page_size 16, 128 pages, fp16",
    "batch_prefill": "batch paged causal prefill: 4 requests (1711, 409, 577, 680 tokens), 32/8 heads, "
                     "page_size 16, shuffled pages, bf16",
    "pod": "POD fused step: 2 x 2048-token causal prefill + 128 x 1-token decode on 2048 keys, "
           "64/8 heads, head_dim 128, page_size 1, bf16",
    "pod_chunked": "chunked-prefill POD: 4096-token chunk on a 16384-token prefix + 256 x 4-token "
                   "decode (kv 1024..32768), window_left 4096, fp32 sinks, 64/8 heads, page_size 16, bf16",
    "pod_fp8": "POD fused step as `pod` with the decode K/V cache in FP8 E4M3 (q_scale 1, "
               "k_scale 0.75, v_scale 1.25); q, prefill K/V and outputs bf16",
}


def work_counts(w):
    """Algorithmic work of one step: FLOPs over valid (row, key) pairs and HBM
    bytes with every needed K/V row of each kv head counted once."""
    spec = w.spec
    D, Hq, Hk = spec.head_dim, spec.num_qo_heads, spec.num_kv_heads
    eb = 2
    out = {}
    for name, r in w.roles():
        kv_eb = 1 if (name == "decode" and spec.decode_kv_dtype == "fp8_e4m3") else eb
        pairs = 0
        kv_tokens = 0
        for qo, kv in zip(r.qo_lens, r.kv_lens):
            if qo == 0:
                continue
            lo_first = None
            for i in range(qo):
                p = kv - qo + i
                hi = p if r.causal else kv - 1
                lo = max(0, p - r.window_left) if r.window_left >= 0 else 0
                pairs += max(0, hi - lo + 1)
                lo_first = lo if lo_first is None else min(lo_first, lo)
            last_hi = kv - 1
            kv_tokens += last_hi - lo_first + 1
        rows = sum(r.qo_lens)
        flops = 4.0 * D * Hq * pairs
        kv_bytes = float(kv_tokens) * Hk * D * 2 * kv_eb
        io_bytes = rows * Hq * D * eb * 2 + rows * Hq * 4
        out[name] = dict(flops=flops, kv_bytes=kv_bytes, io_bytes=io_bytes, rows=rows)
    return out


def _code_only(text):
    """C/C++ source without comments and blank space (string literals kept), so
    an edit of a comment does not mark the measured kernel as changed."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash():
    """Hash of the code (comments and spacing left out) of the sources that
    decide what the kernel reads and writes."""
    h = hashlib.sha256()
    for f in ("planner.cpp", "pod_api.cpp", "pod_kernels.hip", "pod_internal.h"):
        with open(os.path.join(ROOT, "serving_attention_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"pod_grid_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def make_layers(name, n_layers, device):
    from workloads import build, named_spec
    layers = []
    for i in range(n_layers):
        spec = named_spec(name)
        spec.value_seed += 7919 * i
        layers.append(build(spec, device=device))
    return layers


def plan(pod, w, roles, decode_chunk, order):
    import torch
    spec = w.spec
    p = w.prefill if "prefill" in roles else None
    d = w.decode if "decode" in roles else None
    pod.plan(p.qo_indptr if p else None, p.kv_indptr if p else None, p.last_page_len if p else None,
             d.qo_indptr if d else None, d.kv_indptr if d else None, d.last_page_len if d else None,
             num_qo_heads=spec.num_qo_heads, num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
             page_size=spec.page_size,
             dtype={"f16": torch.float16, "bf16": torch.bfloat16}[spec.dtype],
             causal_p=p.causal if p else True, causal_d=d.causal if d else True,
             window_left_p=p.window_left if p else -1, window_left_d=d.window_left if d else -1,
             sm_scale_p=p.sm_scale if p else None, sm_scale_d=d.sm_scale if d else None,
             sinks=spec.sinks, decode_chunk=decode_chunk, order=order,
             kv_dtype_d=torch.float8_e4m3fn if (d and spec.decode_kv_dtype == "fp8_e4m3") else None)


def run(pod, w, roles, outs):
    p = w.prefill if "prefill" in roles else None
    d = w.decode if "decode" in roles else None
    return pod.run(p.q if p else None, p.kv_cache if p else None, p.kv_indices_dev if p else None,
                   d.q if d else None, d.kv_cache if d else None, d.kv_indices_dev if d else None,
                   sinks=w.sinks if w.spec.sinks else None, return_lse=True,
                   out_p=outs[0][0], lse_p=outs[0][1], out_d=outs[1][0], lse_d=outs[1][1],
                   **fp8_args(w.spec, d is not None))


def fp8_args(spec, has_decode):
    if not has_decode or spec.decode_kv_dtype != "fp8_e4m3":
        return {}
    qs, ks, vs = spec.fp8_scales
    return dict(q_scale_d=qs, k_scale_d=ks, v_scale_d=vs)


def alloc_outs(w, roles):
    import torch
    res = []
    for name in ("prefill", "decode"):
        r = getattr(w, name)
        if r is None or name not in roles:
            res.append((None, None))
        else:
            res.append((torch.empty_like(r.q),
                        torch.empty(r.q.shape[:2], dtype=torch.float32, device=r.q.device)))
    return res


def time_kernel(pod, layers, roles, steps, warmup, decode_chunk, order, replan):
    """Mean wall time per step (plan + launch, GPU kept busy), the launch
    durations inside that timed region (HIP events on the launch stream), and
    the launch durations measured apart with each launch queued ahead of its
    start event."""
    import torch
    outs = [alloc_outs(w, roles) for w in layers]
    plan(pod, layers[0], roles, decode_chunk, order)
    for i in range(warmup):
        w = layers[i % len(layers)]
        if replan:
            plan(pod, w, roles, decode_chunk, order)
        run(pod, w, roles, outs[i % len(layers)])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    plan_s = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        w = layers[i % len(layers)]
        if replan:
            tp = time.perf_counter()
            plan(pod, w, roles, decode_chunk, order)
            plan_s += time.perf_counter() - tp
        ev[i][0].record(stream)
        run(pod, w, roles, outs[i % len(layers)])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)   # us
    # A launch shorter than the host's plan + argument marshalling leaves the
    # GPU idle between steps, and then a start event can fire before its launch
    # is queued. Here each launch (after its plan, as in a step) waits behind a
    # short GPU spin recorded ahead of the start event, so only the launch
    # itself is timed.
    ev2 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for i in range(steps):
        w = layers[i % len(layers)]
        if replan:
            plan(pod, w, roles, decode_chunk, order)
        torch.cuda._sleep(SPIN_CYCLES)
        ev2[i][0].record(stream)
        run(pod, w, roles, outs[i % len(layers)])
        ev2[i][1].record(stream)
    torch.cuda.synchronize()
    spaced = sorted(a.elapsed_time(b) * 1e3 for a, b in ev2)
    # In the loop, plan() also waits for the launch that last read the
    # workspace half it writes (the host runs ahead of the GPU). Its own cost
    # is timed apart, with the GPU idle, after the timed region.
    plan_cost = None
    if replan:
        n = min(steps, 20)
        tp = 0.0
        for i in range(n):
            torch.cuda.synchronize()
            t = time.perf_counter()
            plan(pod, layers[i % len(layers)], roles, decode_chunk, order)
            tp += time.perf_counter() - t
        plan_cost = tp / n * 1e6
    return dict(step_us=wall / steps * 1e6, kernel_us=sum(kern) / len(kern),
                kernel_p10_us=kern[len(kern) // 10],
                kernel_p90_us=kern[min(len(kern) - 1, (9 * len(kern)) // 10)],
                kernel_spaced_us=sum(spaced) / len(spaced),
                kernel_spaced_p50_us=spaced[len(spaced) // 2],
                plan_us=plan_cost,
                plan_in_loop_us=plan_s / steps * 1e6 if replan else None)


def cpu_baseline(w, budget_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same step,
    scaled to a whole step. Returns the dict of the cpu_baseline field."""
    import numpy as np
    import torch

    import oracle

    threads, blas = None, None
    try:
        from threadpoolctl import threadpool_info
        pools = threadpool_info()
        threads = max((i.get("num_threads", 0) for i in pools), default=None)
        blas = "; ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')}, "
                         f"{i.get('num_threads')} threads)" for i in pools if i.get("user_api") == "blas")
    except Exception:
        pass
    cpu_model = platform.processor() or platform.machine()
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    spec = w.spec
    sinks = w.sinks.cpu().numpy() if spec.sinks else None
    est = 0.0
    parts = []
    for name, r in w.roles():
        # host copies of a few requests' pages, made before the clock starts
        rng = np.random.default_rng(0)
        order = rng.permutation(r.batch)
        t_role, rows_done, rows_total = 0.0, 0, sum(r.qo_lens)
        for b in order:
            if t_role > budget_s / 2 and rows_done > 0:
                break
            p0, p1 = int(r.kv_indptr[b]), int(r.kv_indptr[b + 1])
            idx = torch.from_numpy(r.kv_indices[p0:p1].astype(np.int64)).to(r.k_pool.device)
            if r.k_pool.dtype == torch.float8_e4m3fn:   # the oracle decodes FP8 itself
                kp = oracle.e4m3_to_float(r.k_pool.view(torch.uint8).index_select(0, idx).cpu().numpy())
                vp = oracle.e4m3_to_float(r.v_pool.view(torch.uint8).index_select(0, idx).cpu().numpy())
            else:
                kp = r.k_pool.index_select(0, idx).float().cpu().numpy()
                vp = r.v_pool.index_select(0, idx).float().cpu().numpy()
            q0, q1 = int(r.qo_indptr[b]), int(r.qo_indptr[b + 1])
            q = r.q[q0:q1].float().cpu().numpy()
            qo = q1 - q0
            # long requests: a block of consecutive rows (every row costs the same in the oracle)
            nrows = qo if qo <= 64 else 64
            t = time.perf_counter()
            oracle.attend_role(q, kp, vp, np.array([0, qo]), np.array([0, p1 - p0]), None,
                               r.last_page_len[b:b + 1], spec.page_size, spec.num_qo_heads,
                               spec.num_kv_heads, r.causal, r.window_left, r.sm_scale, sinks,
                               rows_of=lambda _: np.arange(qo - nrows, qo))
            t_role += time.perf_counter() - t
            rows_done += nrows
        est += t_role * rows_total / rows_done
        parts.append(f"{name}: {rows_done} of {rows_total} rows")
    return {"value": est * 1e6, "unit": "us", "cores": threads or os.cpu_count(),
            "kind": "oracle",
            "sample": "fp64 numpy oracle timed on " + "; ".join(parts) +
                      " (last rows of randomly chosen requests), scaled by rows to one step",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model, "blas": blas or "unknown"}


CASCADE = dict(prefix=1536, suffix=512, requests=128, num_qo_heads=64, num_kv_heads=8, page_size=16)


def timed_events(fn, steps, warmup):
    """Mean duration (us) of fn() over `steps` calls, HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(s)
        fn()
        b.record(s)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps * 1e3


def cascade_bench(args):
    """Shared-prefix decode: 128 one-token requests whose 2048 keys are a shared
    1536-token prefix plus 512 keys of their own (the decode shape of the `pod`
    workload with three quarters of each context shared). Two-level cascade: one
    fused launch (prefix as the prefill role over all 128 rows, suffixes as the
    decode role) plus the merge, against the one-level decode that reads every
    request's 2048 keys."""
    import torch
    from serving_attention_amd import BatchPOD, merge_states
    from workloads import build_cascade
    c = CASCADE
    cw = build_cascade(c["prefix"], [c["suffix"]] * c["requests"], q_len=1,
                       num_qo_heads=c["num_qo_heads"], num_kv_heads=c["num_kv_heads"],
                       page_size=c["page_size"], device="cuda")
    ws = torch.empty(128 << 20, dtype=torch.uint8, device="cuda")
    kv = (cw.k_pool, cw.v_pool)
    rows = int(cw.qo_indptr[-1])
    H, D = c["num_qo_heads"], 128
    kw = dict(num_qo_heads=H, num_kv_heads=c["num_kv_heads"], head_dim=D,
              page_size=c["page_size"], dtype=torch.bfloat16)
    idx_pre = torch.from_numpy(cw.prefix_indices).cuda()
    idx_suf = torch.from_numpy(cw.suffix_indices).cuda()
    idx_flat = torch.from_numpy(cw.flat_indices).cuda()
    op, lp = torch.empty_like(cw.q), torch.empty(rows, H, device="cuda")
    od, ld = torch.empty_like(cw.q), torch.empty(rows, H, device="cuda")
    o, lse = torch.empty_like(cw.q), torch.empty(rows, H, device="cuda")

    casc = BatchPOD(ws, "NHD", int_workspace_bytes=8 << 20)
    casc.plan([0, rows], [0, len(cw.prefix_indices)], [cw.prefix_last_page_len],
              cw.qo_indptr, cw.suffix_kv_indptr, cw.suffix_last_page_len,
              causal_p=False, causal_d=True, **kw)

    def run_pod():
        casc.run(cw.q, kv, idx_pre, cw.q, kv, idx_suf, return_lse=True,
                 out_p=op, lse_p=lp, out_d=od, lse_d=ld)

    def run_merge():
        merge_states(op, lp, od, ld, out=o, lse_out=lse)

    def run_cascade():
        run_pod()
        run_merge()

    t_casc = timed_events(run_cascade, args.steps, args.warmup)
    t_pod = timed_events(run_pod, args.steps, args.warmup)
    t_merge = timed_events(run_merge, args.steps, args.warmup)

    ws2 = torch.empty(128 << 20, dtype=torch.uint8, device="cuda")
    flat = BatchPOD(ws2, "NHD", int_workspace_bytes=8 << 20)
    flat.plan(None, None, None, cw.qo_indptr, cw.flat_kv_indptr, cw.flat_last_page_len, causal_d=True, **kw)
    fo, fl = torch.empty_like(cw.q), torch.empty(rows, H, device="cuda")
    t_flat = timed_events(lambda: flat.run(None, None, None, cw.q, kv, idx_flat, return_lse=True,
                                           out_d=fo, lse_d=fl), args.steps, args.warmup)
    # the merge at streaming size (the cascade's own merge is launch-bound: 8192
    # (row, head) pairs, 6 MB): 32768 rows x 64 heads, seeded N(0,1) states
    big = 32768
    gen = torch.Generator(device="cuda").manual_seed(11)
    ba = torch.randn(big, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    bb = torch.randn(big, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    bla = torch.randn(big, H, generator=gen, device="cuda")
    blb = torch.randn(big, H, generator=gen, device="cuda")
    bo, bl = torch.empty_like(ba), torch.empty_like(bla)
    t_merge_big = timed_events(lambda: merge_states(ba, bla, bb, blb, out=bo, lse_out=bl),
                               args.steps, args.warmup)
    torch.cuda.synchronize()
    # merge traffic: two O and two LSE in, one of each out (bf16 O, fp32 LSE)
    merge_bytes = rows * H * (3 * D * 2 + 3 * 4)
    big_bytes = big * H * (3 * D * 2 + 3 * 4)
    kv_row = c["num_kv_heads"] * D * 2 * 2          # K and V bytes per token over all kv heads
    print(json.dumps({
        "metric": "shared-prefix decode step latency (us): two-level cascade vs one-level decode",
        "value": t_casc, "unit": "us", "higher_is_better": False, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) values, shuffled pages)",
        "config": {"workload": "cascade", "requests": c["requests"], "prefix": c["prefix"],
                   "suffix": c["suffix"], "heads": f'{H}/{c["num_kv_heads"]}', "page_size": c["page_size"]},
        "cascade_us": t_casc, "cascade_launch_us": t_pod, "merge_us": t_merge, "flat_decode_us": t_flat,
        "speedup_vs_flat": t_flat / t_casc,
        "kv_bytes_cascade": (c["prefix"] + c["requests"] * c["suffix"]) * kv_row,
        "kv_bytes_flat": c["requests"] * (c["prefix"] + c["suffix"]) * kv_row,
        "merge_bytes": merge_bytes,
        "merge_roofline": {"bound": "hbm", "achieved": big_bytes / (t_merge_big * 1e-6) / 1e9,
                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": big_bytes / (t_merge_big * 1e-6) / 1e9 / PEAK_HBM_GBS,
                           "bytes": big_bytes, "kernel_us": t_merge_big,
                           "shape": f"{big} rows x {H} heads x {D}, bf16"},
    }))


def graph_bench(args):
    """Per-layer cost of run(): eager calls through the Python binding against
    replays of one HIP graph captured from a graph-mode context (plan once, then
    `layers` runs back to back, as a model's attention layers would call it).
    Wall time per run with the GPU kept busy, so host overhead shows where the
    kernel is short."""
    import torch
    from serving_attention_amd import BatchPOD
    layers = 32
    w = make_layers(args.workload, 1, "cuda")[0]
    roles = tuple(n for n, _ in w.roles())
    spec = w.spec
    outs = alloc_outs(w, roles)
    res = {}
    for mode in ("eager", "graph"):
        ws = torch.empty(128 << 20, dtype=torch.uint8, device="cuda")
        kw = {}
        if mode == "graph":
            kw = dict(use_cuda_graph=True,
                      prefill_batch_size=w.prefill.batch if w.prefill is not None else 0,
                      decode_batch_size=w.decode.batch if w.decode is not None else 0)
        pod = BatchPOD(ws, spec.kv_layout, int_workspace_bytes=8 << 20, **kw)
        plan(pod, w, roles, args.decode_chunk, args.order)
        run(pod, w, roles, outs)
        torch.cuda.synchronize()
        if mode == "graph":
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(layers):
                    run(pod, w, roles, outs)
            step = g.replay
        else:
            def step():
                for _ in range(layers):
                    run(pod, w, roles, outs)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        res[mode] = (time.perf_counter() - t0) / (args.steps * layers) * 1e6
        del pod
    print(json.dumps({
        "metric": "attention run() cost per layer (us), eager calls vs graph replay",
        "value": res["graph"], "unit": "us", "higher_is_better": False, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "layers_per_step": layers},
        "eager_us_per_layer": res["eager"], "graph_us_per_layer": res["graph"],
        "speedup": res["eager"] / res["graph"],
    }))


def _smi_sample():
    """(socket power W, graphics clock MHz) from one amd-smi reading, or None."""
    import re
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=5)
    except (OSError, subprocess.SubprocessError):
        return None
    pw = re.search(r"SOCKET_POWER:\s*(\d+)", r.stdout)
    gfx = r.stdout.find("GFX_0")
    clk = re.search(r"\n\s+CLK:\s*(\d+)\s*MHz", r.stdout[gfx:]) if gfx >= 0 else None
    if not pw or not clk:
        return None
    return int(pw.group(1)), int(clk.group(1))


def power_bench(args):
    """Board power and graphics clock while each role set of --workload runs
    launch after launch (no planning between them) for --power-secs seconds,
    and for an idle stretch: amd-smi readings in a thread beside the launches.
    Energy per launch = mean power x launch time."""
    import threading
    import torch
    from serving_attention_amd import BatchPOD
    w = make_layers(args.workload, 1, "cuda")[0]
    ws = torch.empty(128 << 20, dtype=torch.uint8, device="cuda")
    pod = BatchPOD(ws, w.spec.kv_layout, int_workspace_bytes=8 << 20)
    all_roles = tuple(n for n, _ in w.roles())
    sets = [(r,) for r in all_roles] + ([all_roles] if len(all_roles) == 2 else []) + [()]
    res = {}
    for roles in sets:
        name = "+".join(roles) or "idle"
        samples, stop = [], threading.Event()

        def sampler():
            time.sleep(0.3)   # let the clock settle
            while not stop.is_set():
                x = _smi_sample()
                if x:
                    samples.append(x)
        if roles:
            outs = alloc_outs(w, roles)
            plan(pod, w, roles, args.decode_chunk, args.order)
            for _ in range(5):
                run(pod, w, roles, outs)
            torch.cuda.synchronize()
        th = threading.Thread(target=sampler)
        th.start()
        n, t0 = 0, time.perf_counter()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        while time.perf_counter() - t0 < args.power_secs:
            if roles:
                for _ in range(20):
                    run(pod, w, roles, outs)
                n += 20
                torch.cuda.synchronize()
            else:
                time.sleep(0.05)
        ev1.record()
        torch.cuda.synchronize()
        stop.set()
        th.join()
        us = ev0.elapsed_time(ev1) * 1e3 / n if n else None
        pw = [p for p, _ in samples]
        ck = [c for _, c in samples]
        res[name] = dict(launches=n, us_per_launch=us, samples=len(samples),
                         power_w=sum(pw) / len(pw) if pw else None, power_w_max=max(pw) if pw else None,
                         gfx_mhz=sum(ck) / len(ck) if ck else None,
                         mj_per_launch=(sum(pw) / len(pw)) * us * 1e-3 if pw and us else None)
        print(json.dumps({"mode": name, **res[name]}), file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "board power (W) and graphics clock (MHz) per role set, launches back to back",
        "value": res.get("+".join(all_roles), {}).get("power_w"), "unit": "W", "higher_is_better": False,
        "n_gpus": 1, "dtype": w.spec.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "seconds_per_mode": args.power_secs},
        "modes": res,
    }))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="pod_chunked", choices=sorted(DESCR))
    ap.add_argument("--layers", type=int, default=None,
                    help="distinct KV caches / queries cycled per step (default: 4, 1 for pod_chunked)")
    ap.add_argument("--decode-chunk", type=int, default=0)
    ap.add_argument("--order", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-roles", action="store_true", help="skip the role-isolated launches")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--only", choices=("prefill", "decode"), default=None,
                    help="time launches that carry one role only (for per-role profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 1 GiB device copies (for scaling rocprofv3 byte counters)")
    ap.add_argument("--graph", action="store_true",
                    help="time per-layer eager run() calls against replays of one captured graph "
                         "(graph-mode context) on --workload")
    ap.add_argument("--power", action="store_true",
                    help="board power and graphics clock (amd-smi) while each role set of --workload "
                         "runs launch after launch, and idle")
    ap.add_argument("--power-secs", type=float, default=4.0)
    ap.add_argument("--cascade", action="store_true",
                    help="time the two-level shared-prefix cascade (one launch + merge) "
                         "against the one-level decode over the same keys")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component; see the sharding notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    from serving_attention_amd import BatchPOD

    if args.cascade:
        cascade_bench(args)
        return
    if args.power:
        power_bench(args)
        return
    if args.graph:
        graph_bench(args)
        return

    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": a.numel() * 4, "copies": 3}))
        return

    n_layers = args.layers or (1 if args.workload == "pod_chunked" else 4)
    layers = make_layers(args.workload, n_layers, "cuda")
    w0 = layers[0]
    ws = torch.empty(128 << 20, dtype=torch.uint8, device="cuda")
    pod = BatchPOD(ws, w0.spec.kv_layout, int_workspace_bytes=8 << 20)
    all_roles = tuple(n for n, _ in w0.roles())
    if args.only:
        all_roles = (args.only,)

    main_t = time_kernel(pod, layers, all_roles, args.steps, args.warmup, args.decode_chunk,
                         args.order, replan=True)
    info = pod.plan_info()
    work = {k: v for k, v in work_counts(w0).items() if k in all_roles}
    flops_p = work.get("prefill", {}).get("flops", 0.0)
    kv_all = sum(v["kv_bytes"] for v in work.values())
    io_all = sum(v["io_bytes"] for v in work.values())
    k_us = main_t["kernel_us"]
    t_star = max(flops_p / (PEAK_BF16_TFLOPS * 1e12), (kv_all + io_all) / (PEAK_HBM_GBS * 1e9)) * 1e6

    roles_out = {}
    if not args.no_roles and len(all_roles) == 2:
        for name in all_roles:
            t = time_kernel(pod, layers, (name,), max(5, args.steps // 2), 2, args.decode_chunk,
                            args.order, replan=False)
            wk = work[name]
            roles_out[name] = dict(
                kernel_us=t["kernel_us"],
                kernel_spaced_us=t["kernel_spaced_us"],
                tflops=wk["flops"] / (t["kernel_us"] * 1e-6) / 1e12,
                kv_gbs=wk["kv_bytes"] / (t["kernel_us"] * 1e-6) / 1e9,
                hbm_gbs=(wk["kv_bytes"] + wk["io_bytes"]) / (t["kernel_us"] * 1e-6) / 1e9)
        plan(pod, w0, all_roles, args.decode_chunk, args.order)

    algo_bytes = kv_all + io_all
    bound = "hbm" if (kv_all + io_all) / (PEAK_HBM_GBS * 1e9) >= flops_p / (PEAK_BF16_TFLOPS * 1e12) else "mfma"
    if bound == "hbm":
        achieved = algo_bytes / (k_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = flops_p / (k_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS}
    roof["traffic"] = committed_traffic(args.workload)
    roof["algorithmic_bytes_per_launch"] = algo_bytes
    roof["kernel"] = KERNEL_NAME
    roof["kernel_us"] = k_us

    result = {
        "metric": METRIC,
        "value": main_t["step_us"],
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_t["step_us"] / 1e3,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w0.spec.dtype,
        "data": "synthetic (seeded N(0,1) values, lengths and page tables of the named workload)",
        "config": {"workload": args.workload, "description": DESCR[args.workload],
                   "layers_cycled": n_layers, "decode_chunk": info["decode_chunk"],
                   "order": args.order, "items": info["n_items"], "grid": info["grid"]},
        "kernel_us": k_us,
        "kernel_p10_us": main_t["kernel_p10_us"],
        "kernel_p90_us": main_t["kernel_p90_us"],
        "kernel_spaced_us": main_t["kernel_spaced_us"],
        "kernel_spaced_p50_us": main_t["kernel_spaced_p50_us"],
        "plan_us": main_t["plan_us"],
        "plan_in_loop_us": main_t["plan_in_loop_us"],
        "prefill_tflops": flops_p / (k_us * 1e-6) / 1e12 if flops_p else None,
        "decode_kv_gbs": work["decode"]["kv_bytes"] / (k_us * 1e-6) / 1e9 if "decode" in work else None,
        "t_star_us": t_star,
        "t_star_frac": t_star / k_us,
        "roles_isolated": roles_out or None,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w0, args.cpu_budget)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
