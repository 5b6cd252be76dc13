#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X; prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one sdpa_forward call (every kernel of the path) on one batch of
seeded synthetic input already resident in HBM.  The headline workload is the
bf16 grouped-query decode with head dim 256 (B=1, qL=1, Hq=32, Hkv=8,
Lk=4096, additive [1,1,1,Lk] mask): value = K+V bytes per step / step time.
Decode steps rotate over enough K/V replicas (> 2 x the 256 MB Infinity
Cache) that every step reads cold HBM.  The K steps of a workload are
captured in one HIP graph; after an untimed replay, one replay is timed with
HIP events on the replaying stream, bracketed by synchronisations (the host
launch cost of the Python binding would otherwise dominate a ~10 us step).

roofline (per workload): algorithmic work per step (decode: K+V bytes;
prefill: 4 B Hq Lq Lk D flops, halved for causal) / the graph-timed step.
Every workload listed here runs one kernel launch per step, so this is also
that kernel's launch-to-launch duration, the figure rocprofv3's kernel trace
gives for back-to-back launches (`--summarize-trace` derives it from a
trace).  traffic: HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE
counters (profiles/counters.json) when they were taken on the current
kernel sources.
ceiling: one launch of the library's plain streaming read of the same number
of bytes as the headline decode, timed the same way (cold replicas, graph).
cpu_baseline: the float64 oracle on the host, one process per core, one
(batch, head) per task, on a bounded sample of each workload.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SDPA prefill TFLOP/s + decode KV GB/s, each as % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 matrix
COLD_BYTES = 600 << 20         # K/V replicas per decode run: > 2 x 256 MB Infinity Cache
WORKLOAD_BYTES_PRIMARY = 2 * 8 * 4096 * 256 * 2  # K+V bytes of the headline decode (the ceiling reads as many)
MAX_POOL = 16                  # host cores one GPU's share may use

WORKLOADS = {
    "decode-d256-lk4096": dict(kind="decode", D=256, Lk=4096),
    "decode-d256-lk1024": dict(kind="decode", D=256, Lk=1024),
    "decode-d512-lk4096": dict(kind="decode", D=512, Lk=4096),
    "decode-d512-lk1024": dict(kind="decode", D=512, Lk=1024),
    "prefill-d72-none": dict(kind="prefill72", mask="none"),
    "prefill-d72-boolean": dict(kind="prefill72", mask="boolean"),
    "prefill-d72-causal": dict(kind="prefill72", mask="causal"),
    "prefill-d512-causal": dict(kind="prefill512"),
    "prefill-d256-sliding-w1024": dict(kind="sliding", q_len=4096, kv_len=4096, window=1024),
    "decode-d256-sliding-w1024": dict(kind="sliding", q_len=1, kv_len=4096, window=1024),
    "decode-qk192-v128-lk4096": dict(kind="decode_dv", Lk=4096),
    "tiny-f32": dict(kind="tiny"),
}
PRIMARY = "decode-d256-lk4096"
PREFILL = ("prefill-d512-causal", "prefill-d72-none", "prefill-d72-causal", "prefill-d72-boolean")
CPU_WORKLOADS = ("decode-d256-lk4096", "decode-d512-lk4096", "prefill-d72-none", "prefill-d72-boolean",
                 "prefill-d72-causal", "prefill-d512-causal")


def kernel_hash(name: str = PRIMARY) -> str:
    """Hash of every source the library is built from (any change makes counters stale)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "scaled_dot_product_sdpa_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "sdpa.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def make_case(name: str):
    import sdpa_inputs as si
    w = WORKLOADS[name]
    if w["kind"] == "decode":
        return si.decode_case(w["D"], w["Lk"])
    if w["kind"] == "prefill72":
        return si.prefill72_case(w["mask"])
    if w["kind"] == "prefill512":
        return si.prefill512_case()
    if w["kind"] == "sliding":
        return si.sliding_case(w["q_len"], w["kv_len"], w["window"])
    if w["kind"] == "decode_dv":
        return si.decode_dv_case(w["Lk"])
    return si.tiny_case("random")


def describe(name: str, c) -> dict:
    d = c.dims
    return {"workload": name, "batch": d["batch"], "q_len": d["q_len"], "kv_len": d["kv_len"],
            "n_q_heads": d["n_q_heads"], "n_kv_heads": d["n_kv_heads"], "head_dim": d["head_dim"],
            "v_head_dim": int(c.v.shape[3]),
            "mask": c.mask_kind, "layout": c.layout, "dtype": str(c.q.dtype).replace("torch.", "")}


def work(c) -> tuple[float, str]:
    """Algorithmic work of one call: K+V bytes for decode, flops for prefill.

    Causal prefill counts half the score matrix; a sliding window counts the
    (query, key) pairs it keeps, and a sliding decode the keys any query reaches.
    """
    d = c.dims
    Lq, Lk = d["q_len"], d["kv_len"]
    if Lq <= 8:
        es = c.k.element_size()
        keys = Lk
        if c.mask_kind == "sliding":
            keys = min(Lk, c.meta["window"] + Lq - 1)
        return float(d["batch"] * d["n_kv_heads"] * keys * (d["head_dim"] + c.v.shape[3]) * es), "bytes"
    per_pair = 4.0 * d["batch"] * d["n_q_heads"] * d["head_dim"]
    if c.mask_kind == "sliding":
        w, off = c.meta["window"], Lk - Lq
        pairs = sum(min(w, i + off + 1) for i in range(Lq))
        return per_pair * pairs, "flops"
    f = per_pair * Lq * Lk
    return (f / 2 if c.mask_kind == "causal" else f), "flops"


def launches_per_step(route: str) -> int:
    """Kernel launches one call makes: the split + combine decode route makes two, and so does a
    boolean-mask prefill that builds lane words first."""
    if route.startswith("vector ") and "splits=1 " not in route:
        return 2
    if "lane-words+prepass" in route:
        return 2
    return 1


COVER_CYCLES = 2_000_000  # spin before a timed replay (about 1 ms): the host submits the replay meanwhile


def graph_time(step, steps: int) -> float:
    """ms per step: `steps` calls captured in one graph, one untimed replay, one timed replay.

    The timed replay is queued behind an untimed spin kernel, so the host's submission of the
    replay's launches happens while the GPU spins: the events bracket exactly the `steps` calls
    running back to back, not the submission latency of the first one (on an idle GPU the start
    event fires at once and the first kernel only when its launch arrives)."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                step(i)
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(COVER_CYCLES)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


MARKER = "spin_kernel"  # torch.cuda._sleep's kernel: starts each measured workload in a trace
MARKER_MAX_NS = 100_000  # a marker spins about a microsecond; the spin before a timed replay, a millisecond


def mark_workload():
    """A few-microsecond spin kernel that opens each workload's stretch of a kernel trace."""
    import torch
    torch.cuda._sleep(1000)


def measure(name: str, steps: int, warmup: int, eager: bool = False) -> dict:
    import torch
    import scaled_dot_product_sdpa_amd as sdpa
    import sdpa_inputs as si

    mark_workload()
    c = make_case(name)
    amount, unit = work(c)
    decode = unit == "bytes"
    kv_bytes = 2 * c.k.numel() * c.k.element_size()
    nrep = max(2, -(-COLD_BYTES // kv_bytes)) if decode else 1
    reps = [si.to_device(c) for _ in range(nrep)]
    torch.cuda.synchronize()
    q0 = reps[0][0]
    out = torch.empty(q0.shape[:3] + (c.v.shape[3],), dtype=q0.dtype, device="cuda")
    d = c.dims
    ws_bytes = sdpa.workspace_size(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"],
                                   d["head_dim"], q0.dtype, v_head_dim=c.v.shape[3])
    ws = torch.zeros(max(ws_bytes, 32768), dtype=torch.uint8, device="cuda")  # arrival words start at zero

    def step(i):
        q, k, v, m = reps[i % nrep]
        sdpa.forward(q, k, v, scale=c.scale, mask=m, mask_kind=c.mask_kind, out=out, workspace=ws,
                     window=c.meta.get("window"))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    eager_ms = None
    if eager:  # host launch cost included
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / steps
    ms = graph_time(step, steps)
    route = sdpa.describe_route(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"],
                                d["head_dim"], q0.dtype, c.mask_kind, v_head_dim=c.v.shape[3])
    if decode:
        rate, runit, peak, bound = amount / (ms * 1e-3) / 1e9, "GB/s", HBM_PEAK_GBS, "hbm"
    else:
        peak = FP32_PEAK_TFLOPS if q0.dtype == torch.float32 else BF16_PEAK_TFLOPS
        rate, runit, bound = amount / (ms * 1e-3) / 1e12, "TFLOP/s", "mfma"
    nl = launches_per_step(route)
    roof = {"bound": bound, "achieved": rate, "peak": peak, "unit": runit, "frac": rate / peak,
            "traffic": load_traffic(name), "launches_per_step": nl, "launch_ms": ms / nl,
            "work_per_launch": amount, "work_unit": unit}
    prof = load_profiled(name)
    if prof:  # rocprofv3 kernel durations of the same command (profiles/kernel_times.json)
        roof["profiled"] = {"kernel_us_per_step": prof["step_kernel_us"], "frac": prof["frac_of_peak"],
                            "kernels": {k: round(v["avg_us"], 3) for k, v in prof["kernels"].items()}}
    res = dict(config=describe(name, c), route=route, value=rate, unit=runit, ms_per_step=ms,
               eager_ms_per_step=eager_ms, replicas=nrep, roofline=roof)
    del reps
    torch.cuda.empty_cache()
    return res


def ceiling(nbytes: int, steps: int) -> dict:
    """The library's plain streaming read of nbytes, cold, timed like a decode step."""
    import torch
    import scaled_dot_product_sdpa_amd as sdpa
    mark_workload()
    nrep = max(2, -(-COLD_BYTES // nbytes))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nrep)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i in range(3):
        sdpa.probe_stream_read(bufs[i % nrep], sink)
    ms = graph_time(lambda i: sdpa.probe_stream_read(bufs[i % nrep], sink), steps)
    rate = nbytes / (ms * 1e-3) / 1e9
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "ms_per_launch": ms, "value": rate, "unit": "GB/s", "frac": rate / HBM_PEAK_GBS,
            "kernel": "stream_read_kernel (one 256-thread workgroup per CU, 8 x 16-byte loads in flight)"}


# ---------------------------------------------------------------- CPU baseline
TRACE_LIB = os.path.join(ROOT, "scaled_dot_product_sdpa_amd", "libsdpa_trace.so")
TRACE_BUILD = ("python3 -m scaled_dot_product_sdpa_amd.build -D SDPA_TRACE_DECODE=1 "
               "--out scaled_dot_product_sdpa_amd/libsdpa_trace.so --build-dir scaled_dot_product_sdpa_amd/_build/trace")
TRACE_WORDS = 14
TRACE_STAGES = (  # (record word, what the workgroup has done by then, last workgroups only)
    (0, "started (arguments loaded)", False),
    (1, "wave 0: first 16-key block in registers (its S^T products done)", False),
    (3, "every wave: its keys done (after the merge barrier)", False),
    (8, "wave partials in LDS (barrier)", False),
    (9, "partial stores issued", False),
    (4, "partial stored in L2 (s_waitcnt vmcnt(0) + barrier)", False),
    (5, "arrival add returned", False),
    (10, "last workgroup of a group: merge weights in LDS", True),
    (11, "last workgroup of a group: weighted partial sums in LDS", True),
    (6, "last workgroup of a group: output stored", True),
    (12, "(a second clock read right after 'every wave: its keys done')", False),
    (13, "(a second clock read right after 'partial stores issued')", False),
)


def timeline(name: str, calls: int, warmup: int, command: str, burst: int = 20) -> str:
    """In-kernel timeline of the single-launch decode kernel, from the timeline build of the library
    (libsdpa_trace.so): every workgroup records the constant 100 MHz clock at the stages of
    TRACE_STAGES.  Each sample is the last of `burst` calls launched back to back (the GPU busy, as
    in a timed step); times are relative to the first workgroup's start in that call.  Returns a
    markdown summary."""
    import re
    import statistics as stt
    import numpy as np
    import torch
    import scaled_dot_product_sdpa_amd as sdpa
    import sdpa_inputs as si

    c = make_case(name)
    d = c.dims
    dv = int(c.v.shape[3])
    kv_bytes = 2 * c.k.numel() * c.k.element_size()
    nrep = max(2, -(-COLD_BYTES // kv_bytes))
    reps = [si.to_device(c) for _ in range(nrep)]
    q0 = reps[0][0]
    out = torch.empty(q0.shape[:3] + (dv,), dtype=q0.dtype, device="cuda")
    ws_bytes = sdpa.workspace_size(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"],
                                   d["head_dim"], q0.dtype, v_head_dim=dv)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device="cuda")
    route = sdpa.describe_route(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"],
                                d["head_dim"], q0.dtype, c.mask_kind, v_head_dim=dv)
    if not route.startswith("vector-fused"):
        raise SystemExit(f"{name}: not the single-launch decode kernel ({route})")
    G, S = (int(re.search(k + r"=(\d+)", route).group(1)) for k in ("groups", "splits"))
    rv = min(16, d["n_q_heads"] // d["n_kv_heads"] * d["q_len"])
    a256 = lambda x: (x + 255) // 256 * 256
    slots = G * S * rv
    off = 32768 + a256(slots * dv * 4) + a256(slots * 8)
    nwg = G * S
    rb = TRACE_WORDS * 8
    if S < 2 or off + nwg * rb > ws_bytes:
        raise SystemExit(f"{name}: no timeline records in this library's workspace (is it the timeline build?)")
    recs, durs = [], []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def step(i):
        q, k, v, m = reps[i % nrep]
        sdpa.forward(q, k, v, scale=c.scale, mask=m, mask_kind=c.mask_kind, out=out, workspace=ws)

    for i in range(3):
        step(i)
    # `burst` calls back to back in one graph, replayed like a timed step; the last call's records are kept
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for i in range(burst):
                step(i)
    torch.cuda.current_stream().wait_stream(st)
    for i in range(warmup + calls):
        ws[off:off + nwg * rb].zero_()
        torch.cuda.synchronize()
        torch.cuda._sleep(COVER_CYCLES)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        if i >= warmup:
            r = ws[off:off + nwg * rb].view(torch.int64).view(nwg, TRACE_WORDS).cpu().numpy().copy()
            if (r[:, 0] == 0).any() or (r[:, 5] == 0).any():
                raise SystemExit("incomplete timeline records (a group recomputed off its XCD?)")
            recs.append(r)
            durs.append(e0.elapsed_time(e1) * 1000 / burst)
    us = 0.01  # microseconds per tick of the 100 MHz clock
    per = {k: ([], []) for k, _, _ in TRACE_STAGES}
    segs = {n: [] for n in ("load", "keys", "store", "arrive", "merge", "span")}
    crit = {k: [] for k, _, _ in TRACE_STAGES}
    crit_keys = []
    for r in recs:
        t0 = r[:, 0].min()
        t = (np.where(r > 0, r, t0) - t0) * us
        last = ((r[:, 7] >> 4) & 1) == 1
        grp = r[:, 7] >> 16
        for k, _, lo in TRACE_STAGES:
            col = t[last, k] if lo else t[:, k]
            per[k][0].append(float(np.median(col)))
            per[k][1].append(float(col.max()))
        segs["load"].append(float(np.median(t[:, 1] - t[:, 0])))
        segs["keys"].append(float(np.median(t[:, 3] - t[:, 1])))
        segs["store"].append(float(np.median(t[:, 4] - t[:, 3])))
        segs["arrive"].append(float(np.median(t[:, 5] - t[:, 4])))
        segs["merge"].append(float(np.median(t[last, 6] - t[last, 5])))
        segs["span"].append(float(t[last, 6].max()))
        w = int(np.argmax(np.where(last, t[:, 6], -1)))  # the workgroup that finished the call
        for k, _, _ in TRACE_STAGES:
            crit[k].append(float(t[w, k]))
        crit_keys.append(float(t[grp == grp[w], 3].max()))
    med = stt.median
    lines = [f"# Single-launch decode: in-kernel timeline, {name}", "",
             f"Route: `{route}`.", "",
             "Built and run from the repository root (the timeline build is the library compiled with",
             "`SDPA_TRACE_DECODE=1`: each workgroup records the 100 MHz real-time clock at the stages below",
             "into the workspace; the product build has none of it):", "",
             "```", TRACE_BUILD, command, "```", "",
             f"{calls} samples on cold K/V replicas, each the last of {burst} calls replayed back to back from one",
             "graph (as a timed step); times in µs from the first workgroup's start in that call, medians over the",
             f"samples; 10 ns resolution. HIP-event time per call of a replay: {med(durs):.2f} µs.", "",
             "| stage | median workgroup | last workgroup |", "|---|---|---|"]
    for k, label, _ in TRACE_STAGES:
        lines.append(f"| {label} | {med(per[k][0]):.2f} | {med(per[k][1]):.2f} |")
    lines += ["", "Per-workgroup segments (median workgroup, medians over the calls):", "",
              "| segment | µs |", "|---|---|",
              f"| start → first block in registers (load latency under the full stream) | {med(segs['load']):.2f} |",
              f"| first block → every wave's keys done | {med(segs['keys']):.2f} |",
              f"| keys done → partial stored in L2 (wave merge, stores, their completion) | {med(segs['store']):.2f} |",
              f"| partial stored → arrival add returned | {med(segs['arrive']):.2f} |",
              f"| arrival → output stored (last workgroups: the merge of {S} partials) | {med(segs['merge']):.2f} |",
              f"| first start → last output stored (in-kernel span) | {med(segs['span']):.2f} |",
              "", "Critical path (the workgroup that stored the call's last output, medians over the calls):", "",
              "| stage | µs |", "|---|---|"]
    for k, label, _ in TRACE_STAGES:
        lines.append(f"| {label} | {med(crit[k]):.2f} |")
    lines.append(f"| latest split of that group done with its keys | {med(crit_keys):.2f} |")
    return "\n".join(lines) + "\n"


def _oracle_task(args):
    """One (batch, query head) of a workload through the float64 oracle, single-threaded BLAS."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    q, k, v, scale, kind, mask, rows = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        oracle.sdpa(q, k, v, np.float32(scale), kind, mask, q_rows=rows)
        return time.perf_counter() - t0


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(name: str, budget_s: float, pool, cores: int) -> dict:
    """The float64 oracle, as it is, on a bounded sample of the workload: (batch, query
    head) tasks spread over a process pool, rows sampled for long prefills."""
    import numpy as np
    c = make_case(name)
    amount, unit = work(c)
    d = c.dims
    B, Hq, Hkv, Lq = d["batch"], d["n_q_heads"], d["n_kv_heads"], d["q_len"]
    rep = Hq // Hkv
    q, k, v = (t.double().numpy() for t in (c.q, c.k, c.v))
    mask = None
    if c.mask_kind == "sliding":
        mask = c.meta["window"]
    elif c.mask is not None:
        mask = c.mask.double().numpy() if c.mask_kind == "additive" else c.mask.numpy()
    rows, frac_rows = None, 1.0
    if Lq > 64:  # prefill: evenly spaced query rows, work scaled by their share
        n = 64
        rows = np.linspace(0, Lq - 1, n).astype(np.int64)
        frac_rows = n / Lq
        if c.mask_kind == "causal":  # a causal row's work grows with its index: scale by the keys kept
            off = d["kv_len"] - Lq
            frac_rows = float(sum(min(d["kv_len"], int(r) + off + 1) for r in rows)) / (Lq * (Lq + 1) / 2)
    tasks = []
    for b in range(B):
        for h in range(Hq):
            g = h // rep
            m = mask
            if isinstance(mask, np.ndarray):
                m = mask[min(b, mask.shape[0] - 1):min(b, mask.shape[0] - 1) + 1,
                         min(h, mask.shape[1] - 1):min(h, mask.shape[1] - 1) + 1]
            tasks.append((q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1], c.scale, c.mask_kind, m,
                          rows))
    per_call = amount * frac_rows  # one full pass over every (b, h), sampled rows
    t0 = time.perf_counter()
    passes = 0
    while True:
        list(pool.map(_oracle_task, tasks))
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / passes
    if unit == "bytes":
        val, u = per_call / dt / 1e9, "GB/s"
    else:
        val, u = per_call / dt / 1e12, "TFLOP/s"
    sample = (f"{name}: every (batch, head) of one call, {passes} passes in {dt * passes:.1f}s" if rows is None else
              f"{name}: {len(rows)} of {Lq} query rows of every (batch, head), work scaled by "
              f"{frac_rows:.4f}, {passes} passes in {dt * passes:.1f}s")
    return {"value": val, "unit": u, "cores": cores, "kind": "oracle", "sample": sample,
            "seconds_per_call": dt / frac_rows, "cpu_model": cpu_model(), "tasks": len(tasks)}


def load_traffic(name: str):
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        data = json.load(open(p))
    except Exception:
        return None
    ent = data.get("workloads", {}).get(name)
    if not ent or ent.get("kernel_hash") != kernel_hash(name):
        return None
    return ent.get("hbm_bytes_per_launch")


# ------------------------------------------------------- rocprofv3 post-processing
def _short(kernel: str) -> str:
    s = kernel.split("(")[0].replace("sdpa_dev::", "").replace("void ", "")
    return s


def trace_runs(trace_csv: str, steps: int):
    """Per workload of a default bench run, from a rocprofv3 kernel trace of it: the library's kernels
    of each workload's timed graph replay (the last `steps` launches of each kernel in that
    workload's stretch of the trace), their average duration and the average start-to-start period.

    Workloads are measured one after another, each opened by a marker kernel (mark_workload);
    the stretches between markers are named in the bench's order: the primary workload, the
    others in WORKLOADS order, then the streaming-read ceiling.  (A trace without markers is
    split at gaps of more than 5 ms instead.)"""
    rows = list(csv.DictReader(open(trace_csv)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    def is_marker(r):
        return MARKER in r["Kernel_Name"] and int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) < MARKER_MAX_NS
    marked = any(is_marker(r) for r in rows)
    segs, cur, prev = [], [], None
    for r in rows:
        s0, e0 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        if is_marker(r) if marked else (prev is not None and s0 - prev > 5_000_000):
            if cur:
                segs.append(cur)
            cur = []
        cur.append(r)
        prev = e0
    segs.append(cur)
    order = [PRIMARY] + [w for w in WORKLOADS if w != PRIMARY]
    out, i = [], 0
    for seg in segs:
        ours = [r for r in seg if "sdpa_dev::" in r["Kernel_Name"]]
        kernels = {}
        for r in ours:
            grid = int(r["Grid_Size_X"]) * int(r.get("Grid_Size_Y") or 1) * int(r.get("Grid_Size_Z") or 1)
            k = (_short(r["Kernel_Name"]), grid // max(1, int(r["Workgroup_Size_X"])))
            kernels.setdefault(k, []).append(r)
        lib = {k: v for k, v in kernels.items() if not k[0].startswith("stream_read_kernel")}
        if lib and i < len(order):
            out.append((order[i], _run_stats(lib, steps)))
            i += 1
        probe = {k: v for k, v in kernels.items() if k[0].startswith("stream_read_kernel")}
        if probe:
            out.append(("ceiling", _run_stats(probe, steps)))
    return out


def _run_stats(kernels: dict, steps: int) -> dict:
    res = {}
    for (k, wg), rs in kernels.items():
        last = rs[-steps:]
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in last]
        st = [int(r["Start_Timestamp"]) for r in last]
        per = [(b - a) / 1000.0 for a, b in zip(st, st[1:])]
        ds = sorted(d)
        q = lambda f: ds[min(len(ds) - 1, int(round(f * (len(ds) - 1))))]
        res[(k, wg)] = {"workgroups": wg, "launches": len(rs), "timed": len(last), "avg_us": sum(d) / len(d),
                        "p10_us": q(0.1), "median_us": q(0.5), "p90_us": q(0.9),
                        "period_us": (sum(per) / len(per)) if per else None}
    return res


def summarize_trace(trace_csv: str, command: str, steps: int = 20) -> str:
    """Markdown summary of a rocprofv3 kernel trace of a default bench run (see trace_runs), plus
    profiles/kernel_times.json with the same figures keyed by the kernel sources' hash."""
    runs = trace_runs(trace_csv, steps)
    out = ["Command (repo root, one MI355X, `export TMPDIR=/tmp`):", "", "```", command, "```", "",
           f"Per workload, the library's kernels of the timed graph replay (the last {steps} launches of each "
           "kernel in that workload's part of the trace): average kernel duration, its p10 / median / p90 over "
           "those launches, and the average start-to-start period of consecutive launches. A step of a "
           "two-kernel route is the sum of its kernels.", "",
           "| workload | kernel | workgroups | launches (timed) | avg kernel us | p10 / median / p90 us | "
           "avg period us | work per launch | rate from avg kernel | of peak |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    table = {}
    for name, ks in runs:
        tot = sum(v["avg_us"] for v in ks.values())
        work_amt, unit, peak = None, None, BF16_PEAK_TFLOPS
        if name in WORKLOADS:
            c = make_case(name)
            work_amt, unit = work(c)
            if c.q.element_size() == 4:
                peak = FP32_PEAK_TFLOPS
        elif name == "ceiling":
            work_amt, unit = float(WORKLOAD_BYTES_PRIMARY), "bytes"

        def rate_of(us):
            if work_amt is None:
                return "", "", None
            if unit == "bytes":
                r = work_amt / (us * 1e-6) / 1e9
                return f"{r:.0f} GB/s", f"{r / HBM_PEAK_GBS:.3f}", r / HBM_PEAK_GBS
            r = work_amt / (us * 1e-6) / 1e12
            return f"{r:.1f} TFLOP/s", f"{r / peak:.3f}", r / peak
        wstr = "" if work_amt is None else (f"{work_amt / 1e6:.2f} MB" if unit == "bytes" else
                                           f"{work_amt / 1e9:.3f} GFLOP")
        for (k, wg), v in sorted(ks.items(), key=lambda x: -x[1]["avg_us"]):
            rate, frac, _ = rate_of(v["avg_us"]) if len(ks) == 1 else ("", "", None)
            per = f"{v['period_us']:.2f}" if v["period_us"] is not None else "-"
            out.append(f"| {name} | `{k}` | {wg} | {v['launches']} ({v['timed']}) | {v['avg_us']:.2f} | "
                       f"{v['p10_us']:.2f} / {v['median_us']:.2f} / {v['p90_us']:.2f} | {per} | "
                       f"{wstr} | {rate} | {frac} |")
        rate, frac, fv = rate_of(tot)
        if len(ks) > 1:
            out.append(f"| {name} | step: the kernels above | | | {tot:.2f} | | | {wstr} | {rate} | {frac} |")
        table[name] = {"kernels": {k: v for (k, _), v in ks.items()}, "step_kernel_us": tot,
                       "work_per_step": work_amt, "work_unit": unit, "frac_of_peak": fv}
    with open(os.path.join(ROOT, "profiles", "kernel_times.json"), "w") as f:
        json.dump({"command": command, "kernel_hash": kernel_hash(), "steps": steps, "workloads": table}, f, indent=1)
    # one file per workload, named for its kernel and the workload: the rows above and,
    # where profiles/counters.json holds them for the current sources, its HBM bytes
    counters = {}
    cp = os.path.join(ROOT, "profiles", "counters.json")
    if os.path.exists(cp):
        counters = json.load(open(cp)).get("workloads", {})
    head = out[:10]
    for name, ks in runs:
        main_k = max(ks.items(), key=lambda x: x[1]["avg_us"])[0][0]
        stem = main_k.split("<")[0] + "_" + name
        rows = [r for r in out[10:] if r.startswith(f"| {name} |")]
        text = [f"# `{main_k}`: {name}", ""] + head + rows + [""]
        ent = counters.get(name)
        if ent and ent.get("kernel_hash") == kernel_hash(name) and "hbm_bytes_per_launch" in ent:
            text += ["HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a device-to-device "
                     "copy; profiles/counters.json):", "",
                     f"- read {ent['hbm_read_bytes_per_launch'] / 1e6:.2f} MB, written "
                     f"{ent['hbm_write_bytes_per_launch'] / 1e6:.2f} MB; Q+K+V {ent['qkv_bytes'] / 1e6:.2f} MB, "
                     f"O {ent['o_bytes'] / 1e6:.2f} MB (`{ent.get('kernel', '')}`)", ""]
            if len(ent.get("kernels", {})) > 1:
                text += [f"- `{k}`: read {v.get('hbm_read_bytes_per_launch', 0) / 1e6:.2f} MB, written "
                         f"{v.get('hbm_write_bytes_per_launch', 0) / 1e6:.2f} MB" for k, v in ent["kernels"].items()]
                text += [""]
            text += ["```"] + ent.get("commands", []) + ["```", ""]
        with open(os.path.join(ROOT, "profiles", stem + ".md"), "w") as f:
            f.write("\n".join(text))
    return "\n".join(out) + "\n"


def load_profiled(name: str):
    """The rocprofv3 figures for a workload (profiles/kernel_times.json), if taken on the current sources."""
    p = os.path.join(ROOT, "profiles", "kernel_times.json")
    if not os.path.exists(p):
        return None
    try:
        data = json.load(open(p))
    except Exception:
        return None
    if data.get("kernel_hash") != kernel_hash():
        return None
    return data.get("workloads", {}).get(name)


def ingest_counters(pmc_dir: str, calib_bytes: int):
    """counters.json from rocprofv3 --pmc passes: <pmc_dir>/<counter>_<workload>/.../*counter_collection.csv,
    with <counter>_copy holding a device-to-device copy of calib_bytes for the scale factor."""
    def per_dispatch(pattern, counter, kernel_filter=None):
        vals = {}
        for f in glob.glob(os.path.join(pmc_dir, pattern, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Counter_Name") != counter:
                    continue
                kn = r["Kernel_Name"]
                if kernel_filter and not kernel_filter(kn):
                    continue
                vals.setdefault((kn, r["Dispatch_Id"]), 0.0)
                vals[(kn, r["Dispatch_Id"])] += float(r["Counter_Value"])
        return vals
    out = {"note": "HBM bytes per launch of each workload's kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, "
                   "one rocprofv3 --pmc pass each) times the factor a device-to-device copy of known size gives "
                   "for the same counter", "calibration": {}, "workloads": {}}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        v = per_dispatch(f"{counter}_copy", counter, lambda k: "copy" in k.lower())
        big = max(v.values()) if v else 0.0
        out["calibration"][counter] = {"copy_bytes": calib_bytes, "counter_kib_per_copy": big,
                                       "factor": calib_bytes / (big * 1024.0) if big else None,
                                       "command": f"rocprofv3 --pmc {counter} -d gpurun_out/prof/pmc/{counter}_copy -o run "
                                                  f"-f csv -- python3 bench.py --profile-copy {calib_bytes >> 20} --steps 5"}
    for d in sorted(glob.glob(os.path.join(pmc_dir, "FETCH_SIZE_*"))):
        name = os.path.basename(d)[len("FETCH_SIZE_"):]
        if name == "copy" or name not in WORKLOADS:
            continue
        ent = {"kernel_hash": kernel_hash(name),
               "commands": [f"rocprofv3 --pmc {c} -d gpurun_out/prof/pmc/{c}_{name} -o run -f csv -- python3 bench.py "
                            f"--profile-run --workload {name} --steps 5" for c in ("FETCH_SIZE", "WRITE_SIZE")]}
        for counter, key in (("FETCH_SIZE", "read"), ("WRITE_SIZE", "write")):
            v = per_dispatch(f"{counter}_{name}", counter, lambda k: "sdpa_dev" in k)
            if not v:
                continue
            f = out["calibration"][counter]["factor"] or 1.0
            # every kernel of the route (a pre-pass, a combine) per launch; the totals below are
            # the dominant kernel's, the one with the most traffic
            for kk in sorted(set(k for k, _ in v)):
                xk = [x for (k2, _), x in v.items() if k2 == kk]
                ent.setdefault("kernels", {}).setdefault(_short(kk), {})[f"hbm_{key}_bytes_per_launch"] = \
                    sum(xk) / len(xk) * 1024.0 * f
            kern = max(set(k for k, _ in v), key=lambda kk: sum(x for (k2, _), x in v.items() if k2 == kk))
            xs = [x for (k, _), x in v.items() if k == kern]
            ent["kernel"] = _short(kern)
            ent[f"{key}_kib_per_dispatch"] = sum(xs) / len(xs)
            ent[f"hbm_{key}_bytes_per_launch"] = sum(xs) / len(xs) * 1024.0 * f
            ent["dispatches"] = len(xs)
        if "hbm_read_bytes_per_launch" in ent and "hbm_write_bytes_per_launch" in ent:
            ent["hbm_bytes_per_launch"] = ent["hbm_read_bytes_per_launch"] + ent["hbm_write_bytes_per_launch"]
            c = make_case(name)
            ent["algorithmic_per_launch"], ent["algorithmic_unit"] = work(c)
            qkv = sum(t.numel() * t.element_size() for t in (c.q, c.k, c.v))
            ent["qkv_bytes"] = qkv
            ent["o_bytes"] = c.q.shape[0] * c.q.shape[1] * c.q.shape[2] * c.v.shape[3] * c.q.element_size()
        out["workloads"][name] = ent
    return out


SQ_PASSES = (  # two rocprofv3 --pmc passes (8 SQ counters and GRBM_GUI_ACTIVE each)
    ("p1", "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_VALU_MFMA_BUSY_CYCLES "
           "SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_INST_LDS SQ_WAIT_ANY GRBM_GUI_ACTIVE"),
    ("p2", "SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_VALU_TRANS_F32 "
           "SQ_LDS_BANK_CONFLICT SQ_INST_LEVEL_LDS SQ_INSTS_LDS GRBM_GUI_ACTIVE"),
    ("p3", "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE"),
)
MOPS_FLOPS = 512  # flops per unit of SQ_INSTS_VALU_MFMA_MOPS_* (checked against the instruction mix)
SQ_WORKLOADS = ("prefill-d72-none", "prefill-d72-causal", "prefill-d72-boolean", "prefill-d512-causal",
                "prefill-d256-sliding-w1024")


def ingest_sq(pmc_dir: str) -> str:
    """Markdown table of SQ-counter figures for the prefill kernels, from <pmc_dir>/<W>_kt (kernel
    trace), <W>_p1 and <W>_p2 (the SQ_PASSES) of `bench.py --profile-run --workload <W> --steps 3`."""
    def files(sub, suffix):
        return glob.glob(os.path.join(pmc_dir, sub, "**", f"*{suffix}.csv"), recursive=True)

    rows = ["| workload | kernel | µs | clock GHz | MFMA busy | co-exec | VALU/MFMA | exp/MFMA | LDS/MFMA | "
            "LDS bank-conflict cycles | waiting / ready / issuing | matrix flops issued (counted) / algorithmic |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for w in SQ_WORKLOADS:
        kt = files(f"{w}_kt", "kernel_trace")
        if not kt:
            continue
        durs = {}
        for r in csv.DictReader(open(kt[0])):
            if "prefill" in r["Kernel_Name"]:
                durs.setdefault(_short(r["Kernel_Name"]), []).append(
                    (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
        if not durs:
            continue
        kern = max(durs, key=lambda k: sum(durs[k]))
        us = sum(durs[kern]) / len(durs[kern])
        c = {}
        for sub, _ in SQ_PASSES:
            for f in files(f"{w}_{sub}", "counter_collection"):
                per = {}
                for r in csv.DictReader(open(f)):
                    if _short(r["Kernel_Name"]) != kern:
                        continue
                    key = (r["Dispatch_Id"], r["Counter_Name"])
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
                names = set(n for _, n in per)
                for n in names:
                    vals = [v for (d, nn), v in per.items() if nn == n]
                    c[n if n != "GRBM_GUI_ACTIVE" else f"GRBM_{sub}"] = sum(vals) / len(vals)
        need = ("GRBM_p1", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
                "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY",
                "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY")
        if any(n not in c for n in need):
            continue
        cyc = c["GRBM_p1"] / 8.0  # GRBM_GUI_ACTIVE counts on every XCD
        mf = c["SQ_INSTS_MFMA"]
        wc = c["SQ_WAVE_CYCLES"]
        mops = c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        alg, _ = work(make_case(w))
        issued = (f"{mops * MOPS_FLOPS / 1e9:.1f} GFLOP / {alg / 1e9:.1f} GFLOP = {mops * MOPS_FLOPS / alg:.3f}"
                  if mops else "")
        rows.append(
            f"| {w} | `{kern}` | {us:.1f} | {cyc / (us * 1e3):.2f} | {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024):.1%} | "
            f"{c['SQ_VALU_MFMA_COEXEC_CYCLES'] / c['SQ_VALU_MFMA_BUSY_CYCLES']:.1%} | "
            f"{(c['SQ_INSTS_VALU'] - mf) / mf:.2f} | {c['SQ_INSTS_VALU_TRANS_F32'] / mf:.2f} | "
            f"{c['SQ_INSTS_LDS'] / mf:.2f} | {c['SQ_LDS_BANK_CONFLICT']:.3g} | "
            f"{c['SQ_WAIT_ANY'] / wc:.0%} / {c['SQ_WAIT_INST_ANY'] / wc:.0%} / {c['SQ_ACTIVE_INST_ANY'] / wc:.0%} | "
            f"{issued} |")
    return "\n".join(rows) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=PRIMARY, choices=sorted(WORKLOADS))
    ap.add_argument("--no-secondary", action="store_true", help="skip the other configurations")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=3.0, help="oracle budget per workload")
    ap.add_argument("--eager", action="store_true", help="also time eager (host-launched) steps")
    ap.add_argument("--profile-run", action="store_true",
                    help="only run --steps eager calls of --workload (for rocprofv3), print nothing else")
    ap.add_argument("--profile-copy", type=int, default=0, metavar="MIB",
                    help="only run --steps device-to-device copies of MIB MiB (calibrates rocprofv3 byte counters)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("CSV", "COMMAND"),
                    help="print a markdown summary of a rocprofv3 kernel trace (no GPU needed)")
    ap.add_argument("--timeline", action="store_true",
                    help="in-kernel timeline of --workload's single-launch decode (needs libsdpa_trace.so)")
    ap.add_argument("--ingest-sq", metavar="DIR",
                    help="print the SQ-counter table of the prefill kernels from rocprofv3 output (no GPU needed)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("DIR", "COPY_MIB"),
                    help="write profiles/counters.json from rocprofv3 --pmc output (no GPU needed)")
    a = ap.parse_args()

    if a.summarize_trace:
        print(summarize_trace(a.summarize_trace[0], a.summarize_trace[1], a.steps if a.steps != 200 else 20))
        return
    if a.ingest_sq:
        print(ingest_sq(a.ingest_sq), end="")
        return
    if a.ingest_counters:
        res = ingest_counters(a.ingest_counters[0], int(a.ingest_counters[1]) << 20)
        with open(os.path.join(ROOT, "profiles", "counters.json"), "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res, indent=1))
        return

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "one GPU only: a multi-GPU run (sharding by kv head) is not implemented",
                          "n_gpus": a.gpus}))
        sys.exit(2)

    import torch
    import scaled_dot_product_sdpa_amd as sdpa
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    if a.timeline:
        from scaled_dot_product_sdpa_amd import _lib
        if not os.path.exists(TRACE_LIB):
            raise SystemExit(f"{TRACE_LIB} not built: {TRACE_BUILD}")
        _lib.load(TRACE_LIB)
        cmd = "python3 bench.py --timeline" + (f" --workload {a.workload}" if a.workload != PRIMARY else "")
        print(timeline(a.workload, a.steps if a.steps != 200 else 50, 5, cmd), flush=True)
        return
    sdpa.load()

    if a.profile_copy:
        n = a.profile_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] profile copy: {a.steps} x {n} bytes", flush=True)
        return

    if a.profile_run:
        c = make_case(a.workload)
        import sdpa_inputs as si
        q, k, v, m = si.to_device(c)
        d = c.dims
        ws = torch.zeros(max(32768, sdpa.workspace_size(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"],
                                                       d["n_kv_heads"], d["head_dim"], q.dtype,
                                                       v_head_dim=c.v.shape[3])),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty(q.shape[:3] + (c.v.shape[3],), dtype=q.dtype, device="cuda")
        for _ in range(a.steps):
            sdpa.forward(q, k, v, scale=c.scale, mask=m, mask_kind=c.mask_kind, out=out, workspace=ws,
                         window=c.meta.get("window"))
        torch.cuda.synchronize()
        print(f"[bench] profile run: {a.steps} x {a.workload}", flush=True)
        return

    t_start = time.time()
    print(f"[bench] measuring {a.workload}", file=sys.stderr, flush=True)
    prim = measure(a.workload, a.steps, a.warmup, a.eager)
    results = {a.workload: prim}
    if not a.no_secondary:
        for name in WORKLOADS:
            if name == a.workload:
                continue
            st = a.steps if WORKLOADS[name]["kind"] in ("decode", "tiny", "decode_dv") else max(5, min(a.steps, 20))
            print(f"[bench] measuring {name}", file=sys.stderr, flush=True)
            results[name] = measure(name, st, max(2, min(a.warmup, 5)), a.eager)
    print("[bench] streaming-read ceiling", file=sys.stderr, flush=True)
    ceil = ceiling(int(prim["roofline"]["work_per_launch"]), a.steps) if prim["unit"] == "GB/s" else None

    cpu, cpus = None, {}
    if not a.no_cpu:
        import concurrent.futures as cf
        import multiprocessing as mp
        cores = min(len(os.sched_getaffinity(0)), MAX_POOL)
        names = [n for n in CPU_WORKLOADS if n in results] or [a.workload]
        if a.workload not in names:
            names.insert(0, a.workload)
        with cf.ProcessPoolExecutor(cores, mp_context=mp.get_context("spawn")) as pool:
            for n in names:
                print(f"[bench] oracle CPU baseline {n}", file=sys.stderr, flush=True)
                cpus[n] = cpu_baseline(n, a.cpu_seconds, pool, cores)
        cpu = cpus[a.workload]

    def entry(r):
        return {k: r[k] for k in ("value", "unit", "ms_per_step", "eager_ms_per_step", "route", "roofline")}

    line = {
        "metric": METRIC, "value": prim["value"], "unit": prim["unit"], "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": prim["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": prim["config"]["dtype"], "data": "synthetic (seeded, see sdpa_inputs.py)",
        "config": prim["config"], "eager_ms_per_step": prim["eager_ms_per_step"],
        "timing": "HIP graph of K steps: one untimed replay, then one replay timed with HIP events, queued "
                  "behind an untimed spin kernel so that its submission is not inside the timed region",
        "cold_cache_replicas": prim["replicas"], "route": prim["route"], "roofline": prim["roofline"],
        "prefill": {n: entry(results[n]) for n in PREFILL if n in results},
        "ceiling": ceil, "cpu_baseline": cpu,
        "cpu_baselines": cpus,
        "secondary": {n: entry(r) for n, r in results.items() if n != a.workload and n not in PREFILL},
        "kernel_hash": kernel_hash(a.workload), "wall_s": round(time.time() - t_start, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
