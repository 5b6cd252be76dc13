#!/usr/bin/env python3
"""Benchmark of the fused attention hot path on one MI355X; prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one sdpa_forward call (every kernel of the path) on one batch of
seeded synthetic input already resident in HBM.  The headline workload is the
bf16 grouped-query decode with head dim 256 (B=1, qL=1, Hq=32, Hkv=8,
Lk=4096, additive [1,1,1,Lk] mask): value = K+V bytes per step / step time.
Decode steps rotate over enough K/V replicas (> 2 x the 256 MB Infinity
Cache) that every step reads cold HBM.  K steps are captured in one HIP
graph and replayed (the host launch cost of the Python binding would
otherwise dominate a ~10 us step); the eager per-step time is reported too.

roofline: the dominant kernel's algorithmic work per launch / its average
duration, timed with HIP events the library records around each launch on
the launch stream (sdpa_timing_start/stop); traffic from rocprofv3 counters
(profiles/counters.json) when they were taken on the current kernel sources.
cpu_baseline: the float64 oracle on the host, on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SDPA prefill TFLOP/s + decode KV GB/s, each as % of MI355X roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 matrix
COLD_BYTES = 600 << 20         # K/V replicas per decode run: > 2 x 256 MB Infinity Cache

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


# kernel sources each workload's kernels are built from (counters taken on
# other sources are stale)
KERNEL_SOURCES = {
    "decode": ["attn_common.h", "decode_kernel.h", "attn_kernel.h", "launch.h", "inst_template.hip.in"],
    "prefill72": ["attn_common.h", "prefill_kernel.h", "launch.h", "inst_template.hip.in"],
    "prefill512": ["attn_common.h", "prefill_sd_kernel.h", "launch.h", "inst_template.hip.in"],
    "sliding": ["attn_common.h", "prefill_sd_kernel.h", "decode_kernel.h", "attn_kernel.h", "launch.h",
                "inst_template.hip.in"],
    "decode_dv": ["attn_common.h", "decode_kernel.h", "attn_kernel.h", "launch.h", "inst_pair_template.hip.in"],
    "tiny": ["attn_common.h", "attn_kernel.h", "tile_configs.h", "launch.h", "inst_template.hip.in"],
}


def kernel_hash(name: str = PRIMARY) -> str:
    """Hash of the sources of `name`'s kernels."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[WORKLOADS[name]["kind"]]:
        h.update(open(os.path.join(ROOT, "scaled_dot_product_sdpa_amd", "csrc", f), "rb").read())
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


def to_device_replicas(c, n):
    import torch
    import sdpa_inputs as si
    reps = [si.to_device(c) for _ in range(n)]
    torch.cuda.synchronize()
    return reps


def measure(name: str, steps: int, warmup: int) -> dict:
    import torch
    import scaled_dot_product_sdpa_amd as sdpa

    c = make_case(name)
    amount, unit = work(c)
    decode = unit == "bytes"
    kv_bytes = 2 * c.k.numel() * c.k.element_size()
    nrep = max(2, -(-COLD_BYTES // kv_bytes)) if decode else 1
    reps = to_device_replicas(c, nrep)
    q0 = reps[0][0]
    out = torch.empty(q0.shape[:3] + (c.v.shape[3],), dtype=q0.dtype, device="cuda")
    d = c.dims
    ws_bytes = sdpa.workspace_size(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"],
                                   d["head_dim"], q0.dtype, v_head_dim=c.v.shape[3])
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")

    def step(i):
        q, k, v, m = reps[i % nrep]
        sdpa.forward(q, k, v, scale=c.scale, mask=m, mask_kind=c.mask_kind, out=out, workspace=ws,
                     window=c.meta.get("window"))

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()

    # eager steps (host launch cost included)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps

    # per-kernel times from events recorded by the library on the launch stream
    with sdpa.kernel_timing(steps) as kt:
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    k_ms = sorted(t[0] for t in kt.ms)
    c_ms = [t[1] for t in kt.ms]
    kernel_ms = sum(k_ms) / len(k_ms)
    combine_ms = sum(c_ms) / len(c_ms)

    # graph: K steps captured once, replayed (warm-up replay, then the timed one)
    graph_ms = None
    try:
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
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / steps
    except Exception as ex:  # graph capture unavailable: report eager only
        print(f"[bench] graph capture failed: {ex}", file=sys.stderr)
    ms = graph_ms if graph_ms is not None else eager_ms
    route = sdpa.describe_route(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"],
                                d["head_dim"], q0.dtype, c.mask_kind, v_head_dim=c.v.shape[3])
    res = dict(config=describe(name, c), route=route, ms_per_step=ms, eager_ms_per_step=eager_ms,
               graph_ms_per_step=graph_ms, kernel_ms=kernel_ms, kernel_ms_p10=k_ms[len(k_ms) // 10],
               kernel_ms_p90=k_ms[(9 * len(k_ms)) // 10], combine_ms=combine_ms, replicas=nrep,
               work=amount, work_unit=unit)
    if decode:
        res.update(value=amount / (ms * 1e-3) / 1e9, unit="GB/s",
                   kernel_rate=amount / (kernel_ms * 1e-3) / 1e9, peak=HBM_PEAK_GBS, bound="hbm", rate_unit="GB/s")
    else:
        peak = FP32_PEAK_TFLOPS if str(q0.dtype) == "torch.float32" else BF16_PEAK_TFLOPS
        res.update(value=amount / (ms * 1e-3) / 1e12, unit="TFLOP/s",
                   kernel_rate=amount / (kernel_ms * 1e-3) / 1e12, peak=peak, bound="mfma", rate_unit="TFLOP/s")
    res["frac"] = res["kernel_rate"] / res["peak"]
    del reps
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name: str, budget_s: float) -> dict:
    """The float64 oracle, as it is, on the host; a bounded sample of the same workload."""
    import numpy as np
    import oracle
    c = make_case(name)
    amount, unit = work(c)
    mask = None
    if c.mask_kind == "sliding":
        mask = c.meta["window"]
    elif c.mask is not None:
        mask = c.mask.double().numpy() if c.mask_kind == "additive" else c.mask.numpy()
    q, k, v = (t.double().numpy() for t in (c.q, c.k, c.v))
    Lq = q.shape[2]
    rows = None
    frac = 1.0
    if Lq > 64:  # prefill: a sample of query rows, scaled
        n = 64
        rows = np.linspace(0, Lq - 1, n).astype(np.int64)
        frac = n / Lq
    t0 = time.perf_counter()
    calls = 0
    while True:
        oracle.sdpa(q, k, v, np.float32(c.scale), c.mask_kind, mask, q_rows=rows)
        calls += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = (time.perf_counter() - t0) / calls
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    # the oracle computes every (row, key) pair: scale the sampled rows' share of the work
    per_call = amount * frac
    if unit == "bytes":
        val, u = per_call / dt / 1e9, "GB/s"
    else:
        val, u = per_call / dt / 1e12, "TFLOP/s"
    sample = (f"{name}: full call ({calls} calls in {dt * calls:.1f}s)" if rows is None else
              f"{name}: {len(rows)} of {Lq} query rows per call, work scaled by {frac:.4f} ({calls} calls)")
    return {"value": val, "unit": u, "cores": cores, "kind": "oracle", "sample": sample,
            "seconds_per_call": dt}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=PRIMARY, choices=sorted(WORKLOADS))
    ap.add_argument("--no-secondary", action="store_true", help="skip the other configurations")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile-run", action="store_true",
                    help="only run --steps eager calls of --workload (for rocprofv3), print nothing else")
    ap.add_argument("--profile-copy", type=int, default=0, metavar="MIB",
                    help="only run --steps device-to-device copies of MIB MiB (calibrates rocprofv3 byte counters)")
    a = ap.parse_args()

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
        ws = torch.empty(max(256, sdpa.workspace_size(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"],
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
    prim = measure(a.workload, a.steps, a.warmup)
    secondary = {}
    if not a.no_secondary:
        for name in WORKLOADS:
            if name == a.workload:
                continue
            st = a.steps if WORKLOADS[name]["kind"] in ("decode", "tiny") else max(5, min(a.steps, 20))
            print(f"[bench] measuring {name}", file=sys.stderr, flush=True)
            r = measure(name, st, max(2, min(a.warmup, 5)))
            secondary[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "eager_ms_per_step",
                                                 "kernel_ms", "combine_ms", "kernel_rate", "rate_unit",
                                                 "peak", "frac", "route")}
            secondary[name]["traffic"] = load_traffic(name)
    cpu = None
    if not a.no_cpu:
        print("[bench] oracle CPU baseline", file=sys.stderr, flush=True)
        cpu = cpu_baseline(a.workload, a.cpu_seconds)

    roof = {"bound": prim["bound"], "achieved": prim["kernel_rate"], "peak": prim["peak"],
            "unit": prim["rate_unit"], "frac": prim["frac"], "traffic": load_traffic(a.workload),
            "kernel_ms": prim["kernel_ms"], "kernel_ms_p10": prim["kernel_ms_p10"],
            "kernel_ms_p90": prim["kernel_ms_p90"], "combine_ms": prim["combine_ms"],
            "work_per_launch": prim["work"], "work_unit": prim["work_unit"]}
    line = {
        "metric": METRIC, "value": prim["value"], "unit": prim["unit"], "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": prim["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": prim["config"]["dtype"], "data": "synthetic (seeded, see sdpa_inputs.py)",
        "config": prim["config"], "eager_ms_per_step": prim["eager_ms_per_step"],
        "timing": "HIP graph of K steps, replayed" if prim["graph_ms_per_step"] else "eager",
        "cold_cache_replicas": prim["replicas"], "route": prim["route"], "roofline": roof,
        "cpu_baseline": cpu, "secondary": secondary, "kernel_hash": kernel_hash(a.workload),
        "wall_s": round(time.time() - t_start, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
