"""Host-side logic of bench.py (no GPU): the algorithmic work it divides by, and how it cuts a
rocprofv3 kernel trace into workloads.

The work per call is the spec definition: prefill 4 * B * Hq * Lq * Lk * D flops (halved
for a causal mask), decode the K and V bytes, 2 * B * Hkv * Lk * D * element size.  The numbers
below are written out from the configurations' sizes, not computed by bench.py's formula.
"""
import csv
import os

import pytest

import bench


def test_algorithmic_work_of_the_bench_workloads():
    expect = {
        "decode-d256-lk4096": (2 * 8 * 4096 * 256 * 2, "bytes"),          # 33 554 432
        "decode-d256-lk1024": (2 * 8 * 1024 * 256 * 2, "bytes"),
        "decode-d512-lk4096": (2 * 4 * 4096 * 512 * 2, "bytes"),
        "prefill-d72-none": (4 * 16 * 8192 * 8192 * 72, "flops"),         # 309.2 GFLOP
        "prefill-d72-boolean": (4 * 16 * 8192 * 8192 * 72, "flops"),
        "prefill-d72-causal": (2 * 16 * 8192 * 8192 * 72, "flops"),
        "prefill-d512-causal": (2 * 32 * 4096 * 4096 * 512, "flops"),
    }
    for name, (amount, unit) in expect.items():
        c = bench.make_case(name)
        got, gunit = bench.work(c)
        assert gunit == unit, name
        assert got == float(amount), name


def _write_trace(path, rows):
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z",
            "Workgroup_Size_X"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_trace_is_cut_at_markers_not_at_the_long_spin_before_a_timed_replay(tmp_path):
    """Each workload opens with a marker spin of about a microsecond; its timed replay is queued
    behind a spin of about a millisecond, which must not start a new workload."""
    kern = "void sdpa_dev::decode_fused_kernel<TBF16, DfCfg<TBF16, 256, 256, 8>, 1, false>(sdpa_dev::Params)"
    rows, t = [], 0

    def spin(ns):
        nonlocal t
        rows.append(("spin_kernel(long)", t, t + ns, 64, 1, 1, 64))
        t += ns + 1000

    def launches(n, dur_ns, period_ns):
        nonlocal t
        for _ in range(n):
            rows.append((kern, t, t + dur_ns, 256 * 512, 1, 1, 512))
            t += period_ns

    spin(1_000)                      # marker: first workload (the primary one)
    launches(25, 30_000, 40_000)     # warm-up and untimed replay, slower
    spin(1_000_000)                  # the cover spin before the timed replay
    launches(20, 11_000, 11_200)     # the timed replay
    spin(1_000)                      # marker: the next workload
    launches(25, 8_000, 8_200)
    path = os.path.join(tmp_path, "trace.csv")
    _write_trace(path, rows)
    runs = bench.trace_runs(path, 20)
    assert [name for name, _ in runs] == [bench.PRIMARY, "decode-d256-lk1024"]
    (k, st), = runs[0][1].items()
    assert st["launches"] == 45 and st["timed"] == 20
    assert st["avg_us"] == pytest.approx(11.0)
    assert st["period_us"] == pytest.approx(11.2)
    (k2, st2), = runs[1][1].items()
    assert st2["avg_us"] == pytest.approx(8.0)
