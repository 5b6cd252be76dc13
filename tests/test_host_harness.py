"""The host library's planner and argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no kernel is launched).

tests/host_harness.cpp compiles csrc/sdpa_host.cpp together with recording
stubs in place of the kernel tables, then sweeps decode shapes, mask kinds and
sliding windows: every call must fit the workspace sdpa_workspace_size()
reports (and one byte less must be refused), the single-launch decode
geometry must be the planned one, overlapping buffers must be refused, and
concurrent host queries must agree.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_harness_under_sanitizers(tmp_path):
    exe = tmp_path / "host_harness"
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           # sanitizers on the host code only
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'scaled_dot_product_sdpa_amd', 'csrc')}",
           os.path.join(ROOT, "tests", "host_harness.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="-1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "0 failed" in r.stdout, r.stdout
