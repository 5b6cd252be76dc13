"""Build libsdpa.so for gfx950 with hipcc (in-tree, no JIT cache).

    python -m scaled_dot_product_sdpa_amd.build [--jobs N]

Every call recompiles.  The per-head-dim instantiation units are generated
from csrc/inst_template.hip.in into _build/ and compiled in parallel.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsdpa.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed-fp32 VALU forms are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
    "-Wno-unused-command-line-argument",
]


def head_dims() -> list[int]:
    src = open(os.path.join(CSRC, "launch.h")).read()
    m = re.search(r"#define SDPA_HEAD_DIMS\(X\)(.*)", src)
    return [int(x) for x in re.findall(r"X\((\d+)\)", m.group(1))]


def head_dim_pairs() -> list[tuple[int, int]]:
    src = open(os.path.join(CSRC, "launch.h")).read()
    m = re.search(r"#define SDPA_HEAD_DIM_PAIRS\(X\)(.*)", src)
    return [(int(a), int(b)) for a, b in re.findall(r"X\((\d+),\s*(\d+)\)", m.group(1))]


def _run(cmd):
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    return time.time() - t, err


def build(jobs: int | None = None, verbose: bool = True, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile every unit and link `out`; `defines` are extra -D flags (tuning experiments)."""
    os.makedirs(build_dir, exist_ok=True)
    tmpl = open(os.path.join(CSRC, "inst_template.hip.in")).read()
    ptmpl = open(os.path.join(CSRC, "inst_pair_template.hip.in")).read()
    generated = [(f"inst_d{d}.hip", tmpl.replace("@D@", str(d))) for d in head_dims()]
    generated += [(f"inst_q{a}_v{b}.hip", ptmpl.replace("@DQ@", str(a)).replace("@DV@", str(b)))
                  for a, b in head_dim_pairs()]
    units = []
    for name, text in generated:
        path = os.path.join(build_dir, name)
        if not os.path.exists(path) or open(path).read() != text:
            with open(path, "w") as f:
                f.write(text)
        units.append(path)
    units.append(os.path.join(CSRC, "sdpa_host.cpp"))
    objs = []
    cmds = []
    for u in units:
        o = os.path.join(build_dir, os.path.basename(u) + ".o")
        objs.append(o)
        lang = ["-x", "hip"] if u.endswith(".cpp") else []
        cmds.append([HIPCC] + COMMON + [f"-D{x}" for x in defines] + lang + ["-c", u, "-o", o])
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    t0 = time.time()
    with cf.ThreadPoolExecutor(jobs) as ex:
        for cmd, (dt, err) in zip(cmds, ex.map(_run, cmds)):
            if verbose:
                print(f"[build] {os.path.basename(cmd[-3])}: {dt:.1f}s", flush=True)
            if err.strip() and verbose:
                print(err, file=sys.stderr)
    tmp = out + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
    # a kernel whose host stub was not emitted shows up as an undefined symbol
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-D", "--undefined-only", tmp], capture_output=True, text=True).stdout
        bad = [l.split()[-1] for l in und.splitlines() if "sdpa_dev" in l or "sdpa_host" in l]
        if bad:
            os.remove(tmp)
            raise RuntimeError(f"build failed: {len(bad)} undefined library symbols, e.g. {bad[0]}")
    os.replace(tmp, out)
    if verbose:
        print(f"[build] {out} ({time.time() - t0:.1f}s)", flush=True)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("-D", dest="defines", action="append", default=[], help="extra preprocessor define")
    ap.add_argument("--out", default=LIB)
    ap.add_argument("--build-dir", default=BUILD)
    a = ap.parse_args()
    build(a.jobs, defines=a.defines, out=os.path.abspath(a.out), build_dir=os.path.abspath(a.build_dir))
