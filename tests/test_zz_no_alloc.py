"""The allocation-free entry point, sdpa_forward_noalloc, against sdpa_forward_ex.

Both run the same kernels with the same plan; the allocation-free call keeps
its split partial results and arrival counters in the library's static
device scratch instead of a caller's workspace.  Two calls in a row (the
second smaller, on a different route) must each equal the workspace call bit
for bit and match the oracle; a shape whose workspace exceeds the scratch is
refused before anything is launched.
"""
import numpy as np
import pytest
import torch

import sdpa_inputs as si
from gpu_util import assert_parity, oracle_out, to_device

pytestmark = pytest.mark.gpu

COUNTER_BYTES = 32768


def _both(sdpa, c):
    q, k, v, m = to_device(c)
    d = c.dims
    kw = dict(scale=c.scale, mask=m, mask_kind=c.mask_kind, window=c.meta.get("window"))
    n = sdpa.workspace_size(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"], d["head_dim"],
                            q.dtype, v_head_dim=c.v.shape[3])
    ws = torch.zeros(max(n, COUNTER_BYTES), dtype=torch.uint8, device="cuda")
    ref = sdpa.forward(q, k, v, workspace=ws, **kw)
    out = torch.full_like(ref, float("nan"))
    got = sdpa.forward(q, k, v, out=out, no_alloc=True, **kw)
    torch.cuda.synchronize()
    return got, ref


CASES = [
    # (name, make_case arguments, route fragment)
    ("decode single launch, 32 splits", dict(B=1, Hq=32, Hkv=8, Lq=1, Lk=4096, D=256, mask_kind="additive"),
     "vector-fused"),
    ("decode split + combine, smaller", dict(B=1, Hq=12, Hkv=3, Lq=2, Lk=700, D=128, mask_kind="causal"), "vector "),
    ("decode split + combine, head dim 512", dict(B=1, Hq=32, Hkv=4, Lq=1, Lk=2000, D=512, mask_kind="none"),
     "vector "),
    ("decode sliding, smaller", dict(B=2, Hq=16, Hkv=4, Lq=3, Lk=500, D=64, mask_kind="sliding", window=40),
     "vector-fused"),
    ("prefill (no scratch)", dict(B=1, Hq=4, Hkv=2, Lq=200, Lk=200, D=72, mask_kind="causal"), "full"),
    ("prefill boolean, lane words in the scratch", dict(B=1, Hq=4, Hkv=2, Lq=300, Lk=320, D=72,
                                                      mask_kind="boolean", mask_shape="qk"), "lane-words"),
    ("decode after it, smaller", dict(B=1, Hq=32, Hkv=8, Lq=1, Lk=1000, D=128, mask_kind="none"), "vector-fused"),
]


def _make(kw, seed):
    kw = dict(kw)
    B, Hq, Hkv, Lq, Lk, D = (kw.pop(x) for x in ("B", "Hq", "Hkv", "Lq", "Lk", "D"))
    return si.make_case(B, Hq, Hkv, Lq, Lk, D, seed=seed, **kw)


def test_noalloc_equals_workspace_call_on_consecutive_calls(gpu_lib):
    for i, (name, kw, frag) in enumerate(CASES):
        c = _make(kw, seed=50 + i)
        d = c.dims
        route = gpu_lib.describe_route(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"],
                                       d["head_dim"], c.q.dtype, c.mask_kind)
        assert frag in route, (name, route)
        got, ref = _both(gpu_lib, c)
        assert torch.equal(got, ref), f"{name}: the allocation-free call differs from the workspace call"
        assert_parity(got, oracle_out(c), "bf16", f"no-alloc {name}")


def test_noalloc_repeats_bitwise(gpu_lib):
    """The scratch's arrival counters are left zero: the same call twice gives the same bits."""
    c = _make(CASES[0][1], seed=60)
    q, k, v, m = to_device(c)
    outs = [gpu_lib.forward(q, k, v, scale=c.scale, mask=m, mask_kind=c.mask_kind, out=torch.empty_like(q),
                            no_alloc=True) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_noalloc_refuses_shapes_beyond_the_scratch(gpu_lib):
    import scaled_dot_product_sdpa_amd._lib as L
    cap = L.load().sdpa_noalloc_scratch_bytes()
    assert cap == 8 << 20
    # 64 query heads on one kv head, 8 rows each, D = 512: the split partials need far more than 8 MiB
    need = gpu_lib.workspace_size(1, 8, 32768, 64, 1, 512, torch.bfloat16)
    assert need > cap
    q = torch.zeros(1, 64, 8, 512, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 32768, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.SdpaError) as e:
        gpu_lib.forward(q, k, k, out=torch.empty_like(q), no_alloc=True)
    assert e.value.status == -3
