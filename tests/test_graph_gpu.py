"""HIP graph capture of the forward call: every replay equals the eager call.

The benchmark times its steps as replays of a captured graph, so the captured
launches must compute what an eager call computes.  A captured call records
the same kernel launches, with the caller's pointers: the split decode's
partials and the combine go through the caller's workspace, and nothing in
the call records a memset.  Each case below

  1. runs the call eagerly (the result the parity tests check against the
     float64 oracle);
  2. captures one call into a graph, on a side stream, with an explicit
     workspace that eager calls share;
  3. replays it several times; between replays the workspace's partial
     results are overwritten with 0xff bytes (NaN patterns in float32) and an
     unrelated eager call of another kernel family runs on the same
     workspace, with a synchronisation before each replay.  The workspace's
     leading arrival words are left as the calls leave them (zero).  Every
     replay must equal the eager result bit for bit (the kernels are
     deterministic: fixed split order; the only atomics count arrivals);
  4. refills the captured inputs in place with new data and replays once
     more: the replay must equal an eager call on the new data.
"""
import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs as si

pytestmark = pytest.mark.gpu

COUNTER_BYTES = 32768  # leading arrival words of a decode workspace (zero before and after every call)

# name, make_case arguments, route kind and a fragment of the route string
CASES = [
    ("decode-fused-splits", dict(B=1, Hq=32, Hkv=8, Lq=1, Lk=4096, D=256, mask_kind="additive"),
     "vector-fused", "splits=32"),
    ("decode-d512-splits-combine", dict(B=1, Hq=32, Hkv=4, Lq=1, Lk=4096, D=512, mask_kind="additive"),
     "vector ", "splits="),
    ("decode-splits-combine", dict(B=1, Hq=12, Hkv=3, Lq=2, Lk=3000, D=128, mask_kind="additive"),
     "vector ", "splits="),
    ("decode-one-split", dict(B=64, Hq=16, Hkv=8, Lq=1, Lk=256, D=128), "vector-fused", "splits=1 "),
    ("decode-d512-causal-lq4", dict(B=2, Hq=8, Hkv=2, Lq=4, Lk=1000, D=512, mask_kind="causal"), "vector", ""),
    ("decode-qk192-v128", dict(B=1, Hq=16, Hkv=4, Lq=1, Lk=900, D=192, dv=128, mask_kind="additive"),
     "vector", ""),
    ("decode-f32", dict(B=2, Hq=4, Hkv=4, Lq=3, Lk=82, D=64, dtype="f32"), "vector", ""),
    ("prefill-d72-causal-pairs", dict(B=1, Hq=16, Hkv=16, Lq=4096, Lk=4096, D=72, mask_kind="causal",
                                      layout="blhd"), "full", "causal-pairs"),
    # boolean masks: the lane-word pre-pass and the kernel both captured; the words sit in the
    # clobbered part of the workspace and are rebuilt by every replay
    ("prefill-d128-boolean", dict(B=1, Hq=4, Hkv=2, Lq=300, Lk=333, D=128, mask_kind="boolean",
                                  mask_shape="qk"), "full", "lane-words+prepass"),
    ("prefill-d72-boolean-aligned", dict(B=1, Hq=8, Hkv=2, Lq=256, Lk=320, D=72, mask_kind="boolean",
                                         mask_shape="full"), "full", "lane-words+prepass"),
    # (a launch with dynamic LDS padding: mask tensors below D = 128)
    ("prefill-d72-additive", dict(B=1, Hq=4, Hkv=2, Lq=300, Lk=332, D=72, mask_kind="additive",
                                  mask_shape="qk"), "full", ""),
    ("prefill-d256-sliding", dict(B=1, Hq=4, Hkv=2, Lq=500, Lk=500, D=256, mask_kind="sliding", window=100),
     "full", ""),
    ("prefill-d512-causal", dict(B=1, Hq=8, Hkv=1, Lq=400, Lk=400, D=512, mask_kind="causal"), "full", ""),
    ("prefill-f32", dict(B=2, Hq=4, Hkv=4, Lq=82, Lk=82, D=64, dtype="f32", layout="blhd"), "full", ""),
]


def _make(kw, seed):
    kw = dict(kw)
    B, Hq, Hkv, Lq, Lk, D = (kw.pop(x) for x in ("B", "Hq", "Hkv", "Lq", "Lk", "D"))
    return si.make_case(B, Hq, Hkv, Lq, Lk, D, seed=seed, **kw)


class _Call:
    """One forward call on fixed device buffers (the captured inputs)."""

    def __init__(self, sdpa, case, rope=None):
        self.sdpa, self.case, self.rope = sdpa, case, rope
        self.q, self.k, self.v, self.mask = si.to_device(case)
        self.kw = dict(scale=case.scale, mask=self.mask, mask_kind=case.mask_kind, rope=rope)
        if case.mask_kind == "sliding":
            self.kw["window"] = case.meta["window"]
        B, Hq, Lq, _ = self.q.shape
        Dv = self.v.shape[3]
        self.out = torch.empty((B, Hq, Lq, Dv), dtype=self.q.dtype, device="cuda")

    def __call__(self, out=None, workspace=None):
        return self.sdpa.forward(self.q, self.k, self.v, out=out, workspace=workspace, **self.kw)

    def refill(self, case):
        """Copy another case's values into the captured buffers (same shapes and strides)."""
        q, k, v, mask = si.to_device(case)
        for dst, src in ((self.q, q), (self.k, k), (self.v, v), (self.mask, mask)):
            if dst is not None:
                dst.copy_(src)


def _check_graph(sdpa, call, refill_case, name):
    dims = call.case.dims
    nbytes = sdpa.workspace_size(dims["batch"], dims["q_len"], dims["kv_len"], dims["n_q_heads"],
                                 dims["n_kv_heads"], dims["head_dim"], call.q.dtype,
                                 v_head_dim=call.v.shape[3])
    ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device="cuda")
    eager = call(workspace=ws).clone()
    torch.cuda.synchronize()

    # an unrelated call of another family that shares the workspace between replays
    other = _Call(sdpa, si.make_case(1, 8, 2, 1 if dims["q_len"] > 8 else 96, 700, 128, seed=99,
                                     mask_kind="additive"))
    assert other.sdpa.workspace_size(1, other.q.shape[2], 700, 8, 2, 128, other.q.dtype) <= ws.numel()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call(out=call.out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for rep in range(4):
        ws[COUNTER_BYTES:].fill_(0xFF)  # partial results need no initialisation; arrival words stay as left
        other(workspace=ws)
        call.out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(call.out, eager), f"{name}: replay {rep} differs from the eager call"

    call.refill(refill_case)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    fresh = call(workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(call.out, fresh), f"{name}: replay on refilled inputs differs from the eager call"
    assert not torch.equal(fresh, eager), f"{name}: refilled inputs gave the old output"
    return eager


@pytest.mark.parametrize("name,kw,kind,frag", CASES, ids=[c[0] for c in CASES])
def test_graph_replay_equals_eager(gpu_lib, name, kw, kind, frag):
    case = _make(kw, seed=11)
    d = case.dims
    route = gpu_lib.describe_route(d["batch"], d["q_len"], d["kv_len"], d["n_q_heads"], d["n_kv_heads"],
                                   d["head_dim"], case.q.dtype, case.mask_kind, v_head_dim=case.v.shape[3])
    assert route.startswith(kind) and frag in route, route
    eager = _check_graph(gpu_lib, _Call(gpu_lib, case), _make(kw, seed=12), name)
    # the eager result itself against the oracle on a few rows (parity proper lives elsewhere)
    rows = sorted({0, d["q_len"] // 2, d["q_len"] - 1})
    mask = case.meta["window"] if case.mask_kind == "sliding" else (
        None if case.mask is None else
        (case.mask.double().numpy() if case.mask_kind == "additive" else case.mask.numpy()))
    ref = oracle.sdpa(case.q.double().numpy(), case.k.double().numpy(), case.v.double().numpy(),
                      np.float32(case.scale), case.mask_kind, mask, q_rows=rows)
    got = eager[:, :, rows].double().cpu().numpy()
    tol = 2e-5 if case.q.dtype == torch.float32 else 2e-2
    assert np.abs(got - ref).max() <= tol, f"{name}: eager result off the oracle"


@pytest.mark.parametrize("Lq,D,R", [(1, 128, 64), (150, 128, 64), (1, 256, 256), (150, 256, 256)])
def test_graph_replay_fused_rope(gpu_lib, Lq, D, R):
    """R = 64: the rotation inside the kernels; R = 256: a rotation pass of Q into the output first."""
    Lk = 400
    case = si.make_case(1, 8, 2, Lq, Lk, D, seed=13, mask_kind="causal")
    c, s = oracle.rope_tables(Lk + 8, R)
    rope = (torch.from_numpy(c.astype(np.float32)).cuda(), torch.from_numpy(s.astype(np.float32)).cuda(), R)
    _check_graph(gpu_lib, _Call(gpu_lib, case, rope=rope), si.make_case(1, 8, 2, Lq, Lk, D, seed=14,
                                                                       mask_kind="causal"), f"rope Lq={Lq}")
