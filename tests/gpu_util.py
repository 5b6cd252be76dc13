"""Helpers shared by the GPU tests: device copies of seeded cases, oracle calls, tolerances."""
import numpy as np
import torch

import oracle
import sdpa_inputs as si

# Tolerances against the float64 oracle.
TOL = {"f32": dict(max_abs=2e-5, rel_l2=None), "f16": dict(max_abs=2e-2, rel_l2=1e-2),
       "bf16": dict(max_abs=2e-2, rel_l2=1e-2)}
DT_NAME = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}


to_device = si.to_device


def run_gpu(case: si.Case, **kw):
    import scaled_dot_product_sdpa_amd as sdpa
    q, k, v, mask = to_device(case)
    if case.mask_kind == "sliding":
        kw.setdefault("window", case.meta["window"])
    out = sdpa.forward(q, k, v, scale=case.scale, mask=mask, mask_kind=case.mask_kind, **kw)
    torch.cuda.synchronize()
    return out


def oracle_out(case: si.Case, q_rows=None):
    mask = None
    if case.mask_kind == "sliding":
        mask = case.meta["window"]
    elif case.mask is not None:
        mask = case.mask.double().numpy() if case.mask_kind == "additive" else case.mask.numpy()
    return oracle.sdpa(case.q.double().numpy(), case.k.double().numpy(), case.v.double().numpy(),
                       np.float32(case.scale), case.mask_kind, mask, q_rows=q_rows)


def errors(got: torch.Tensor, ref: np.ndarray):
    g = got.double().cpu().numpy()
    d = g - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    nr = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / nr) if nr > 0 else float(np.linalg.norm(d))
    return max_abs, rel, bool(np.isfinite(g).all())


def assert_parity(got: torch.Tensor, ref: np.ndarray, dtype_name: str, what: str):
    max_abs, rel, finite = errors(got, ref)
    tol = TOL[dtype_name]
    msg = f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e} (tol {tol})"
    assert finite, msg + " non-finite output"
    assert max_abs <= tol["max_abs"], msg
    if tol["rel_l2"] is not None:
        assert rel <= tol["rel_l2"], msg
    return max_abs, rel
