"""Rotary position embedding on the GPU against the float64 oracle.

Two paths: the standalone kernel (sdpa_rope: keys rotated once on their way
into a cache) and the rotation of Q fused into the attention kernels
(sdpa_forward_ex with a table: queries are never written back rotated).  The
cos / sin tables are the usual base-10000 ones, built by the oracle in float64
and rounded to float32 once; the oracle is handed the same float32 values.
"""
import numpy as np
import pytest
import torch

import oracle
import sdpa_inputs as si
from gpu_util import assert_parity

pytestmark = pytest.mark.gpu

# One rounding of a float32 result to the element type: relative error at most
# 2^-9 (bf16), 2^-12 (f16); the fp32 arithmetic itself adds a few ulp of fp32.
REL = {"f32": 2.0 ** -21, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def tables(n_pos, R, device="cuda"):
    c, s = oracle.rope_tables(n_pos, R)
    c32, s32 = c.astype(np.float32), s.astype(np.float32)
    return (torch.from_numpy(c32).to(device), torch.from_numpy(s32).to(device),
            c32.astype(np.float64), s32.astype(np.float64))


def rotate_ref(x: torch.Tensor, c64, s64, R, pos0):
    """Oracle rotation of a logical [B, H, L, D] tensor (any dtype), float64 out."""
    return oracle.rope(x.double().numpy(), c64, s64, R, pos0)


# --------------------------------------------------------------------------
# Standalone kernel: every dtype, full / partial / two-column rotation,
# out-of-place and in place, both layouts, a position offset.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["bhld", "blhd"])
@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("R", [128, 64, 2])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_rope_kernel_matches_oracle(gpu_lib, dtype, R, inplace, layout):
    B, H, L, D, pos0 = 2, 3, 37, 128, 11
    g = si.rng(R + (7 if inplace else 0))
    phys = (B, L, H, D) if layout == "blhd" else (B, H, L, D)
    x_host = torch.from_numpy(g.standard_normal(phys, dtype=np.float32)).to(si.DTYPES[dtype])
    x_log = x_host.transpose(1, 2) if layout == "blhd" else x_host
    cos, sin, c64, s64 = tables(pos0 + L + 3, R)
    ref = rotate_ref(x_log, c64, s64, R, pos0)
    x = x_host.cuda()
    y = gpu_lib.rope(x, cos, sin, R, pos0=pos0, out=x if inplace else None, layout=layout)
    torch.cuda.synchronize()
    got = (y.transpose(1, 2) if layout == "blhd" else y).double().cpu().numpy()
    err = np.abs(got - ref)
    bound = REL[dtype] * np.abs(ref) + 1e-6
    assert (err <= bound).all(), f"rope {dtype} R={R}: worst excess {(err - bound).max():.3e}"
    # columns past the rotated ones pass through bit for bit; out-of-place leaves x alone
    gl = y.transpose(1, 2) if layout == "blhd" else y
    assert torch.equal(gl[..., R:].cpu(), x_log[..., R:])
    if not inplace:
        assert torch.equal(x.cpu(), x_host)


# --------------------------------------------------------------------------
# Fused Q rotation: the 16-bit MFMA prefill kernels (D <= 128 and the wide
# 256 / 512 kernel), the decode kernel and the (192, 128) pairing, against
# softmax(scale * rope(Q) rope(K)^T + mask) V in float64.  K is rotated by
# the oracle and rounded to the input type, as a cache would hold it.
# --------------------------------------------------------------------------
def fused_case(B, Hq, Hkv, Lq, Lk, D, R, dtype, mask_kind, seed, q_pos0=None, dv=None, layout="bhld", window=None):
    c = si.make_case(B, Hq, Hkv, Lq, Lk, D, dtype=dtype, layout=layout, mask_kind=mask_kind, seed=seed,
                     mask_shape="qk", mask_p=0.2, dv=dv, window=window)
    pos0 = Lk - Lq if q_pos0 is None else q_pos0
    cos, sin, c64, s64 = tables(max(Lk, pos0 + Lq) + 5, R)
    k_rot = torch.from_numpy(rotate_ref(c.k, c64, s64, R, 0)).to(c.k.dtype)
    q_rot = rotate_ref(c.q, c64, s64, R, pos0)
    mask = None
    if mask_kind == "sliding":
        mask = window
    elif c.mask is not None:
        mask = c.mask.double().numpy() if mask_kind == "additive" else c.mask.numpy()
    ref = oracle.sdpa(q_rot, k_rot.double().numpy(), c.v.double().numpy(), np.float32(c.scale), mask_kind, mask)
    return c, k_rot, (cos, sin, R), q_pos0, ref


def run_fused(c, k_rot, rope, q_pos0, **kw):
    import scaled_dot_product_sdpa_amd as sdpa
    q = c.q.cuda()
    k = k_rot.cuda()
    v = c.v.cuda()
    mask = None if c.mask is None else c.mask.cuda()
    if c.mask_kind == "sliding":
        kw["window"] = c.meta["window"]
    out = sdpa.forward(q, k, v, scale=c.scale, mask=mask, mask_kind=c.mask_kind, rope=rope, q_pos0=q_pos0, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("mask_kind", ["none", "causal", "additive", "sliding"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D,R", [(64, 64), (72, 64), (128, 128), (128, 64), (256, 256), (256, 64),
                                 (512, 512), (512, 128)])
def test_fused_rope_prefill(gpu_lib, D, R, dtype, mask_kind):
    c, k_rot, rope, pos0, ref = fused_case(1, 4, 2, 150, 170, D, R, dtype, mask_kind, seed=D + R,
                                           window=40 if mask_kind == "sliding" else None)
    assert gpu_lib.select_kernel(1, 150, 170, 4, 2, D, si.DTYPES[dtype], mask_kind)[0] == "full"
    assert_parity(run_fused(c, k_rot, rope, pos0), ref, dtype, f"fused rope prefill D={D} R={R} {dtype} {mask_kind}")


@pytest.mark.parametrize("lq", [1, 5])
@pytest.mark.parametrize("D,R", [(64, 64), (128, 64), (256, 256), (512, 128)])
def test_fused_rope_decode(gpu_lib, D, R, lq):
    for mask_kind in ("none", "additive", "causal"):
        c, k_rot, rope, pos0, ref = fused_case(1, 8, 2, lq, 700, D, R, "bf16", mask_kind, seed=D + lq)
        assert_parity(run_fused(c, k_rot, rope, pos0), ref, "bf16", f"fused rope decode D={D} R={R} Lq={lq} {mask_kind}")


@pytest.mark.parametrize("R", [192, 64])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fused_rope_qk192_v128(gpu_lib, dtype, R):
    c, k_rot, rope, pos0, ref = fused_case(1, 16, 4, 3, 600, 192, R, dtype, "causal", seed=R, dv=128)
    out = run_fused(c, k_rot, rope, pos0)
    assert tuple(out.shape) == (1, 16, 3, 128)
    assert_parity(out, ref, dtype, f"fused rope qk192/v128 R={R} {dtype}")


@pytest.mark.parametrize("mask_kind", ["boolean", "additive"])
@pytest.mark.parametrize("D,R", [(72, 64), (128, 128), (256, 64), (512, 128)])
def test_fused_rope_with_strided_mask(gpu_lib, D, R, mask_kind):
    """A mask whose keys are strided goes through the element-wise mask
    instantiations with the rotary prologue: same bits as the contiguous mask."""
    import scaled_dot_product_sdpa_amd as sdpa
    c, k_rot, rope, pos0, ref = fused_case(1, 4, 2, 150, 164, D, R, "bf16", mask_kind, seed=D + 7)
    plain = run_fused(c, k_rot, rope, pos0)
    dm = c.mask.transpose(-1, -2).contiguous().cuda().transpose(-1, -2)
    assert torch.equal(dm.cpu(), c.mask)
    out = sdpa.forward(c.q.cuda(), k_rot.cuda(), c.v.cuda(), scale=c.scale, mask=dm, mask_kind=mask_kind,
                       rope=rope, q_pos0=pos0)
    torch.cuda.synchronize()
    assert_parity(out, ref, "bf16", f"fused rope strided {mask_kind} mask D={D} R={R}")
    assert torch.equal(out, plain), f"fused rope D={D}: strided and contiguous masks differ"


def test_fused_rope_explicit_positions_and_blhd(gpu_lib):
    # queries of a chunk in the middle of a long sequence: positions 3000.. read deep table rows
    c, k_rot, rope, pos0, ref = fused_case(2, 6, 3, 64, 90, 128, 128, "bf16", "none", seed=5, q_pos0=3000,
                                           layout="blhd")
    assert_parity(run_fused(c, k_rot, rope, pos0), ref, "bf16", "fused rope q_pos0=3000 blhd")


@pytest.mark.parametrize("D,R,lq", [(128, 128, 150), (72, 64, 150), (512, 128, 100), (256, 256, 1), (128, 64, 4)])
def test_fused_equals_rotate_then_attend(gpu_lib, D, R, lq):
    """Rotating Q inside the kernel and rotating it with the standalone kernel
    first round the same fp32 values once: the outputs agree bit for bit."""
    c, k_rot, (cos, sin, _), pos0, _ = fused_case(1, 4, 2, lq, 300, D, R, "bf16", "causal", seed=D)
    fused = run_fused(c, k_rot, (cos, sin, R), None)
    q_rot = gpu_lib.rope(c.q.cuda(), cos, sin, R, pos0=300 - lq)
    two = gpu_lib.forward(q_rot, k_rot.cuda(), c.v.cuda(), scale=c.scale, mask_kind="causal")
    torch.cuda.synchronize()
    assert torch.equal(fused, two)


def test_fused_rope_rejects_bad_positions_and_odd_dims(gpu_lib):
    cos, sin, _, _ = tables(64, 64)
    h = torch.zeros(1, 2, 8, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(gpu_lib.SdpaError):
        gpu_lib.forward(h, h, h, rope=(cos, sin, 64), q_pos0=60)         # rows 60..67 past a 64-row table
    c3, s3, _, _ = tables(64, 34)
    with pytest.raises(gpu_lib.SdpaError):
        gpu_lib.forward(h, h, h, rope=(c3[:, :16].contiguous(), s3[:, :16].contiguous(), 33))  # odd rotary dim


# --------------------------------------------------------------------------
# Any even rotary dim: the 25% partial rotations of the narrow heads (R = 16,
# 18, 20, 32 at D = 64, 72, 80, 128), a two-column one, R not a multiple of 16
# on the wide heads, on the prefill, single-launch decode and split decode
# kernels; and the fp32 kernels with a table.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("mask_kind", ["none", "causal", "additive"])
@pytest.mark.parametrize("D,R", [(64, 16), (72, 18), (80, 20), (96, 24), (128, 32), (128, 2), (256, 40),
                                 (512, 136), (72, 72)])
def test_fused_rope_any_even_dim_prefill(gpu_lib, D, R, mask_kind):
    c, k_rot, rope, pos0, ref = fused_case(1, 4, 2, 150, 170, D, R, "bf16", mask_kind, seed=D + 3 * R)
    assert_parity(run_fused(c, k_rot, rope, pos0), ref, "bf16", f"fused rope prefill D={D} R={R} {mask_kind}")


@pytest.mark.parametrize("lq", [1, 5])
@pytest.mark.parametrize("D,R", [(64, 16), (72, 18), (128, 32), (256, 40), (512, 136), (80, 2)])
def test_fused_rope_any_even_dim_decode(gpu_lib, D, R, lq):
    for hkv in (2, 8):  # 2 kv heads: split + combine kernels; 8 (with 32 query heads): the single launch
        c, k_rot, rope, pos0, ref = fused_case(1, 4 * hkv, hkv, lq, 700, D, R, "bf16", "additive", seed=D + lq)
        route = gpu_lib.describe_route(1, lq, 700, 4 * hkv, hkv, D, torch.bfloat16, "additive")
        assert_parity(run_fused(c, k_rot, rope, pos0), ref, "bf16",
                      f"fused rope decode D={D} R={R} Lq={lq} Hkv={hkv} ({route.split()[0]})")


@pytest.mark.parametrize("D,R,lq", [(72, 18, 150), (128, 32, 4), (256, 40, 1), (64, 16, 150)])
def test_fused_any_even_dim_equals_rotate_then_attend(gpu_lib, D, R, lq):
    c, k_rot, (cos, sin, _), pos0, _ = fused_case(1, 8, 2, lq, 300, D, R, "bf16", "causal", seed=D + R)
    fused = run_fused(c, k_rot, (cos, sin, R), None)
    q_rot = gpu_lib.rope(c.q.cuda(), cos, sin, R, pos0=300 - lq)
    two = gpu_lib.forward(q_rot, k_rot.cuda(), c.v.cuda(), scale=c.scale, mask_kind="causal")
    torch.cuda.synchronize()
    assert torch.equal(fused, two)


@pytest.mark.parametrize("lq,mask_kind", [(82, "none"), (82, "causal"), (3, "additive"), (1, "causal")])
@pytest.mark.parametrize("D,R", [(64, 64), (64, 16), (128, 34)])
def test_fused_rope_f32(gpu_lib, D, R, lq, mask_kind):
    c, k_rot, rope, pos0, ref = fused_case(2, 4, 2, lq, 90, D, R, "f32", mask_kind, seed=D + R + lq)
    assert_parity(run_fused(c, k_rot, rope, pos0), ref, "f32", f"fused rope f32 D={D} R={R} Lq={lq} {mask_kind}")
