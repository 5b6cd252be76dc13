"""GPU invariants: bitwise identities, determinism, split consistency, masks, memory."""
import os

import numpy as np
import pytest
import torch

import sdpa_inputs as si
from gpu_util import assert_parity, oracle_out, run_gpu, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D,dtype", [(72, "bf16"), (128, "f16"), (512, "bf16"), (64, "f32")])
def test_causal_row0_is_v0_bitwise(gpu_lib, D, dtype):
    c = si.make_case(1, 4, 2, 100, 100, D, dtype=dtype, mask_kind="causal", seed=3)
    out = run_gpu(c).cpu()
    v0 = c.v[:, :, :1].repeat_interleave(2, dim=1)
    assert torch.equal(out[:, :, 0:1], v0)


@pytest.mark.parametrize("lq,D,dtype", [(100, 72, "bf16"), (100, 512, "f16"), (100, 64, "f32"),
                                        (1, 256, "bf16"), (6, 128, "f32")])
def test_sliding_window_of_one_key_is_that_v_row_bitwise(gpu_lib, lq, D, dtype):
    """W = 1: every query keeps exactly its own position's key, so P = 1 and O = V[pos]."""
    c = si.make_case(1, 4, 2, lq, 130, D, dtype=dtype, mask_kind="sliding", seed=9, window=1)
    out = run_gpu(c).cpu()
    want = c.v[:, :, 130 - lq:].repeat_interleave(2, dim=1)
    assert torch.equal(out, want)


@pytest.mark.parametrize("lq,D,dtype", [(150, 72, "bf16"), (150, 256, "bf16"), (150, 80, "f32"), (3, 128, "bf16")])
def test_sliding_window_covering_every_key_is_causal_bitwise(gpu_lib, lq, D, dtype):
    c = si.make_case(1, 4, 2, lq, 300, D, dtype=dtype, mask_kind="sliding", seed=21, window=300)
    causal = si.Case(c.q, c.k, c.v, c.scale, "causal", None, c.layout)
    assert torch.equal(run_gpu(c), run_gpu(causal))


@pytest.mark.parametrize("lq", [1, 200])
def test_layout_permutation_is_bitwise_identical(gpu_lib, lq):
    a = si.make_case(1, 8, 4, lq, 300, 72, dtype="bf16", layout="blhd", mask_kind="causal", seed=11)
    b = si.Case(a.q.contiguous(), a.k.contiguous(), a.v.contiguous(), a.scale, "causal", None, "bhld")
    assert torch.equal(run_gpu(a), run_gpu(b))


@pytest.mark.parametrize("lq", [1, 150])
def test_run_to_run_determinism(gpu_lib, lq):
    c = si.make_case(1, 8, 2, lq, 3000, 256, dtype="bf16", mask_kind="additive", seed=5)
    outs = [run_gpu(c) for _ in range(3)]
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_forced_split_counts_agree(gpu_lib, monkeypatch):
    c = si.make_case(1, 8, 2, 2, 1000, 128, dtype="f32", mask_kind="additive", seed=9)
    ref = oracle_out(c)
    outs = []
    for s in ("1", "3", "7", "16"):
        monkeypatch.setenv("SDPA_DECODE_SPLITS", s)
        out = run_gpu(c)
        assert_parity(out, ref, "f32", f"splits={s}")
        outs.append(out)
    for o in outs[1:]:
        assert (o - outs[0]).abs().max().item() <= 2e-6


def test_decode_matches_last_row_of_prefill(gpu_lib):
    """q_len = 1 (vector kernel) vs the last row of a causal q_len = 64 call (full kernel)."""
    full = si.make_case(1, 8, 2, 64, 300, 128, dtype="bf16", mask_kind="causal", seed=21)
    one = si.Case(full.q[:, :, -1:], full.k, full.v, full.scale, "causal")
    a = run_gpu(full)[:, :, -1:].float()
    b = run_gpu(one).float()
    assert (a - b).abs().max().item() <= 1e-2


@pytest.mark.parametrize("D,prefix", [(128, 200), (72, 37), (256, 0)])
def test_bf16_chain_of_single_queries_matches_block_and_oracle(gpu_lib, D, prefix):
    """One T-query causal call (full kernel) against T calls of one query each (vector kernel),
    query i seeing keys [0, prefix + i]: every position, both against the oracle and each other."""
    T = 40
    c = si.make_case(1, 8, 2, T, prefix + T, D, dtype="bf16", mask_kind="causal", seed=31 + D)
    block = run_gpu(c)
    ref = oracle_out(c)
    assert_parity(block, ref, "bf16", "block call")
    chain = torch.empty_like(block)
    for i in range(T):
        e = prefix + i + 1
        one = si.Case(c.q[:, :, i:i + 1], c.k[:, :, :e], c.v[:, :, :e], c.scale, "causal")
        chain[:, :, i:i + 1] = run_gpu(one)
    assert_parity(chain, ref, "bf16", "chain of single-query calls")
    assert (chain.float() - block.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("dtype,tol_name", [("bf16", "bf16"), ("f16", "f16")])
def test_query_chunks_match_the_oracle_in_16_bit(gpu_lib, dtype, tol_name):
    """Chunked queries (bottom-right causal against the keys so far), each chunk against the oracle."""
    c = si.make_case(1, 4, 2, 300, 300, 80, dtype=dtype, mask_kind="causal", seed=17)
    whole = run_gpu(c)
    ref = oracle_out(c)
    assert_parity(whole, ref, tol_name, "block call")
    for s, e in ((0, 1), (1, 9), (9, 40), (40, 172), (172, 300)):
        part = si.Case(c.q[:, :, s:e], c.k[:, :, :e], c.v[:, :, :e], c.scale, "causal")
        assert_parity(run_gpu(part), ref[:, :, s:e], tol_name, f"chunk [{s}, {e})")


def test_query_chunks_match_the_block_call(gpu_lib):
    """Chunked queries (bottom-right causal against the keys so far) = one block call."""
    c = si.make_case(1, 4, 4, 96, 96, 64, dtype="f32", mask_kind="causal", seed=4)
    whole = run_gpu(c)
    for s, e in ((0, 1), (1, 9), (9, 40), (40, 96)):
        part = si.Case(c.q[:, :, s:e], c.k[:, :, :e], c.v[:, :, :e], c.scale, "causal")
        got = run_gpu(part)
        assert (got - whole[:, :, s:e]).abs().max().item() <= 2e-6, (s, e)


def test_boolean_equals_additive_minus_inf_bitwise(gpu_lib):
    c = si.make_case(1, 4, 2, 70, 200, 80, dtype="bf16", mask_kind="boolean", seed=8, mask_shape="qk", mask_p=0.3)
    add = torch.where(c.mask.bool(), torch.tensor(0.0), torch.tensor(-float("inf"))).to(torch.bfloat16)
    d = si.Case(c.q, c.k, c.v, c.scale, "additive", add)
    assert torch.equal(run_gpu(c), run_gpu(d))


@pytest.mark.parametrize("lq", [1, 50])
def test_fully_masked_row_is_zero(gpu_lib, lq):
    c = si.make_case(1, 2, 1, lq, 90, 64, dtype="bf16", mask_kind="boolean", seed=2, mask_shape="qk", mask_p=0.0)
    c.mask[0, 0, lq // 2, :] = 0
    out = run_gpu(c)
    assert torch.isfinite(out).all()
    assert (out[:, :, lq // 2] == 0).all()
    assert_parity(out, oracle_out(c), "bf16", "fully masked row")


def test_f16_minus_1e9_becomes_minus_inf_without_nan(gpu_lib):
    c = si.make_case(1, 8, 2, 1, 500, 128, dtype="f16", mask_kind="additive", seed=12, mask_p=0.5)
    assert torch.isinf(c.mask.float()).any()
    out = run_gpu(c)
    assert torch.isfinite(out).all()
    assert_parity(out, oracle_out(c), "f16", "f16 -inf additive")


def test_single_key_and_large_scores(gpu_lib):
    c = si.make_case(1, 2, 2, 20, 1, 64, dtype="f32", seed=1)
    out = run_gpu(c).cpu()
    assert torch.allclose(out, c.v.expand(1, 2, 20, 64), atol=0, rtol=0)
    big = si.make_case(1, 2, 2, 20, 40, 64, dtype="f32", seed=1, std=30.0)
    assert_parity(run_gpu(big), oracle_out(big), "f32", "large scores")


def test_output_canary_untouched(gpu_lib):
    import scaled_dot_product_sdpa_amd as sdpa
    c = si.make_case(1, 4, 2, 33, 77, 72, dtype="bf16", mask_kind="causal", seed=6)
    q, k, v, _ = to_device(c)
    buf = torch.full((4096 + 1 * 4 * 33 * 72 + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[4096:4096 + 4 * 33 * 72].view(1, 4, 33, 72)
    sdpa.forward(q, k, v, scale=c.scale, mask_kind="causal", out=out)
    torch.cuda.synchronize()
    assert (buf[:4096] == 7.0).all() and (buf[-4096:] == 7.0).all()
    assert_parity(out, oracle_out(c), "bf16", "canary")


@pytest.mark.parametrize("D,mask_kind", [(512, "causal"), (512, "none"), (256, "causal"), (512, "boolean")])
def test_wide_head_output_canary_with_ragged_rows(gpu_lib, D, mask_kind):
    """The wide-head kernel stores whole rows (at D = 512 through an LDS-staged tile, a row pair
    per instruction): rows past Lq in a ragged row tile must not be written, here the last head's
    tail next to the canary."""
    import scaled_dot_product_sdpa_amd as sdpa
    c = si.make_case(1, 4, 2, 45, 77, D, dtype="bf16", mask_kind=mask_kind, seed=7, mask_shape="qk")
    q, k, v, m = to_device(c)
    n = 1 * 4 * 45 * D
    buf = torch.full((4096 + n + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[4096:4096 + n].view(1, 4, 45, D)
    sdpa.forward(q, k, v, scale=c.scale, mask=m, mask_kind=mask_kind, out=out)
    torch.cuda.synchronize()
    assert (buf[:4096] == 7.0).all() and (buf[-4096:] == 7.0).all()
    assert_parity(out, oracle_out(c), "bf16", f"canary D={D} {mask_kind}")


def test_unsupported_shapes_raise_not_fall_back(gpu_lib):
    import scaled_dot_product_sdpa_amd as sdpa
    q = torch.zeros(1, 2, 16, 48, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.forward(q, q, q)
    assert e.value.status == -2
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 3, 16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(sdpa.SdpaError):
        sdpa.forward(q, k, k)
    # d stride != 1
    x = torch.zeros(1, 2, 64, 16, dtype=torch.bfloat16, device="cuda").transpose(2, 3)
    with pytest.raises(sdpa.SdpaError) as e:
        sdpa.forward(x, x, x)
    assert e.value.status == -2


@pytest.mark.parametrize("mask_kind", ["none", "boolean"])
def test_c4_peak_allocation_is_q_k_v_o_plus_mask(gpu_lib, mask_kind):
    """The head-dim-72 prefill at 16 heads x 8192: the whole run's peak device allocation is
    Q + K + V + O (4 x 18 MiB = 72 MiB) plus the mask tensor and the library's workspace (8 MiB
    of lane masks), nothing for scores."""
    import scaled_dot_product_sdpa_amd as sdpa
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    g = torch.Generator(device="cuda").manual_seed(4)
    shape = (1, 8192, 16, 72)  # [B, L, H, D]
    # filled in place: no temporaries in the measured peak
    q, k, v = (torch.empty(shape, device="cuda", dtype=torch.bfloat16).normal_(generator=g) for _ in range(3))
    out = torch.empty(shape, device="cuda", dtype=torch.bfloat16)
    mask = None
    if mask_kind == "boolean":  # uint8 0 / 1, 1 in 20 keys masked
        mask = torch.empty((1, 1, 8192, 8192), device="cuda", dtype=torch.uint8).random_(0, 20, generator=g)
        mask.clamp_(max=1)
    mask_bytes = mask.numel() if mask is not None else 0
    # the workspace the library asks for: 32 KiB of arrival words, then a boolean mask's lane
    # masks (32 words per 32 rows x 64 keys, 1/8 of a byte per mask element), allocated once by
    # the binding
    ws = sdpa.workspace_size(1, 8192, 8192, 16, 16, 72, torch.bfloat16)
    assert ws == 32768 + (8192 // 32) * (8192 // 64) * 256
    sdpa.forward(q, k, v, scale=72 ** -0.5, mask=mask, mask_kind=mask_kind, out=out, layout="blhd")
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    assert peak <= (72 << 20) + mask_bytes + ws, f"peak {peak / 2**20:.2f} MiB (mask {mask_bytes / 2**20:.0f} MiB)"
    assert torch.isfinite(out).all()


def test_no_score_tensor_is_materialised(gpu_lib):
    """Peak memory growth of a prefill call stays at the output size (no [B,H,L,L] scores)."""
    import scaled_dot_product_sdpa_amd as sdpa
    c = si.prefill512_case(seq=4096)
    q, k, v, _ = to_device(c)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    sdpa.forward(q, k, v, scale=c.scale, mask_kind="causal", out=out)
    torch.cuda.synchronize()
    grown = torch.cuda.max_memory_allocated() - base
    assert grown < (1 << 20), f"peak grew by {grown} bytes"
