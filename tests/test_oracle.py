"""Pins for the float64 oracle (CPU only).

Each test ties the oracle to something other than itself: values printed on
the pages, closed forms, invariants of softmax attention, an independent
library routine (torch's CPU attention in float64) and pure-Python brute
force.  The mutation tests at the end plant plausible mistakes in the oracle
and check that the pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sdpa_oracle as so
import sdpa_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p1_printed_values.json")


def _rand(shape, seed, std=1.0):
    return si.rng(seed).standard_normal(shape) * std


# ---------------------------------------------------------------------------
# Page 1 (mlx issue #3585): printed values of the deterministic reproduction.
# ---------------------------------------------------------------------------
def _p1_arrays():
    g = json.load(open(GOLDEN))
    B, S, H, D = g["shape_blhd"]
    a = si.linspace_block((B, S, H, D)).astype(np.float64)
    scale = float(np.float32(D ** -0.5))
    # the page's "manual": softmax with no axis = over the whole score array
    qt = a.transpose(0, 2, 1, 3)
    sc = qt @ qt.transpose(0, 1, 3, 2) * scale
    e = np.exp(sc - sc.max())
    manual = ((e / e.sum()) @ qt).transpose(0, 2, 1, 3)
    flat = a.reshape(-1)
    blhd = (S * H * D, D, H * D, 1)     # logical (b, h, l, d) strides of [B,S,H,D] storage
    bhld = (S * H * D, H * D, D, 1)     # the same buffer read as if it were [B,H,L,D]
    correct = oracle.sdpa_strided(flat, blhd, flat, blhd, flat, blhd, B, S, S, H, H, D, scale)
    swapped = oracle.sdpa_strided(flat, bhld, flat, bhld, flat, bhld, B, H, H, S, S, D, scale)
    return g, manual, correct.transpose(0, 2, 1, 3), swapped


def test_p1_input_generator_matches_printed_array():
    g = json.load(open(GOLDEN))
    a = si.linspace_block(g["shape_blhd"])
    assert a.dtype == np.float32
    for idx, val in g["input_entries"]:
        x = float(a[tuple(idx)])
        # numpy prints 6 significant digits
        assert abs(x - val) <= 5e-7 * max(abs(val), 1e-5) * 10 or abs(x - val) < 1e-12, (idx, x, val)


def test_p1_layout_bug_reproduces_printed_max_diff():
    g, manual, _, swapped = _p1_arrays()
    d = np.abs(manual - swapped)
    assert abs(d.max() - g["max_diff_manual_vs_fused"]) < 5e-8, d.max()
    worst = np.unravel_index(d.argmax(), d.shape)
    assert tuple(int(i) for i in worst) == (0, 0, 7, 0)
    assert abs(manual[worst] - g["worst_element_manual"]) < 5e-7
    assert abs(swapped[worst] - g["worst_element_fused"]) < 5e-7


def test_p1_correct_attention_reproduces_printed_pytorch_diff():
    g, manual, correct, _ = _p1_arrays()
    assert abs(np.abs(manual - correct).max() - g["max_diff_manual_vs_pytorch"]) < 5e-8


def test_p1_layout_bug_is_not_float_noise():
    _, _, correct, swapped = _p1_arrays()
    assert np.abs(correct - swapped.reshape(correct.shape)).max() > 0.2


# ---------------------------------------------------------------------------
# Brute force (math.fsum) on tiny shapes, every mask kind, GQA.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mask_kind", oracle.MASK_KINDS)
@pytest.mark.parametrize("lq,lk", [(3, 5), (5, 3), (1, 4), (4, 4)])
def test_oracle_matches_brute_force(mask_kind, lq, lk):
    B, Hq, Hkv, D = 2, 4, 2, 3
    q, k, v = _rand((B, Hq, lq, D), 1), _rand((B, Hkv, lk, D), 2), _rand((B, Hkv, lk, D), 3)
    mask = None
    if mask_kind == "additive":
        mask = _rand((1, Hq, lq, lk), 4)
    elif mask_kind == "boolean":
        mask = si.rng(5).random((B, 1, lq, lk)) > 0.3
    elif mask_kind == "sliding":
        mask = 2
    ref = oracle.brute_force_sdpa(q, k, v, 0.37, mask_kind, mask)
    got = oracle.sdpa(q, k, v, 0.37, mask_kind, mask)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# An independent library routine: torch's CPU attention in float64.
# (torch's is_causal is top-left aligned; it agrees with bottom-right when Lq == Lk.)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mask_kind", oracle.MASK_KINDS)
def test_oracle_matches_torch_float64(mask_kind):
    B, Hq, Hkv, L, D = 2, 8, 2, 37, 24
    q, k, v = _rand((B, Hq, L, D), 11), _rand((B, Hkv, L, D), 12), _rand((B, Hkv, L, D), 13)
    mask = None
    kw = {}
    if mask_kind == "additive":
        mask = _rand((B, 1, L, L), 14) * 3
        kw["attn_mask"] = torch.from_numpy(mask)
    elif mask_kind == "boolean":
        mask = si.rng(15).random((1, Hq, L, L)) > 0.2
        np.fill_diagonal(mask[0, 0], True)
        kw["attn_mask"] = torch.from_numpy(mask)
    elif mask_kind == "causal":
        kw["is_causal"] = True
    elif mask_kind == "sliding":
        # torch has no sliding kind: keep the lower triangle minus everything
        # W or more diagonals below it (Lq == Lk here)
        mask = 5
        ones = torch.ones(L, L, dtype=torch.bool)
        kw["attn_mask"] = torch.tril(ones) & ~torch.tril(ones, diagonal=-mask)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.21, enable_gqa=True, **kw)
    got = oracle.sdpa(q, k, v, 0.21, mask_kind, mask)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Closed forms and invariants.
# ---------------------------------------------------------------------------
def test_constant_v_gives_that_row():
    q, k = _rand((1, 2, 9, 8), 1), _rand((1, 2, 13, 8), 2)
    v = np.broadcast_to(_rand((1, 2, 1, 8), 3), (1, 2, 13, 8))
    out = oracle.sdpa(q, k, v, 0.5, "additive", _rand((1, 1, 9, 13), 4))
    np.testing.assert_allclose(out, np.broadcast_to(v[:, :, :1], out.shape), rtol=1e-14, atol=1e-14)


def test_identical_keys_give_mean_of_v_and_causal_prefix_means():
    k = np.broadcast_to(_rand((1, 1, 1, 6), 1), (1, 1, 10, 6))
    q, v = _rand((1, 1, 10, 6), 2), _rand((1, 1, 10, 6), 3)
    out = oracle.sdpa(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0].mean(0), (10, 6)), rtol=1e-13, atol=1e-14)
    out = oracle.sdpa(q, k, v, 1.0, "causal")
    for i in range(10):
        np.testing.assert_allclose(out[0, 0, i], v[0, 0, : i + 1].mean(0), rtol=1e-13, atol=1e-14)
    # bottom-right alignment with Lq < Lk: query i sees keys 0 .. i + (Lk - Lq)
    out = oracle.sdpa(q[:, :, :3], k, v, 1.0, "causal")
    for i in range(3):
        np.testing.assert_allclose(out[0, 0, i], v[0, 0, : i + 8].mean(0), rtol=1e-13, atol=1e-14)


def test_probability_rows_sum_to_one_and_are_nonnegative():
    q, k = _rand((2, 4, 7, 5), 1), _rand((2, 2, 11, 5), 2)
    for kind, mask in (("none", None), ("causal", None), ("additive", _rand((2, 4, 7, 11), 3)),
                       ("boolean", si.rng(4).random((1, 1, 7, 11)) > 0.5)):
        p = oracle.attention_weights(q, k, 0.7, kind, mask)
        s = p.sum(-1)
        live = s > 0
        np.testing.assert_allclose(s[live], 1.0, atol=1e-12)
        assert (p >= 0).all()


def test_attention_weights_group_query_heads_by_consecutive_runs():
    """Query head h reads kv head h // n_rep (consecutive runs of n_rep heads share a kv head):
    kv head 0 has identical keys (uniform weights), kv head 1 one key far above the rest (a
    one-hot row).  A mapping h % Hkv would give heads 1 and 2 the other kv head's pattern."""
    Lk, D = 6, 4
    q = np.ones((1, 4, 2, D))
    k = np.zeros((1, 2, Lk, D))
    k[0, 1, 3] = 50.0
    p = oracle.attention_weights(q, k, 1.0)
    for h in (0, 1):
        np.testing.assert_allclose(p[0, h], 1.0 / Lk, atol=1e-15)
    for h in (2, 3):
        np.testing.assert_allclose(p[0, h, :, 3], 1.0, atol=1e-12)
        np.testing.assert_allclose(np.delete(p[0, h], 3, axis=-1), 0.0, atol=1e-12)


def test_rope_tables_are_the_base_10000_angles():
    """cos/sin of angle(pos, j) = pos * 10000^(-2j/R): at pos 1 column j's angle is the j-th power of
    10000^(-2/R) (R = 64: 0.74989420933...), the angle grows linearly with the position, and column 0
    turns one radian per position (cos 1 = 0.5403023058681398, sin 1 = 0.8414709848078965)."""
    c, s_ = oracle.rope_tables(9, 64)
    assert c.shape == s_.shape == (9, 32)
    assert c[1, 0] == pytest.approx(0.5403023058681398, abs=1e-15)
    assert s_[1, 0] == pytest.approx(0.8414709848078965, abs=1e-15)
    ang = np.arctan2(s_, c)
    np.testing.assert_allclose(ang[0], 0.0, atol=0)
    ratio = ang[1, 1:] / ang[1, :-1]
    np.testing.assert_allclose(ratio, 0.7498942093324559, rtol=1e-12)
    np.testing.assert_allclose(ang[3], 3.0 * ang[1], rtol=1e-12)  # below pi: no wrap


def test_causal_row0_is_v0_and_single_key_is_v0():
    q, k, v = _rand((1, 3, 6, 4), 1), _rand((1, 3, 6, 4), 2), _rand((1, 3, 6, 4), 3)
    out = oracle.sdpa(q, k, v, 2.0, "causal")
    np.testing.assert_array_equal(out[:, :, 0], v[:, :, 0])
    out = oracle.sdpa(q, k[:, :, :1], v[:, :, :1], 2.0)
    np.testing.assert_allclose(out, np.broadcast_to(v[:, :, :1], out.shape), rtol=1e-15, atol=0)


def test_zero_scale_gives_mean_of_v():
    q, k, v = _rand((1, 2, 5, 4), 1), _rand((1, 2, 9, 4), 2), _rand((1, 2, 9, 4), 3)
    out = oracle.sdpa(q, k, v, 0.0)
    np.testing.assert_allclose(out, np.broadcast_to(v.mean(2, keepdims=True), out.shape), rtol=1e-13, atol=1e-14)


def test_one_hot_scores_do_not_overflow():
    D = 4
    k = np.eye(D)[None, None] * 100.0            # key j along axis j
    v = _rand((1, 1, D, 3), 1)
    q = np.zeros((1, 1, 1, D))
    q[..., 2] = 100.0                             # score 1e4 on key 2, 0 elsewhere
    out = oracle.sdpa(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, 0, 0], v[0, 0, 2], rtol=1e-15, atol=0)


def test_boolean_mask_equals_additive_minus_inf():
    q, k, v = _rand((2, 4, 6, 5), 1), _rand((2, 2, 8, 5), 2), _rand((2, 2, 8, 5), 3)
    bm = si.rng(4).random((2, 1, 6, 8)) > 0.4
    bm[..., 0] = True
    a = oracle.sdpa(q, k, v, 0.3, "boolean", bm)
    b = oracle.sdpa(q, k, v, 0.3, "additive", np.where(bm, 0.0, -np.inf))
    np.testing.assert_array_equal(a, b)


def test_fully_masked_row_gives_zero():
    q, k, v = _rand((1, 1, 3, 4), 1), _rand((1, 1, 5, 4), 2), _rand((1, 1, 5, 4), 3)
    bm = np.ones((1, 1, 3, 5), bool)
    bm[0, 0, 1] = False
    out = oracle.sdpa(q, k, v, 1.0, "boolean", bm)
    assert (out[0, 0, 1] == 0).all() and np.abs(out[0, 0, 0]).sum() > 0


def test_layout_permutation_with_matching_strides_is_identity():
    B, L, H, D = 2, 7, 3, 5
    x = _rand((B, L, H, D), 1)                    # [B,L,H,D] storage
    y = np.ascontiguousarray(x.transpose(0, 2, 1, 3))  # the same logical tensor stored [B,H,L,D]
    a = oracle.sdpa_strided(x.reshape(-1), (L * H * D, D, H * D, 1), x.reshape(-1), (L * H * D, D, H * D, 1),
                            x.reshape(-1), (L * H * D, D, H * D, 1), B, L, L, H, H, D, 0.4)
    b = oracle.sdpa_strided(y.reshape(-1), (H * L * D, L * D, D, 1), y.reshape(-1), (H * L * D, L * D, D, 1),
                            y.reshape(-1), (H * L * D, L * D, D, 1), B, L, L, H, H, D, 0.4)
    np.testing.assert_array_equal(a, b)


def test_gather_strided_reads_the_named_elements():
    flat = np.arange(2 * 3 * 4 * 5)
    t = oracle.gather_strided(flat, (2, 4, 3, 5), (60, 5, 20, 1))   # [B,L,H,D] storage read as (b,h,l,d)
    assert t[1, 2, 0, 3] == 1 * 60 + 0 * 20 + 2 * 5 + 3
    np.testing.assert_array_equal(t, flat.reshape(2, 3, 4, 5).transpose(0, 2, 1, 3))


def test_gqa_equals_mha_with_repeated_kv():
    q, k, v = _rand((2, 8, 5, 4), 1), _rand((2, 2, 7, 4), 2), _rand((2, 2, 7, 4), 3)
    a = oracle.sdpa(q, k, v, 0.6, "causal")
    b = oracle.sdpa(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.6, "causal")
    np.testing.assert_array_equal(a, b)
    # contiguous groups: head 5 uses kv head 1, not kv head 5 % 2
    c = oracle.sdpa(q[:, 5:6], k[:, 1:2], v[:, 1:2], 0.6, "causal")
    np.testing.assert_array_equal(a[:, 5:6], c)


def test_sliding_window_closed_forms():
    """W = 1 keeps one key (O = V[pos]); W >= every position is plain causal;
    identical keys give the mean of V over the window (Lq < Lk: positions shift)."""
    q, k, v = _rand((1, 2, 6, 4), 1), _rand((1, 1, 9, 4), 2), _rand((1, 1, 9, 4), 3)
    off = 9 - 6
    one = oracle.sdpa(q, k, v, 0.7, "sliding", 1)
    for i in range(6):
        np.testing.assert_allclose(one[0, :, i], np.broadcast_to(v[0, 0, i + off], (2, 4)), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(oracle.sdpa(q, k, v, 0.7, "sliding", 9), oracle.sdpa(q, k, v, 0.7, "causal"))
    np.testing.assert_array_equal(oracle.sdpa(q, k, v, 0.7, "sliding", 50), oracle.sdpa(q, k, v, 0.7, "causal"))
    same = np.broadcast_to(k[:, :, :1], k.shape)
    for w in (2, 4):
        got = oracle.sdpa(q, same, v, 0.7, "sliding", w)
        for i in range(6):
            lo = max(0, i + off - w + 1)
            np.testing.assert_allclose(got[0, 0, i], v[0, 0, lo:i + off + 1].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_sliding_window_chunks_match_the_block():
    """Query chunks against the full key range, bottom-right aligned, equal the block."""
    q, k, v = _rand((1, 2, 12, 4), 5), _rand((1, 2, 12, 4), 6), _rand((1, 2, 12, 4), 7)
    full = oracle.sdpa(q, k, v, 0.5, "sliding", 4)
    for s0 in range(0, 12, 5):
        s1 = min(12, s0 + 5)
        part = oracle.sdpa(q[:, :, s0:s1], k[:, :, :s1], v[:, :, :s1], 0.5, "sliding", 4)
        np.testing.assert_allclose(part, full[:, :, s0:s1], rtol=1e-13, atol=1e-14)


def test_value_head_dim_columns_are_independent():
    """O's columns depend only on the matching V columns: a V head dim of 128
    under 192-wide queries and keys is the first 128 columns of the 192-wide
    result (the (192, 128) pairing); brute force agrees."""
    q, k, v = _rand((1, 4, 5, 192), 1), _rand((1, 2, 9, 192), 2), _rand((1, 2, 9, 192), 3)
    for kind, m in (("none", None), ("causal", None), ("sliding", 3)):
        wide = oracle.sdpa(q, k, v, 0.07, kind, m)
        narrow = oracle.sdpa(q, k, v[..., :128], 0.07, kind, m)
        assert narrow.shape == (1, 4, 5, 128)
        np.testing.assert_array_equal(narrow, wide[..., :128])
    small = (q[:, :, :3, :6], k[:, :, :4, :6], v[:, :, :4, :2])
    np.testing.assert_allclose(oracle.sdpa(*small, 0.3, "causal"), oracle.brute_force_sdpa(*small, 0.3, "causal"),
                               rtol=1e-13, atol=1e-14)


def test_rope_scores_depend_only_on_relative_position():
    """With the usual tables, <RoPE(q) at i, RoPE(k) at j> depends on i - j only."""
    cos, sin = oracle.rope_tables(64, 32)
    q, k = _rand((1, 1, 1, 48), 1), _rand((1, 1, 1, 48), 2)
    def dot(i, j):
        return float((oracle.rope(q, cos, sin, 32, i) * oracle.rope(k, cos, sin, 32, j)).sum())
    for i, j, shift in ((5, 2, 7), (0, 9, 30), (20, 20, 11)):
        assert abs(dot(i, j) - dot(i + shift, j + shift)) < 1e-12
    assert abs(dot(5, 2) - dot(2, 5)) > 1e-3  # but the sign of i - j matters


def test_rope_closed_forms():
    x = _rand((2, 3, 4, 16), 3)
    cos, sin = oracle.rope_tables(8, 8)
    y = oracle.rope(x, cos, sin, 8, 2)
    np.testing.assert_array_equal(y[..., 8:], x[..., 8:])                  # columns >= R pass through
    np.testing.assert_array_equal(oracle.rope(x, cos, sin, 0), x)          # R = 0: identity
    np.testing.assert_allclose(oracle.rope(x[..., :1, :], cos, sin, 8, 0), x[..., :1, :], atol=0)  # position 0
    pair = x[..., :4] ** 2 + x[..., 4:8] ** 2                              # each (j, j + R/2) pair keeps its norm
    np.testing.assert_allclose(y[..., :4] ** 2 + y[..., 4:8] ** 2, pair, rtol=1e-13)
    np.testing.assert_allclose(oracle.rope(y, cos, -sin, 8, 2), x, rtol=1e-13, atol=1e-14)  # inverse rotation
    # a quarter turn maps (a, b) to (-b, a)
    qc, qs = np.zeros((1, 1)), np.ones((1, 1))
    v = np.array([[[[3.0, 5.0]]]])
    np.testing.assert_array_equal(oracle.rope(v, qc, qs, 2, 0), np.array([[[[-5.0, 3.0]]]]))
    # the tables are the angle pos * 10000^(-2j/R)
    c, s_ = oracle.rope_tables(5, 6)
    assert abs(c[3, 2] - math.cos(3 * 10000 ** (-4 / 6))) < 1e-15 and abs(s_[4, 1] - math.sin(4 * 10000 ** (-2 / 6))) < 1e-15


def test_constant_additive_shift_is_invariant():
    q, k, v = _rand((1, 2, 6, 4), 1), _rand((1, 2, 9, 4), 2), _rand((1, 2, 9, 4), 3)
    m = _rand((1, 1, 6, 9), 4)
    a = oracle.sdpa(q, k, v, 0.5, "additive", m)
    b = oracle.sdpa(q, k, v, 0.5, "additive", m + 1234.5)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("cuts", [[0, 9], [0, 1, 9], [0, 4, 5, 9], [0, 2, 3, 6, 8, 9]])
def test_lse_merge_of_any_key_partition_is_the_full_result(cuts):
    q, k, v = _rand((1, 4, 3, 5), 1), _rand((1, 2, 9, 5), 2), _rand((1, 2, 9, 5), 3)
    m = np.where(si.rng(4).random((1, 1, 3, 9)) < 0.3, -np.inf, 0.0)
    m[..., 0] = 0.0
    states = [oracle.partial_state(q, k, v, 0.8, "additive", m, a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    np.testing.assert_allclose(oracle.merge_states(states), oracle.sdpa(q, k, v, 0.8, "additive", m),
                               rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("chunk", [1, 2, 3, 5])
def test_query_chunks_with_bottom_right_causal_match_the_block(chunk):
    """Chunked queries against the full K = the unchunked call (mlxcel issue #1065, tests 1 and 2)."""
    L = 7
    q, k, v = _rand((1, 2, L, 4), 1), _rand((1, 2, L, 4), 2), _rand((1, 2, L, 4), 3)
    full = oracle.sdpa(q, k, v, 0.9, "causal")
    for s in range(0, L, chunk):
        e = min(L, s + chunk)
        # the chunk's queries sit at positions s..e-1 and may see keys 0..e-1
        part = oracle.sdpa(q[:, :, s:e], k[:, :, :e], v[:, :, :e], 0.9, "causal")
        np.testing.assert_allclose(part, full[:, :, s:e], rtol=1e-13, atol=1e-14)


def test_q_rows_subset_matches_full_computation():
    q, k, v = _rand((1, 2, 12, 4), 1), _rand((1, 2, 12, 4), 2), _rand((1, 2, 12, 4), 3)
    full = oracle.sdpa(q, k, v, 0.9, "causal")
    rows = [0, 5, 11]
    np.testing.assert_array_equal(oracle.sdpa(q, k, v, 0.9, "causal", q_rows=rows), full[:, :, rows])


def test_bf16_minus_1e9_mask_value_is_what_the_oracle_adds():
    # bf16 rounds -1e9 to -998244352; fp16 overflows it to -inf (a reading the kernels must honour)
    assert float(torch.tensor(-1e9).to(torch.bfloat16)) == -998244352.0
    assert float(torch.tensor(-1e9).to(torch.float16)) == -math.inf


# ---------------------------------------------------------------------------
# Planted mistakes: each must break at least one pin above.
# ---------------------------------------------------------------------------
def _pins_hold():
    """Run a representative set of pins; False as soon as one fails."""
    pins = [test_p1_correct_attention_reproduces_printed_pytorch_diff,
            test_p1_layout_bug_reproduces_printed_max_diff,
            test_gqa_equals_mha_with_repeated_kv,
            test_identical_keys_give_mean_of_v_and_causal_prefix_means,
            test_one_hot_scores_do_not_overflow,
            test_sliding_window_closed_forms,
            test_rope_closed_forms]
    pins += [lambda k=k: test_oracle_matches_torch_float64(k) for k in oracle.MASK_KINDS]
    pins += [lambda k=k: test_oracle_matches_brute_force(k, 3, 5) for k in oracle.MASK_KINDS]
    with np.errstate(all="ignore"):
        for pin in pins:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                return False
    return True


def test_pins_hold_for_the_real_oracle():
    assert _pins_hold()


@pytest.mark.parametrize("mutation", ["no_scale", "softmax_over_queries", "reversed_v_rows",
                                      "head_modulo", "causal_top_left", "mask_dropped",
                                      "mask_scaled", "no_max_shift", "sliding_window_plus_one",
                                      "rope_sign_flip", "rope_adjacent_pairs"])
def test_planted_mistakes_are_caught(monkeypatch, mutation):
    """Plant a plausible mistake in the oracle (CPU) and check that a pin fails."""
    if mutation == "no_scale":
        monkeypatch.setattr(so, "_scores", lambda qh, kg, scale, b: qh @ kg.T + b)
    elif mutation == "softmax_over_queries":
        orig = so._softmax_rows
        monkeypatch.setattr(so, "_softmax_rows", lambda s: orig(s.T).T)
    elif mutation == "reversed_v_rows":
        orig = so._softmax_rows
        monkeypatch.setattr(so, "_softmax_rows", lambda s: orig(s)[..., ::-1])
    elif mutation == "head_modulo":
        orig_prepare = so._prepare

        def bad_prepare(q, k, v, kind, mask):
            q2, k2, v2, n_rep, bias = orig_prepare(q, k, v, kind, mask)
            hq, hkv = q2.shape[1], k2.shape[1]
            idx = np.arange(hq) % hkv             # interleaved instead of contiguous groups
            return q2, k2[:, idx], v2[:, idx], 1, bias
        monkeypatch.setattr(so, "_prepare", bad_prepare)
    elif mutation == "causal_top_left":
        orig = so.mask_bias

        def bad_bias(kind, mask, lq, lk):
            if kind == "causal":
                j = np.arange(lk)[None, :]
                i = np.arange(lq)[:, None]
                return np.where(j <= i, 0.0, -np.inf)[None, None]
            return orig(kind, mask, lq, lk)
        monkeypatch.setattr(so, "mask_bias", bad_bias)
    elif mutation == "mask_dropped":
        orig = so.mask_bias
        monkeypatch.setattr(so, "mask_bias", lambda kind, mask, lq, lk:
                            orig("none", None, lq, lk) if kind == "additive" else orig(kind, mask, lq, lk))
    elif mutation == "mask_scaled":
        monkeypatch.setattr(so, "_scores", lambda qh, kg, scale, b: (qh @ kg.T + b) * float(scale))
    elif mutation == "rope_sign_flip":
        orig = so.rope

        def bad(x, cos, sin, r, pos0=0):
            return orig(x, cos, -np.asarray(sin), r, pos0)
        monkeypatch.setattr(so, "rope", bad)
        monkeypatch.setattr(oracle, "rope", bad)
    elif mutation == "rope_adjacent_pairs":   # the interleaved (2j, 2j+1) convention instead of (j, j + R/2)
        orig = so.rope

        def bad(x, cos, sin, r, pos0=0):
            x = np.asarray(x, dtype=np.float64)
            if r == 0:
                return x.copy()
            idx = np.concatenate([np.arange(0, r, 2), np.arange(1, r, 2), np.arange(r, x.shape[-1])])
            inv = np.argsort(idx)
            return orig(x[..., idx], cos, sin, r, pos0)[..., inv]
        monkeypatch.setattr(so, "rope", bad)
        monkeypatch.setattr(oracle, "rope", bad)
    elif mutation == "sliding_window_plus_one":
        orig = so.mask_bias
        monkeypatch.setattr(so, "mask_bias", lambda kind, mask, lq, lk:
                            orig(kind, int(mask) + 1, lq, lk) if kind == "sliding" else orig(kind, mask, lq, lk))
    elif mutation == "no_max_shift":
        monkeypatch.setattr(so, "_softmax_rows", lambda s: np.nan_to_num(
            np.exp(s) / np.exp(s).sum(-1, keepdims=True)))
    assert not _pins_hold(), mutation
