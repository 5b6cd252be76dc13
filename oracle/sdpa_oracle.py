"""Oracle for fused scaled dot-product attention: plain, slow, float64, CPU.

TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import or run this module. The GPU library
never calls it, and it shares no code, header, table or helper with the GPU
library: it is the definition written out, so that a reader can check it
against the pages by eye.

What it computes (for every batch b, query head h and query row i):

    g        = h // (Hq / Hkv)                      grouped-query head mapping
    s[i, j]  = scale * <Q[b,h,i,:], K[b,g,j,:]> + M[i, j]
    p[i, j]  = exp(s[i,j] - max_j s[i,j]) / sum_j exp(s[i,j] - max_j s[i,j])
    O[b,h,i] = sum_j p[i, j] * V[b,g,j,:]

Sources (titles of the pages; section in brackets):
  * mlx issue "mx.fast.scaled_dot_product_attention produces incorrect
    attention scores (MLX 0.31.2)" [Reproduction]: the manual attention that
    replaces the fused call -- transpose to [B,H,L,D], Q K^T times scale,
    softmax over the key axis (axis=-1), times V, transpose back.  The same
    page [root-cause comment] explains that the kernel indexes Q by explicit
    batch / head / sequence strides; `gather_strided` is that indexing.
  * mlx issue #3885 "Metal SDPA: no fused path for head_dim=512" [Prefill
    paragraph]: grouped-query attention scores have shape
    [B, n_kv, n_rep, qL, kL], i.e. query heads form contiguous groups of
    n_rep per key/value head.
  * mlx PR #4330 "Support head dimension 72 in Metal full attention"
    [Proposed changes]: the mask kinds are none, additive, boolean, causal.
  * mlx issue #3885 [Summary]: the d=256 model whose shapes drive the decode
    configuration alternates "sliding" (local) layers with global ones; the
    sliding kind here is that local attention.

Readings where the pages are silent (each is also listed in the design notes):
  * boolean masks: true / nonzero = attend, false = masked (bias -inf);
  * causal masks are aligned bottom-right: query row i sits at key position
    i + (Lk - Lq), and attends to keys j <= that position;
  * an additive mask is added after the scale (it is not scaled);
  * a row whose every key is masked has no defined softmax; its output is 0;
  * rotary position embedding (RoPE) follows the rotate-half convention of
    the pre-computed cos/sin tables named in mlx issue #3585 [Model config]
    ([positions, head_dim] tables, base 10000): the first R head-dim columns
    form pairs (c, c + R/2) rotated by the angle of (position, c); columns
    >= R pass through ("25% partial RoPE" in mlx issue #3885 [Summary] is
    R = D/4).  The tables are inputs: cos[pos][c], sin[pos][c], c < R/2;
  * sliding (local) attention keeps the causal alignment and a window of W
    keys: query i at position pos = i + (Lk - Lq) attends keys j with
    pos - W < j <= pos (the page names the layer type, not its formula; this
    is the usual local-causal window, the current key included).

Parity pins for every function here live in tests/test_oracle.py.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence

import numpy as np

MASK_KINDS = ("none", "additive", "boolean", "causal", "sliding")


# --------------------------------------------------------------------------
# Strided reads: a logical (b, h, l, d) tensor out of a flat buffer.
# --------------------------------------------------------------------------
def gather_strided(flat, shape: Sequence[int], strides: Sequence[int], offset: int = 0) -> np.ndarray:
    """Read the logical tensor of `shape` from the 1-D buffer `flat`.

    Element (i0, i1, ...) of the result is flat[offset + sum_k i_k * strides[k]].
    Strides are in elements.  This is how a kernel that is handed explicit
    batch / head / sequence strides reads its operands (mlx issue 3585,
    root-cause comment: Q is advanced by Q_strides[0..2] for batch, head and
    sequence).  Passing the strides of another layout reads the same memory as
    a different logical tensor -- which is exactly that page's layout bug.
    """
    flat = np.asarray(flat).reshape(-1)
    idx = np.full(tuple(shape), offset, dtype=np.int64)
    for axis, (n, st) in enumerate(zip(shape, strides)):
        view = [1] * len(shape)
        view[axis] = n
        idx = idx + (np.arange(n, dtype=np.int64) * int(st)).reshape(view)
    return flat[idx]


# --------------------------------------------------------------------------
# Mask -> additive bias (float64), broadcastable to [B, Hq, Lq, Lk].
# --------------------------------------------------------------------------
def mask_bias(mask_kind: str, mask, q_len: int, kv_len: int) -> np.ndarray:
    """Bias added to the scaled scores for each mask kind.

    none     -> 0
    additive -> the stored mask values, widened exactly to float64
    boolean  -> 0 where the mask is true (nonzero), -inf where it is false
    causal   -> 0 where key j <= i + (kv_len - q_len), else -inf
    sliding  -> `mask` is the window W >= 1: 0 where pos - W < j <= pos with
                pos = i + (kv_len - q_len), else -inf
    """
    if mask_kind == "none":
        return np.zeros((1, 1, 1, 1), dtype=np.float64)
    if mask_kind == "additive":
        return np.asarray(mask, dtype=np.float64)
    if mask_kind == "boolean":
        m = np.asarray(mask)
        return np.where(m != 0, 0.0, -np.inf)
    if mask_kind == "causal":
        pos = np.arange(q_len, dtype=np.int64)[:, None] + (kv_len - q_len)
        key = np.arange(kv_len, dtype=np.int64)[None, :]
        return np.where(key <= pos, 0.0, -np.inf)[None, None, :, :]
    if mask_kind == "sliding":
        window = int(mask)
        if window < 1:
            raise ValueError("sliding window must be >= 1")
        pos = np.arange(q_len, dtype=np.int64)[:, None] + (kv_len - q_len)
        key = np.arange(kv_len, dtype=np.int64)[None, :]
        return np.where((key <= pos) & (key > pos - window), 0.0, -np.inf)[None, None, :, :]
    raise ValueError(f"unknown mask kind {mask_kind!r}")


def _group_size(n_q_heads: int, n_kv_heads: int) -> int:
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return n_q_heads // n_kv_heads


def _scores(qh: np.ndarray, kg: np.ndarray, scale: float, bias_rows: np.ndarray) -> np.ndarray:
    """scale * Q K^T + bias for one (b, h): [rows, Lk] float64."""
    return (qh @ kg.T) * float(scale) + bias_rows


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Numerically stable softmax over the last axis; fully masked rows -> 0."""
    m = s.max(axis=-1, keepdims=True)
    dead = ~np.isfinite(m)  # every entry is -inf
    m = np.where(dead, 0.0, m)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    z = np.where(dead, 1.0, z)
    return e / z


def _prepare(q, k, v, mask_kind, mask):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be 4-D logical [B, H, L, D]")
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if (Bk, Dk) != (B, D) or v.shape[:3] != k.shape[:3]:
        raise ValueError("shape mismatch between q, k, v")
    n_rep = _group_size(Hq, Hkv)
    bias = np.broadcast_to(mask_bias(mask_kind, mask, Lq, Lk), (B, Hq, Lq, Lk))
    return q, k, v, n_rep, bias


def attention_weights(q, k, scale: float, mask_kind: str = "none", mask=None) -> np.ndarray:
    """The probability tensor p[b, h, i, j] (float64, materialised; small inputs only)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, Lq, _ = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    n_rep = _group_size(Hq, Hkv)
    bias = np.broadcast_to(mask_bias(mask_kind, mask, Lq, Lk), (B, Hq, Lq, Lk))
    out = np.empty((B, Hq, Lq, Lk), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            s = _scores(q[b, h], k[b, h // n_rep], scale, bias[b, h])
            out[b, h] = _softmax_rows(s)
    return out


def sdpa(q, k, v, scale: float, mask_kind: str = "none", mask=None,
         q_rows: Iterable[int] | None = None) -> np.ndarray:
    """softmax(scale * Q K^T + M) V with grouped-query heads, in float64.

    q: logical [B, Hq, Lq, D]; k: logical [B, Hkv, Lk, D]; v: logical
    [B, Hkv, Lk, Dv] (Dv may differ from D; any real dtype, widened exactly).
    mask: broadcastable to [B, Hq, Lq, Lk] for the additive (float values) and
    boolean (nonzero = attend) kinds; the window W for the sliding kind;
    ignored for none and causal.  q_rows restricts the computation to those
    query rows (all rows if None); row indices keep their meaning for the
    causal and sliding masks.
    Returns float64 [B, Hq, len(rows), Dv].
    """
    q, k, v, n_rep, bias = _prepare(q, k, v, mask_kind, mask)
    B, Hq, Lq, D = q.shape
    rows = np.arange(Lq) if q_rows is None else np.asarray(list(q_rows), dtype=np.int64)
    out = np.empty((B, Hq, len(rows), v.shape[-1]), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            s = _scores(q[b, h, rows], k[b, g], scale, bias[b, h][rows])
            out[b, h] = _softmax_rows(s) @ v[b, g]
    return out


def sdpa_strided(q_flat, q_strides, k_flat, k_strides, v_flat, v_strides,
                 batch: int, q_len: int, kv_len: int, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, scale: float, mask_kind: str = "none", mask=None) -> np.ndarray:
    """sdpa() on operands given as flat buffers plus logical (b, h, l, d) strides."""
    q = gather_strided(q_flat, (batch, n_q_heads, q_len, head_dim), q_strides)
    k = gather_strided(k_flat, (batch, n_kv_heads, kv_len, head_dim), k_strides)
    v = gather_strided(v_flat, (batch, n_kv_heads, kv_len, head_dim), v_strides)
    return sdpa(q, k, v, scale, mask_kind, mask)


# --------------------------------------------------------------------------
# Rotary position embedding (applied to Q and K before the scores).
# --------------------------------------------------------------------------
def rope(x, cos, sin, rotary_dim: int, pos0: int = 0) -> np.ndarray:
    """Rotate the first rotary_dim columns of x (logical [..., L, D]) in pairs.

    Row l sits at position pos0 + l.  With R = rotary_dim, h = R / 2 and
    (c, s) = (cos[pos][j], sin[pos][j]) for j < h:
        y[j]     = x[j] * c - x[j + h] * s
        y[j + h] = x[j + h] * c + x[j] * s
    and y[j] = x[j] for j >= R.  float64 throughout.
    """
    x = np.asarray(x, dtype=np.float64)
    R = int(rotary_dim)
    if R == 0:
        return x.copy()
    if R < 0 or R % 2 or R > x.shape[-1]:
        raise ValueError("rotary_dim must be even and at most the head dim")
    h = R // 2
    L = x.shape[-2]
    c = np.asarray(cos, dtype=np.float64)[pos0:pos0 + L, :h]
    s = np.asarray(sin, dtype=np.float64)[pos0:pos0 + L, :h]
    if c.shape[0] != L:
        raise ValueError("the tables do not cover every position")
    y = x.copy()
    a, b = x[..., :h], x[..., h:R]
    y[..., :h] = a * c - b * s
    y[..., h:R] = b * c + a * s
    return y


def rope_tables(n_pos: int, rotary_dim: int, base: float = 10000.0):
    """The usual tables: angle(pos, j) = pos * base ** (-2 j / R), j < R / 2."""
    h = rotary_dim // 2
    inv = base ** (-2.0 * np.arange(h, dtype=np.float64) / rotary_dim)
    ang = np.arange(n_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


# --------------------------------------------------------------------------
# Split-key partial states and their log-sum-exp merge.
# --------------------------------------------------------------------------
def partial_state(q, k, v, scale: float, mask_kind: str, mask, key_lo: int, key_hi: int):
    """Softmax state over keys [key_lo, key_hi) only, for every (b, h, i).

    Returns (acc, m, l) with m = max_j s_ij, l = sum_j exp(s_ij - m) and
    acc = sum_j exp(s_ij - m) V_j over the keys of the range (acc and l are 0
    and m is -inf where every key of the range is masked).  softmax over all
    keys equals merge_states() of the states of any partition of the keys:
    the split-key decode scheme of mlx issue #3885 ("2-pass" vector kernel,
    nkv x blocks threadgroups then a combine) rests on that identity.
    """
    q, k, v, n_rep, bias = _prepare(q, k, v, mask_kind, mask)
    B, Hq, Lq, D = q.shape
    acc = np.zeros((B, Hq, Lq, v.shape[-1]))
    m = np.full((B, Hq, Lq), -np.inf)
    l = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            s = _scores(q[b, h], k[b, g, key_lo:key_hi], scale, bias[b, h][:, key_lo:key_hi])
            if s.shape[1] == 0:
                continue
            mm = s.max(axis=-1)
            live = np.isfinite(mm)
            e = np.where(live[:, None], np.exp(s - np.where(live, mm, 0.0)[:, None]), 0.0)
            m[b, h] = mm
            l[b, h] = e.sum(axis=-1)
            acc[b, h] = e @ v[b, g, key_lo:key_hi]
    return acc, m, l


def merge_states(states) -> np.ndarray:
    """Combine partial (acc, m, l) states: O = sum_s e^(m_s-M) acc_s / sum_s e^(m_s-M) l_s."""
    ms = np.stack([s[1] for s in states])
    big_m = ms.max(axis=0)
    live = np.isfinite(big_m)
    ref = np.where(live, big_m, 0.0)
    num = 0.0
    den = 0.0
    for acc, m, l in states:
        w = np.where(np.isfinite(m), np.exp(np.where(np.isfinite(m), m, 0.0) - ref), 0.0)
        num = num + w[..., None] * acc
        den = den + w * l
    den = np.where(live, den, 1.0)
    return np.where(live[..., None], num / den[..., None], 0.0)


# --------------------------------------------------------------------------
# Brute force: pure-Python loops with exactly rounded sums (tiny shapes only).
# --------------------------------------------------------------------------
def brute_force_sdpa(q, k, v, scale: float, mask_kind: str = "none", mask=None):
    """Same definition as sdpa(), one scalar at a time with math.fsum.

    For shapes of a few elements per axis; it exists to check sdpa() itself.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Lq, D = q.shape
    Hkv, Lk, Dv = k.shape[1], k.shape[2], v.shape[3]
    n_rep = Hq // Hkv
    window = None
    if mask_kind == "sliding":
        window = int(mask)
    elif mask is not None:
        mask = np.broadcast_to(np.asarray(mask), (B, Hq, Lq, Lk))
    out = [[[[0.0] * Dv for _ in range(Lq)] for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // n_rep
            for i in range(Lq):
                scores = []
                for j in range(Lk):
                    s = float(scale) * math.fsum(float(q[b, h, i, d]) * float(k[b, g, j, d]) for d in range(D))
                    if mask_kind == "additive":
                        s += float(mask[b, h, i, j])
                    elif mask_kind == "boolean" and not mask[b, h, i, j]:
                        s = -math.inf
                    elif mask_kind == "causal" and j > i + (Lk - Lq):
                        s = -math.inf
                    elif mask_kind == "sliding" and not (i + (Lk - Lq) - window < j <= i + (Lk - Lq)):
                        s = -math.inf
                    scores.append(s)
                top = max(scores)
                if top == -math.inf:
                    continue
                weights = [math.exp(s - top) if s != -math.inf else 0.0 for s in scores]
                z = math.fsum(weights)
                for d in range(Dv):
                    out[b][h][i][d] = math.fsum(w * float(v[b, g, j, d]) for j, w in enumerate(weights)) / z
    return np.array(out, dtype=np.float64)

