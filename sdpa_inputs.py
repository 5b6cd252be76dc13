"""Seeded synthetic inputs for scaled dot-product attention.

Shared by the oracle's tests and the GPU tests / benchmark.  This module
draws and lays out numbers; it holds none of the attention arithmetic.

Recipe (all configurations):
  * numpy Generator(PCG64(seed)) draws float32 N(0, 1) (times `std`) in the
    order q, k, v, each in its physical layout; the mask is drawn from a
    second generator seeded with seed + 100;
  * half-precision inputs are rounded from those float32 draws by torch on
    the host (round to nearest even), so both sides read the same stored
    values;
  * additive masks hold 0 or -1e9 (Bernoulli(p) for -1e9) in the input
    dtype (bf16 rounds -1e9 to -998244352); boolean masks hold uint8 1
    (attend) or 0 (masked, Bernoulli(p));
  * the deterministic variant of the tiny configuration is the one printed
    in mlx issue "mx.fast.scaled_dot_product_attention produces incorrect
    attention scores (MLX 0.31.2)" [minimal reproduction]: n evenly spaced
    float32 values in [-0.5, 0.5) reshaped row-major to [B, L, H, D], the same
    array for q, k and v.

Tensors are returned as torch CPU tensors of logical shape [B, H, L, D]
(a view over the physical layout: "blhd" storage is transposed into the
logical order without copying).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Case:
    """One attention problem: logical [B,H,L,D] views plus mask and scale."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    scale: float
    mask_kind: str = "none"
    mask: Optional[torch.Tensor] = None
    layout: str = "bhld"
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def dims(self):
        B, Hq, Lq, D = self.q.shape
        return dict(batch=B, n_q_heads=Hq, q_len=Lq, kv_len=self.k.shape[2],
                    n_kv_heads=self.k.shape[1], head_dim=D)


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def logical_view(phys: torch.Tensor, layout: str) -> torch.Tensor:
    """[B,L,H,D] storage -> logical [B,H,L,D] view (no copy); [B,H,L,D] unchanged."""
    if layout == "blhd":
        return phys.transpose(1, 2)
    if layout == "bhld":
        return phys
    raise ValueError(layout)


def _phys_shape(B, H, L, D, layout):
    return (B, L, H, D) if layout == "blhd" else (B, H, L, D)


def linspace_block(shape) -> np.ndarray:
    """n evenly spaced float32 values in [-0.5, 0.5), row-major, as in the page's repro."""
    n = int(np.prod(shape))
    return np.linspace(-0.5, 0.5, n, endpoint=False, dtype=np.float32).reshape(shape)


def make_case(B, Hq, Hkv, Lq, Lk, D, dtype="bf16", layout="bhld", mask_kind="none",
              seed=0, std=1.0, scale=None, mask_p=None, mask_shape="key",
              mask_dtype=None, name="", window=None, dv=None) -> Case:
    """Seeded random case.

    dv: head dim of V (and of the output) when it differs from D.

    window: keys per query for mask_kind="sliding" (kept in meta["window"]).

    mask_shape for additive / boolean masks: "key" -> [1,1,1,Lk];
    "qk" -> [1,1,Lq,Lk]; "full" -> [B,Hq,Lq,Lk].
    mask_p: probability that an entry is masked (additive -1e9 / boolean 0);
    defaults 0.1 (additive) and 0.05 (boolean).
    """
    tdt = DTYPES[dtype]
    g = rng(seed)
    tensors = []
    for H, L, DD in ((Hq, Lq, D), (Hkv, Lk, D), (Hkv, Lk, dv or D)):
        x = g.standard_normal(_phys_shape(B, H, L, DD, layout), dtype=np.float32) * np.float32(std)
        tensors.append(logical_view(torch.from_numpy(x).to(tdt), layout))
    q, k, v = tensors
    if scale is None:
        scale = float(np.float32(D ** -0.5))
    mask = None
    if mask_kind in ("additive", "boolean"):
        gm = rng(seed + 100)
        shp = {"key": (1, 1, 1, Lk), "qk": (1, 1, Lq, Lk), "full": (B, Hq, Lq, Lk)}[mask_shape]
        p = mask_p if mask_p is not None else (0.1 if mask_kind == "additive" else 0.05)
        hit = gm.random(shp, dtype=np.float32) < np.float32(p)
        if mask_kind == "additive":
            mdt = DTYPES[mask_dtype or dtype]
            mask = torch.from_numpy(np.where(hit, np.float32(-1e9), np.float32(0.0))).to(mdt)
        else:
            mask = torch.from_numpy((~hit).astype(np.uint8))
    meta = dict(seed=seed, dtype=dtype, std=std)
    if mask_kind == "sliding":
        if window is None or int(window) < 1:
            raise ValueError("a sliding case needs window >= 1")
        meta["window"] = int(window)
    return Case(q, k, v, float(scale), mask_kind, mask, layout, name, meta)


def tiny_case(variant="random", transposed=False) -> Case:
    """Tiny fp32 full attention: B=2, Lq=Lk=82, Hq=Hkv=8, D=64, [B,L,H,D] storage.

    variant "random": 0.5 * N(0,1) from seed 1; "linspace": the page's
    deterministic array.  transposed=True stores the same logical tensors
    physically as [B,H,L,D] (a permuted copy), so both layouts must give the
    same output.
    """
    B, L, H, D = 2, 82, 8, 64
    if variant == "linspace":
        a = linspace_block((B, L, H, D))
        q, k, v = (logical_view(torch.from_numpy(a.copy()), "blhd") for _ in range(3))
        c = Case(q, k, v, float(np.float32(D ** -0.5)), "none", None, "blhd", "tiny-linspace",
                 dict(seed=None, dtype="f32", std=None))
    else:
        c = make_case(B, H, H, L, L, D, dtype="f32", layout="blhd", seed=1, std=0.5, name="tiny-random")
    if transposed:
        c.q, c.k, c.v = (t.contiguous() for t in (c.q, c.k, c.v))  # logical order becomes the storage order
        c.layout = "bhld"
        c.name += "-bhld"
    return c


DECODE_LENGTHS = (1024, 4096)


def decode_case(head_dim: int, kv_len: int, dtype="bf16") -> Case:
    """bf16 decode, B=1, qL=1, Hq=32, additive [1,1,1,Lk] mask (10% -1e9), [B,H,L,D].

    head_dim 256 -> Hkv=8 (seed 2); head_dim 512 -> Hkv=4 (seed 3).
    """
    hkv, seed = {256: (8, 2), 512: (4, 3)}[head_dim]
    return make_case(1, 32, hkv, 1, kv_len, head_dim, dtype=dtype, layout="bhld",
                     mask_kind="additive", seed=seed, name=f"decode-d{head_dim}-lk{kv_len}")


def prefill72_case(mask_kind="none", seq=8192, dtype="bf16") -> Case:
    """bf16 prefill B=1, Hq=Hkv=16, Lq=Lk=seq, D=72, [B,L,H,D]; none / boolean [1,1,L,L] 5% false / causal."""
    return make_case(1, 16, 16, seq, seq, 72, dtype=dtype, layout="blhd", mask_kind=mask_kind,
                     seed=4, mask_shape="qk", name=f"prefill-d72-{mask_kind}-L{seq}")


def prefill512_case(seq=4096, dtype="bf16") -> Case:
    """bf16 prefill B=1, Hq=32, Hkv=4, D=512, Lq=Lk=seq, causal, [B,H,L,D]."""
    return make_case(1, 32, 4, seq, seq, 512, dtype=dtype, layout="bhld", mask_kind="causal",
                     seed=5, name=f"prefill-d512-causal-L{seq}")


def sliding_case(q_len=4096, kv_len=4096, window=1024, dtype="bf16") -> Case:
    """bf16 sliding-window (local causal) attention with the shapes of the d=256
    local layers named in mlx issue #3885 [Summary]: B=1, Hq=32, Hkv=16, D=256,
    [B,H,L,D]; q_len=1 is a decode step over a kv_len cache (seed 6)."""
    return make_case(1, 32, 16, q_len, kv_len, 256, dtype=dtype, layout="bhld", mask_kind="sliding",
                     seed=6, window=window, name=f"sliding-d256-q{q_len}-k{kv_len}-w{window}")


def decode_dv_case(kv_len=4096, dtype="bf16") -> Case:
    """bf16 decode with the (192, 128) head-dim pairing of the vector kernel in
    mlx issue #3885 [Current routing]: B=1, qL=1, Hq=32, Hkv=8, Q/K head dim 192,
    V head dim 128, additive [1,1,1,Lk] mask (10% -1e9), [B,H,L,D] (seed 7)."""
    return make_case(1, 32, 8, 1, kv_len, 192, dtype=dtype, layout="bhld", mask_kind="additive", seed=7,
                     dv=128, name=f"decode-qk192-v128-lk{kv_len}")


def to_device(case: Case, device="cuda"):
    """Copy a case's physical storage to `device`; return the same logical views (q, k, v, mask)."""
    def dev(t):
        if case.layout == "blhd":
            return t.transpose(1, 2).contiguous().to(device).transpose(1, 2)
        return t.contiguous().to(device)
    q, k, v = dev(case.q), dev(case.k), dev(case.v)
    mask = case.mask.to(device) if case.mask is not None else None
    return q, k, v, mask
