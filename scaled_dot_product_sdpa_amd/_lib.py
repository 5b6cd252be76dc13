"""ctypes binding of libsdpa.so (include/sdpa.h).  Argument marshalling only.

torch supplies device memory and the current stream; every step of the
attention runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a shape is unsupported, the call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdpa.so")

SDPA_F32, SDPA_F16, SDPA_BF16, SDPA_U8 = 0, 1, 2, 3
MASK_KINDS = {"none": 0, "additive": 1, "boolean": 2, "causal": 3, "sliding": 4}
KERNELS = {0: "unsupported", 1: "full", 2: "vector"}
STATUS = {0: "SDPA_OK", -1: "SDPA_EINVAL", -2: "SDPA_EUNSUPPORTED", -3: "SDPA_EWORKSPACE",
          -4: "SDPA_ELAUNCH", -5: "SDPA_EHIP"}
_TORCH_DT = {torch.float32: SDPA_F32, torch.float16: SDPA_F16, torch.bfloat16: SDPA_BF16,
             torch.uint8: SDPA_U8, torch.bool: SDPA_U8}

# Every symbol include/sdpa.h declares (checked by the CPU test suite).
EXPORTS = ("sdpa_forward", "sdpa_forward_sliding", "sdpa_forward_ex", "sdpa_rope", "sdpa_select_kernel",
           "sdpa_select_kernel_ex", "sdpa_describe_route", "sdpa_describe_route_ex", "sdpa_workspace_size",
           "sdpa_workspace_size_ex",
           "sdpa_head_dims", "sdpa_strerror", "sdpa_last_hip_error", "sdpa_route_counters",
           "sdpa_timing_start", "sdpa_timing_stop", "sdpa_probe_stream_read", "sdpa_forward_noalloc",
           "sdpa_noalloc_scratch_bytes")


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("l", ctypes.c_int64), ("d", ctypes.c_int64)]


class RopeTable(ctypes.Structure):
    _fields_ = [("rotary_dim", ctypes.c_int), ("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p),
                ("n_pos", ctypes.c_int)]


class SdpaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_strerror(status)})")


_lib = None
_lock = threading.Lock()


def load(path: str = LIB_PATH):
    """Load libsdpa.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} not found: build it with `python -m scaled_dot_product_sdpa_amd.build`")
        lib = ctypes.CDLL(path)
        i, i64, sz, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
        lib.sdpa_forward.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                     i, i, i, i, i, i, i, ctypes.c_float, i, vp, Strides, i, vp, sz, vp]
        lib.sdpa_forward.restype = i
        lib.sdpa_forward_sliding.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                             i, i, i, i, i, i, i, ctypes.c_float, i, vp, sz, vp]
        lib.sdpa_forward_sliding.restype = i
        lib.sdpa_forward_ex.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                        i, i, i, i, i, i, i, i, ctypes.c_float, i, vp, Strides, i, i,
                                        ctypes.POINTER(RopeTable), i, vp, sz, vp]
        lib.sdpa_rope.argtypes = [vp, Strides, vp, Strides, i, i, i, i, i, ctypes.POINTER(RopeTable), i, vp]
        lib.sdpa_rope.restype = i
        lib.sdpa_forward_ex.restype = i
        dims = [i, i, i, i, i, i, i]
        lib.sdpa_select_kernel.argtypes = dims + [i, ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.sdpa_select_kernel.restype = i
        lib.sdpa_describe_route.argtypes = dims + [i, ctypes.c_char_p, sz]
        lib.sdpa_describe_route.restype = i
        lib.sdpa_describe_route_ex.argtypes = dims + [i, i, ctypes.c_char_p, sz]
        lib.sdpa_describe_route_ex.restype = i
        lib.sdpa_workspace_size.argtypes = dims
        lib.sdpa_workspace_size.restype = sz
        lib.sdpa_select_kernel_ex.argtypes = dims + [i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        lib.sdpa_select_kernel_ex.restype = i
        lib.sdpa_workspace_size_ex.argtypes = dims + [i]
        lib.sdpa_workspace_size_ex.restype = sz
        lib.sdpa_head_dims.argtypes = [ctypes.POINTER(i), i]
        lib.sdpa_head_dims.restype = i
        lib.sdpa_strerror.argtypes = [i]
        lib.sdpa_strerror.restype = ctypes.c_char_p
        lib.sdpa_last_hip_error.argtypes = []
        lib.sdpa_last_hip_error.restype = i
        lib.sdpa_route_counters.argtypes = [ctypes.POINTER(ctypes.c_uint64), i]
        lib.sdpa_route_counters.restype = i
        lib.sdpa_timing_start.argtypes = [i]
        lib.sdpa_timing_start.restype = i
        lib.sdpa_timing_stop.argtypes = [ctypes.POINTER(ctypes.c_float), i]
        lib.sdpa_timing_stop.restype = i
        lib.sdpa_probe_stream_read.argtypes = [vp, sz, vp, vp]
        lib.sdpa_probe_stream_read.restype = i
        lib.sdpa_forward_noalloc.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                             i, i, i, i, i, i, i, i, ctypes.c_float, i, vp, Strides, i, i,
                                             ctypes.POINTER(RopeTable), i, vp]
        lib.sdpa_forward_noalloc.restype = i
        lib.sdpa_noalloc_scratch_bytes.argtypes = []
        lib.sdpa_noalloc_scratch_bytes.restype = sz
        _lib = lib
        return lib


def _strerror(status: int) -> str:
    try:
        return load().sdpa_strerror(status).decode()
    except Exception:  # library not loadable: the status name is enough
        return "?"


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _TORCH_DT:
        raise SdpaError(-2, f"dtype {dt}")
    return _TORCH_DT[dt]


def select_kernel(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, dtype, mask_kind="none",
                  v_head_dim=None):
    """(kernel name, reason code, status) from the library's routing predicate."""
    k, r = ctypes.c_int(), ctypes.c_int()
    if v_head_dim is None:
        st = load().sdpa_select_kernel(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim,
                                       _as_code(dtype), MASK_KINDS[mask_kind], ctypes.byref(k), ctypes.byref(r))
    else:
        st = load().sdpa_select_kernel_ex(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim,
                                          _as_code(dtype), MASK_KINDS[mask_kind], ctypes.byref(k), ctypes.byref(r))
    return KERNELS[k.value], r.value, st


def describe_route(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, dtype, mask_kind="none",
                   v_head_dim=None) -> str:
    buf = ctypes.create_string_buffer(512)
    if v_head_dim is None:
        load().sdpa_describe_route(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, _as_code(dtype),
                                   MASK_KINDS[mask_kind], buf, len(buf))
    else:
        load().sdpa_describe_route_ex(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim,
                                      _as_code(dtype), MASK_KINDS[mask_kind], buf, len(buf))
    return buf.value.decode()


def workspace_size(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, dtype, v_head_dim=None) -> int:
    if v_head_dim is None:
        return int(load().sdpa_workspace_size(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim,
                                              _as_code(dtype)))
    return int(load().sdpa_workspace_size_ex(batch, q_len, kv_len, n_q_heads, n_kv_heads, head_dim, v_head_dim,
                                             _as_code(dtype)))


def head_dims() -> list:
    n = load().sdpa_head_dims(None, 0)
    arr = (ctypes.c_int * n)()
    load().sdpa_head_dims(arr, n)
    return list(arr)


def route_counters() -> dict:
    arr = (ctypes.c_uint64 * 4)()
    load().sdpa_route_counters(arr, 4)
    return dict(zip(("calls", "full", "vector", "rejected"), (int(x) for x in arr)))


class kernel_timing:
    """Context manager: per-kernel milliseconds of the sdpa_forward calls made inside it.

    with kernel_timing(n) as t: ...calls...;  t.ms -> [(attention_ms, combine_ms), ...]
    """

    def __init__(self, max_calls: int):
        self.max_calls = max_calls
        self.ms = []

    def __enter__(self):
        st = load().sdpa_timing_start(self.max_calls)
        if st != 0:
            raise SdpaError(st, "sdpa_timing_start")
        return self

    def __exit__(self, *exc):
        buf = (ctypes.c_float * (2 * self.max_calls))()
        n = load().sdpa_timing_stop(buf, len(buf))
        if n < 0:
            raise SdpaError(n, "sdpa_timing_stop")
        self.ms = [(buf[2 * i], buf[2 * i + 1]) for i in range(n)]
        return False


def probe_stream_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """One launch of the library's plain streaming read over src's bytes (diagnostics)."""
    st = load().sdpa_probe_stream_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                                       torch.cuda.current_stream(src.device).cuda_stream)
    if st != 0:
        raise SdpaError(st, "sdpa_probe_stream_read")


def _as_code(dtype) -> int:
    return dtype if isinstance(dtype, int) else dtype_code(dtype)


def _strides(t: torch.Tensor) -> Strides:
    s = t.stride()
    return Strides(*[0 if t.shape[i] == 1 else s[i] for i in range(4)])


def _mask_view(mask: torch.Tensor, shape) -> torch.Tensor:
    """Broadcast a mask to logical [B, Hq, Lq, Lk] without copying (zero strides)."""
    while mask.dim() < 4:
        mask = mask.unsqueeze(0)
    return mask.expand(*shape)


_ws_cache: dict = {}


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        # zero-filled once: its leading arrival words must start at zero (every call leaves them zero)
        buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, scale: Optional[float] = None,
            mask: Optional[torch.Tensor] = None, mask_kind: Optional[str] = None,
            out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            layout: str = "bhld", window: Optional[int] = None, rope=None,
            q_pos0: Optional[int] = None, no_alloc: bool = False) -> torch.Tensor:
    """softmax(scale * q k^T + mask) v on the GPU through libsdpa.so.

    q: [B, Hq, Lq, D], k: [B, Hkv, Lk, D], v: [B, Hkv, Lk, Dv] in logical order (any strides,
    e.g. a transposed view of [B, L, H, D] storage); with layout="blhd" they
    are given in [B, L, H, D] order instead and the result is too.
    mask: broadcastable to [B, Hq, Lq, Lk]; bool/uint8 -> boolean, float ->
    additive; mask_kind="causal" needs no tensor; mask_kind="sliding" takes
    `window` (the number of most recent keys each query attends, >= 1).
    rope: (cos, sin, rotary_dim) rotates Q inside the kernels (K must already
    be rotated, e.g. by rope() below); query row i sits at position
    q_pos0 + i, q_pos0 defaulting to Lk - Lq.
    no_alloc: call sdpa_forward_noalloc (the library's static scratch instead of
    a workspace; pass `out` as well for a call that allocates nothing at all).
    """
    lib = load()
    if layout == "blhd":
        q, k, v = q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2)
        if out is not None:
            out = out.transpose(1, 2)
    elif layout != "bhld":
        raise ValueError(layout)
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise SdpaError(-1, "q, k, v must be device tensors")
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise SdpaError(-1, "q, k, v must be 4-D")
    B, Hq, Lq, D = q.shape
    _, Hkv, Lk, _ = k.shape
    Dv = v.shape[3]
    if k.shape[0] != B or k.shape[3] != D or tuple(v.shape[:3]) != tuple(k.shape[:3]):
        raise SdpaError(-1, f"shapes q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise SdpaError(-1, "q, k, v dtypes differ")
    dt = dtype_code(q.dtype)
    if scale is None:
        scale = D ** -0.5
    if mask_kind is None:
        mask_kind = "none" if mask is None else ("boolean" if mask.dtype in (torch.bool, torch.uint8) else "additive")
    mk = MASK_KINDS[mask_kind]
    mptr, mst, mdt = None, Strides(0, 0, 0, 0), 0
    if mask_kind in ("additive", "boolean"):
        if mask is None:
            raise SdpaError(-1, f"mask_kind={mask_kind} needs a mask")
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        mask = _mask_view(mask, (B, Hq, Lq, Lk))
        if not mask.is_cuda:
            raise SdpaError(-1, "mask must be a device tensor")
        mptr, mst, mdt = mask.data_ptr(), _strides(mask), dtype_code(mask.dtype)
    if out is None:
        out = torch.empty((B, Hq, Lq, Dv), dtype=q.dtype, device=q.device)
    if no_alloc:
        table = _rope_table(*rope, device=q.device) if rope is not None else None
        if q_pos0 is None:
            q_pos0 = Lk - Lq
        st = lib.sdpa_forward_noalloc(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(),
                                      _strides(v), out.data_ptr(), _strides(out), B, Lq, Lk, Hq, Hkv, D, Dv, dt,
                                      float(scale), mk, mptr, mst, mdt, int(window or 0),
                                      ctypes.byref(table) if table is not None else None, int(q_pos0),
                                      torch.cuda.current_stream(q.device).cuda_stream)
        if st != 0:
            raise SdpaError(st, f"sdpa_forward_noalloc(B={B}, Lq={Lq}, Lk={Lk}, Hq={Hq}, Hkv={Hkv}, D={D})")
        return out.transpose(1, 2) if layout == "blhd" else out
    nbytes = lib.sdpa_workspace_size_ex(B, Lq, Lk, Hq, Hkv, D, Dv, dt)
    if workspace is None:
        workspace = _workspace(nbytes, q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wlen = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if Dv != D or rope is not None:
        table = None
        if rope is not None:
            table = _rope_table(*rope, device=q.device)
        if q_pos0 is None:
            q_pos0 = Lk - Lq
        st = lib.sdpa_forward_ex(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
                                 out.data_ptr(), _strides(out), B, Lq, Lk, Hq, Hkv, D, Dv, dt, float(scale),
                                 mk, mptr, mst, mdt, int(window or 0),
                                 ctypes.byref(table) if table is not None else None, int(q_pos0), wptr, wlen, stream)
    elif mask_kind == "sliding":
        if window is None:
            raise SdpaError(-1, "mask_kind=sliding needs window")
        st = lib.sdpa_forward_sliding(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(),
                                      _strides(v), out.data_ptr(), _strides(out), B, Lq, Lk, Hq, Hkv, D, dt,
                                      float(scale), int(window), wptr, wlen, stream)
    else:
        st = lib.sdpa_forward(q.data_ptr(), _strides(q), k.data_ptr(), _strides(k), v.data_ptr(), _strides(v),
                              out.data_ptr(), _strides(out), B, Lq, Lk, Hq, Hkv, D, dt, float(scale),
                              mk, mptr, mst, mdt, wptr, wlen, stream)
    if st != 0:
        raise SdpaError(st, f"sdpa_forward(B={B}, Lq={Lq}, Lk={Lk}, Hq={Hq}, Hkv={Hkv}, D={D}, {q.dtype}, "
                            f"{mask_kind})")
    return out.transpose(1, 2) if layout == "blhd" else out


def _rope_table(cos: torch.Tensor, sin: torch.Tensor, rotary_dim: int, device=None) -> RopeTable:
    """cos / sin: device float32 [n_pos, rotary_dim / 2], row-major."""
    for t in (cos, sin):
        if t.dtype != torch.float32 or not t.is_cuda or t.dim() != 2 or not t.is_contiguous():
            raise SdpaError(-1, "rope tables must be contiguous float32 device tensors [n_pos, rotary_dim / 2]")
        if t.shape[1] != rotary_dim // 2 or t.shape != cos.shape:
            raise SdpaError(-1, f"rope tables {tuple(t.shape)} do not match rotary_dim {rotary_dim}")
    return RopeTable(int(rotary_dim), cos.data_ptr(), sin.data_ptr(), int(cos.shape[0]))


def rope(x: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, rotary_dim: int, *, pos0: int = 0,
         out: Optional[torch.Tensor] = None, layout: str = "bhld") -> torch.Tensor:
    """Rotary embedding of x ([B, H, L, D], or [B, L, H, D] with layout="blhd")
    through libsdpa.so: columns [0, rotary_dim) turn in (j, j + rotary_dim/2)
    pairs by the table angles of position pos0 + l.  out=x rotates in place."""
    lib = load()
    if layout == "blhd":
        x = x.transpose(1, 2)
        if out is not None:
            out = out.transpose(1, 2)
    elif layout != "bhld":
        raise ValueError(layout)
    if out is None:
        out = torch.empty_like(x)
    if not x.is_cuda or x.dim() != 4 or tuple(out.shape) != tuple(x.shape) or out.dtype != x.dtype:
        raise SdpaError(-1, "rope: x and out must be 4-D device tensors of one shape and dtype")
    B, H, L, D = x.shape
    table = _rope_table(cos, sin, rotary_dim)
    st = lib.sdpa_rope(x.data_ptr(), _strides(x), out.data_ptr(), _strides(out), B, H, L, D, dtype_code(x.dtype),
                       ctypes.byref(table), int(pos0), torch.cuda.current_stream(x.device).cuda_stream)
    if st != 0:
        raise SdpaError(st, f"sdpa_rope(B={B}, H={H}, L={L}, D={D}, R={rotary_dim}, pos0={pos0})")
    return out.transpose(1, 2) if layout == "blhd" else out
