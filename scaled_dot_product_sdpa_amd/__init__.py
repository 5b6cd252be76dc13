"""Fused scaled dot-product attention for AMD Instinct MI355X (gfx950).

    import scaled_dot_product_sdpa_amd as sdpa
    out = sdpa.forward(q, k, v, scale=..., mask=..., mask_kind=...)

The work runs in libsdpa.so (hand-written HIP kernels behind the C ABI in
include/sdpa.h); this package only marshals torch tensors into that ABI.
"""
from ._lib import (  # noqa: F401
    EXPORTS,
    KERNELS,
    MASK_KINDS,
    LIB_PATH,
    SdpaError,
    Strides,
    describe_route,
    dtype_code,
    forward,
    head_dims,
    kernel_timing,
    probe_stream_read,
    load,
    rope,
    route_counters,
    select_kernel,
    workspace_size,
)
