"""C-ABI checks that need no GPU: exported symbols, the routing predicate,
workspace sizing, status strings and argument validation (every case here is
rejected before the library touches the device)."""
import ctypes
import os
import re

import pytest

import scaled_dot_product_sdpa_amd as sdpa
from scaled_dot_product_sdpa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sdpa.LIB_PATH):
        pytest.fail("libsdpa.so is not built (python -m scaled_dot_product_sdpa_amd.build)")
    return sdpa.load()


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(sdpa_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_header_symbol(lib):
    names = _header_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_head_dims(lib):
    assert sdpa.head_dims() == [64, 72, 80, 96, 128, 256, 512]


@pytest.mark.parametrize("q_len,kernel", [(1, "vector"), (8, "vector"), (9, "full"), (8192, "full")])
def test_route_by_query_length(lib, q_len, kernel):
    k, r, st = sdpa.select_kernel(1, q_len, 4096, 32, 4, 512, 2)
    assert (k, r, st) == (kernel, 0, 0)


@pytest.mark.parametrize("args,reason,status", [
    ((1, 9, 9, 8, 3, 64, 2), 3, -1),        # Hq % Hkv != 0
    ((1, 9, 9, 8, 4, 65, 2), 1, -2),        # head dim not built
    ((1, 9, 9, 8, 4, 192, 0), 1, -2),
    ((1, 9, 9, 8, 4, 64, 3), 2, -2),        # u8 is a mask type only
    ((0, 9, 9, 8, 4, 64, 2), 4, -1),        # empty batch
    ((1, 0, 9, 8, 4, 64, 2), 4, -1),
    ((1, 9, 0, 8, 4, 64, 2), 4, -1),
])
def test_unsupported_is_an_error_with_a_reason(lib, args, reason, status):
    k, r, st = sdpa.select_kernel(*args)
    assert (k, r, st) == ("unsupported", reason, status)


def test_every_dtype_and_head_dim_is_fused(lib):
    for d in sdpa.head_dims():
        for dt in (0, 1, 2):
            for mk in ("none", "additive", "boolean", "causal", "sliding"):
                assert sdpa.select_kernel(2, 100, 100, 8, 2, d, dt, mk)[0] == "full"
                assert sdpa.select_kernel(2, 1, 100, 8, 2, d, dt, mk)[0] == "vector"


def test_value_head_dim_pairing(lib):
    """(192, 128) exists for the 16-bit vector kernel only; other pairings are
    unsupported with their own reason (6)."""
    for dt in (1, 2):
        assert sdpa.select_kernel(1, 1, 4096, 32, 8, 192, dt, "additive", v_head_dim=128) == ("vector", 0, 0)
        assert sdpa.select_kernel(1, 8, 4096, 32, 8, 192, dt, "sliding", v_head_dim=128) == ("vector", 0, 0)
        assert sdpa.select_kernel(1, 9, 4096, 32, 8, 192, dt, "none", v_head_dim=128) == ("unsupported", 6, -2)
    assert sdpa.select_kernel(1, 1, 4096, 32, 8, 192, 0, "none", v_head_dim=128) == ("unsupported", 6, -2)
    assert sdpa.select_kernel(1, 1, 4096, 32, 8, 128, 2, "none", v_head_dim=64) == ("unsupported", 6, -2)
    assert sdpa.select_kernel(1, 1, 4096, 32, 8, 192, 2, "none") == ("unsupported", 1, -2)
    assert sdpa.select_kernel(1, 1, 4096, 32, 8, 128, 2, "none", v_head_dim=128) == ("vector", 0, 0)
    # partial outputs are v_head_dim wide: same plan, 128 / 192 of the fp32 outputs
    a = sdpa.workspace_size(1, 1, 4096, 32, 8, 128, 2)
    b = sdpa.workspace_size(1, 1, 4096, 32, 8, 192, 2, v_head_dim=128)
    assert a == b > 0
    assert sdpa.workspace_size(1, 9, 4096, 32, 8, 192, 2, v_head_dim=128) == 0


def test_describe_route(lib):
    # head dim 512: split + combine kernels (the single-launch kernel stops at 256)
    s = sdpa.describe_route(1, 1, 4096, 32, 4, 512, 2, "additive")
    assert s.startswith("vector bf16 d512 additive") and "splits=" in s, s
    s = sdpa.describe_route(1, 1, 4096, 32, 8, 256, 2, "additive")
    assert s.startswith("vector-fused bf16 d256 additive") and "groups=8 splits=32" in s, s
    # 4 kv heads cannot spread over 8 XCDs: split + combine
    assert sdpa.describe_route(1, 1, 4096, 32, 4, 256, 2, "additive").startswith("vector bf16")
    # 3 kv heads do not spread evenly over the XCDs: split + combine kernels
    s = sdpa.describe_route(1, 1, 4096, 12, 3, 128, 2, "none")
    assert s.startswith("vector bf16 d128 none") and "splits=" in s, s
    # float32 decode always takes the split + combine kernels
    assert sdpa.describe_route(1, 1, 4096, 32, 8, 256, 0, "none").startswith("vector f32")
    s = sdpa.describe_route(1, 8192, 8192, 16, 16, 72, 2, "causal")
    assert s.startswith("full bf16 d72 causal")
    assert sdpa.describe_route(1, 9, 9, 8, 4, 65, 2).startswith("unsupported")
    # a boolean mask on the 16-bit head-dim <= 128 kernel: lane words built by a pre-pass launch
    assert sdpa.describe_route(1, 8192, 8192, 16, 16, 72, 2, "boolean").endswith(" lane-words+prepass")
    assert "lane-words" not in sdpa.describe_route(1, 8192, 8192, 16, 16, 72, 2, "none")
    assert "lane-words" not in sdpa.describe_route(1, 4096, 4096, 32, 4, 512, 2, "boolean")
    assert "lane-words" not in sdpa.describe_route(1, 100, 100, 8, 2, 64, 0, "boolean")


def test_workspace_size(lib):
    align = lambda x: (x + 255) // 256 * 256
    # prefill: the 32 KiB of arrival words every workspace starts with, then room for the lane
    # masks of a boolean mask shared by batch and heads, 32 words (8 bytes) per 32-row block and
    # 64-key tile, where the 16-bit head-dim <= 128 kernel runs
    assert sdpa.workspace_size(1, 100, 100, 8, 2, 64, 2) == 32768 + 4 * 2 * 32 * 8
    assert sdpa.workspace_size(1, 8192, 8192, 16, 16, 72, 2) == 32768 + 256 * 128 * 256   # c4: 8 MiB
    assert sdpa.workspace_size(1, 100, 100, 8, 2, 64, 0) == 0           # fp32 prefill: none
    assert sdpa.workspace_size(1, 100, 100, 8, 2, 256, 2) == 0          # the wide-head kernel: none
    # single-launch decode: 32 KiB of arrival words, then per (group, split, row) one
    # fp32 partial row of the group's V columns and its (max, sum)
    # (a mask tensor without aligned 4-key runs takes the split + combine kernels: the size covers both)
    ws = sdpa.workspace_size(1, 1, 4096, 32, 8, 256, 2)
    route = sdpa.describe_route(1, 1, 4096, 32, 8, 256, 2)
    G, S = (int(re.search(k + r"=(\d+)", route).group(1)) for k in ("groups", "splits"))
    slots = G * S * 4                                                   # 4 query heads per kv head, q_len 1
    fused = 32768 + align(slots * 256 * 4) + align(slots * 2 * 4)
    split_combine = 32768 + align(32 * 64 * 256 * 4) + align(32 * 64 * 2 * 4)
    assert ws == max(fused, split_combine)
    # split + combine: per (query row, split) one fp32 output row and (max, sum); the
    # split count is the largest any key count up to kv_len plans
    ws = sdpa.workspace_size(1, 1, 4096, 24, 3, 128, 2)
    assert sdpa.describe_route(1, 1, 4096, 24, 3, 128, 2).startswith("vector bf16")
    rows, s = 24, 64
    assert ws == 32768 + align(rows * s * 128 * 4) + align(rows * s * 2 * 4)
    assert sdpa.workspace_size(1, 1, 4096, 32, 4, 65, 2) == 0


def test_split_override_changes_the_plan(lib, monkeypatch):
    monkeypatch.setenv("SDPA_DECODE_SPLITS", "3")
    assert "splits=3 " in sdpa.describe_route(1, 1, 4096, 32, 8, 256, 2)


def test_strerror_covers_every_status(lib):
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.sdpa_strerror(st)
    assert lib.sdpa_strerror(-99) == b"unknown status"


def _forward(lib, q=16, k=16, v=16, o=4096, st=None, dims=(1, 16, 16, 2, 2, 64), dt=2, mk=0, mask=None,
             mdt=3, ws=None, wsb=0):
    S = _lib.Strides
    st = st or S(2 * 16 * 64, 16 * 64, 64, 1)
    return lib.sdpa_forward(q, st, k, st, v, st, o, st, *dims, dt, 0.125, mk, mask, S(0, 0, 0, 1), mdt,
                            ws, wsb, None)


def test_forward_rejects_bad_arguments_before_touching_the_gpu(lib):
    before = sdpa.route_counters()
    S = _lib.Strides
    assert _forward(lib, q=None) == -1                                 # null pointer
    assert _forward(lib, dims=(1, 16, 16, 3, 2, 64)) == -1             # groups
    assert _forward(lib, dims=(1, 16, 16, 2, 2, 48)) == -2             # head dim
    assert _forward(lib, st=S(2048, 1024, 64, 2)) == -2                # d stride != 1
    assert _forward(lib, st=S(2048, 1024, 60, 1)) == -2                # row stride not 16-byte aligned
    assert _forward(lib, q=24) == -2                                   # misaligned base
    assert _forward(lib, st=S(-2048, 1024, 64, 1)) == -1               # negative stride
    assert _forward(lib, o=16) == -1                                   # out overlaps q
    assert _forward(lib, mk=1, mask=None) == -1                        # additive without mask
    assert _forward(lib, mk=2, mask=4096 * 64, mdt=2) == -1            # boolean mask must be u8
    assert _forward(lib, mk=1, mask=4096 * 64, mdt=3) == -1            # additive mask can't be u8
    assert _forward(lib, mk=7) == -1                                   # unknown mask kind
    assert _forward(lib, o=1 << 21, dims=(1, 1, 4096, 2, 2, 64), ws=None, wsb=0) == -3  # decode workspace
    assert _forward(lib, mk=4) == -1                                   # sliding needs the window entry point
    st = S(2 * 16 * 64, 16 * 64, 64, 1)
    assert lib.sdpa_forward_sliding(4096, st, 4096, st, 4096, st, 1 << 20, st, 2, 16, 16, 16, 16, 64, 2, 0.125,
                                    0, None, 0, None) == -1            # window < 1
    assert lib.sdpa_forward_sliding(4096, st, 4096, st, 4096, st, 1 << 20, st, 2, 16, 16, 16, 16, 48, 2, 0.125,
                                    4, None, 0, None) == -2            # head dim not built
    after = sdpa.route_counters()
    assert after["calls"] - before["calls"] == 16
    assert after["rejected"] - before["rejected"] == 16
    assert after["calls"] == after["full"] + after["vector"] + after["rejected"]


def test_rope_arguments_are_checked_before_touching_the_gpu(lib):
    S = _lib.Strides
    st = S(2 * 16 * 64, 16 * 64, 64, 1)
    tab = _lib.RopeTable(64, 4096, 8192, 32)

    def ex(table, dt=2, pos0=0, d=64):
        return lib.sdpa_forward_ex(4096, st, 4096, st, 4096, st, 1 << 20, st, 2, 16, 16, 16, 16, d, d, dt, 0.125,
                                   3, None, S(0, 0, 0, 0), 0, 0, ctypes.byref(table), pos0, None, 0, None)
    assert ex(_lib.RopeTable(33, 4096, 8192, 32)) == -2               # odd rotary_dim
    assert ex(_lib.RopeTable(-2, 4096, 8192, 32)) == -2               # negative rotary_dim
    assert ex(_lib.RopeTable(128, 4096, 8192, 32)) == -2              # rotary_dim > head_dim
    assert ex(_lib.RopeTable(64, None, 8192, 32)) == -1               # missing table
    assert ex(tab, pos0=17) == -1                                     # positions past the table
    assert ex(tab, pos0=-1) == -1
    assert ex(_lib.RopeTable(64, 4100, 8192, 32)) == -2               # table not 16-byte aligned
    rope = lambda t, **kw: lib.sdpa_rope(4096, st, kw.get("y", 1 << 20), st, 2, 16, 16, 64, kw.get("dt", 2),
                                         ctypes.byref(t), kw.get("pos0", 0), None)
    assert rope(_lib.RopeTable(7, 4096, 8192, 32)) == -1              # odd rotary_dim
    assert rope(_lib.RopeTable(66, 4096, 8192, 32)) == -1             # wider than the head
    assert rope(tab, pos0=20) == -1                                   # positions past the table
    assert rope(tab, y=4096 + 64) == -1                               # partial overlap of x and y
    assert rope(tab, dt=3) == -2                                      # u8 is a mask type only


# causal prefill grids: the route names the tile shape and whether row tiles pair
def test_causal_small_grids_route(lib):
    import torch
    import scaled_dot_product_sdpa_amd as sdpa
    route = lambda h, d: sdpa.describe_route(1, 4096, 4096, h, h, d, torch.bfloat16, "causal")
    # 32 heads at D = 256: 256-row workgroups, paired
    assert "waves=8x1" in route(32, 256) and "causal-pairs" in route(32, 256)
    # 16 heads: 256-row workgroups could not pair without idling CUs; 128-row ones pair
    assert "waves=4x1" in route(16, 256) and "causal-pairs" in route(16, 256)
    # 8 heads: 128-row workgroups fill the CUs unpaired
    assert "waves=4x1" in route(8, 256) and "causal-pairs" not in route(8, 256)
    # D = 512 has no smaller variant: 8 heads stay unpaired on 256 workgroups
    assert "waves=8x2" in route(8, 512) and "causal-pairs" not in route(8, 512)
