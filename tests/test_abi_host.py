"""C-ABI checks that need no GPU: the library loads, exports every entry point declared in
include/moe.h, and its pure host functions (workspace layout, shape validation, block-M
choice) behave as documented.  No device work is enqueued here."""
import ctypes
import os
import re

import pytest

import oracle
import token_dispatch_grouped_route_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    names = declared_functions()
    assert len(names) >= 15
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), "missing export " + n
    assert sorted(moe.ENTRY_POINTS) == names


def test_status_strings():
    L = moe.lib()
    for code in range(0, -9, -1):
        assert L.moe_status_string(code) and L.moe_status_string(code) != b"unknown status"
    assert L.moe_status_string(5) == b"unknown status"


@pytest.mark.parametrize("train", [0, 1])
@pytest.mark.parametrize("cfg", [(256, 256, 128, 8, 8, 2), (8192, 7168, 2048, 256, 32, 8),
                                 (4096, 7168, 3072, 384, 48, 6), (0, 256, 128, 8, 8, 2)])
@pytest.mark.parametrize("bm", [32, 64, 128, 256])
def test_workspace_layout(cfg, bm, train):
    T, H, I, E, EL, k = cfg
    s = moe.make_shape(T, H, I, E, EL, k, block_m=bm, train=train)
    L = moe.workspace_layout(s)
    # the static row bound agrees with the oracle's own statement of it
    assert L["rows_capacity"] == oracle.rows_capacity(T, k, EL, bm)
    assert L["num_blocks"] * bm == L["rows_capacity"]
    R = L["rows_capacity"]
    sizes = {"counts": 4 * EL, "padded_offsets": 4 * (EL + 1), "row_pair": 4 * R, "pair_row": 4 * T * k,
             "tile_expert": 4 * (R // bm), "tok_nloc": 4 * T, "meta": 16, "act": 2 * R * I, "stage": 4 * R * H}
    if train:
        sizes.update(hgu=8 * R * I, dact=4 * R * I, dhgu=4 * R * I, dhgu_lo=4 * R * I, wact=2 * R * I,
                     wact_lo=2 * R * I, dtw_part=4 * R * (I // 128))
    sizes["tile_sync"] = 4 * 512
    spans = sorted((L[n], L[n] + sz, n) for n, sz in sizes.items())
    for (a0, a1, na), (b0, b1, nb) in zip(spans, spans[1:]):
        assert a1 <= b0, (na, nb)
    for n in sizes:
        assert L[n] % 256 == 0
    assert L["total_bytes"] >= spans[-1][1] and L["scratch"] + 4 <= L["total_bytes"]
    assert moe.workspace_bytes(s) == L["total_bytes"]
    assert moe.packed_sizes(s) == ((EL, 2 * I * H), (EL, H * I))


@pytest.mark.parametrize("field,value,code", [
    ("block_m", 48, -3), ("block_m", 0, -3), ("H", 100, -2), ("I", 96, -2), ("I", 192, -2), ("EL", 0, -2),
    ("EL", 1025, -2), ("k", 0, -2), ("k", 33, -2), ("T", -1, -2), ("e_lo", 250, -2), ("E", 0, -2),
])
def test_shape_validation(field, value, code):
    s = moe.make_shape(256, 256, 128, 256, 8, 2, block_m=64)
    setattr(s, field, value)
    L = moe.WsLayout()
    assert moe.lib().moe_workspace_layout(ctypes.byref(s), ctypes.byref(L)) == code
    assert moe.lib().moe_workspace_bytes(ctypes.byref(s)) == 0


def test_intermediate_size_is_a_multiple_of_128():
    for train in (0, 1):
        s = moe.make_shape(64, 256, 192, 8, 8, 2, block_m=64, train=train)
        assert moe.lib().moe_workspace_bytes(ctypes.byref(s)) == 0
        s.I = 256
        assert moe.lib().moe_workspace_bytes(ctypes.byref(s)) > 0


def test_null_arguments_are_rejected_before_any_launch():
    L = moe.lib()
    assert L.moe_workspace_layout(None, None) == -1
    s = moe.make_shape(256, 256, 128, 8, 8, 2, block_m=64)
    assert L.moe_route_prologue(ctypes.byref(s), None, None, 0, None) == -1
    assert L.moe_forward(None, None, None, None, None, None, None, 0, None, None) == -1


def test_preferred_block_m():
    pick = lambda T, E, k: moe.preferred_block_m(moe.make_shape(T, 256, 128, E, 8, k, block_m=64))
    assert pick(8192, 256, 8) == 128     # 256 rows per expert on average
    assert pick(4096, 64, 6) == 128      # 384
    assert pick(4096, 384, 6) == 64      # 64
    assert pick(65536, 256, 8) == 256    # 2048
