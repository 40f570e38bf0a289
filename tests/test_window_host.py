"""CPU tests of the host side of the token-order entry points: the library's window
segmentation equals the oracle's (bit-exact), and malformed calls of
mgattn_window_segments / mgattn_window_permute / mgattn_rope2d are refused by name
before any GPU call (fake device addresses; every call here is refused)."""
from __future__ import annotations

import pytest

from oracle import window_rope as W
from vit_perception_encoder_amd import mgattn as mg

pytestmark = pytest.mark.cpu


@pytest.fixture(scope="module")
def lib():
    return mg.load_library()


@pytest.mark.parametrize("grids", [[(5, 7)], [(12, 12), (8, 8)], [(64, 64)], [(128, 96), (64, 64), (32, 32)],
                                   [(112, 96), (72, 56), (40, 40)], [(1, 1)], [(3, 200), (200, 3)]])
@pytest.mark.parametrize("win", [1, 3, 8, 32, 1000])
def test_segments_match_oracle(lib, grids, win):
    _, cu = W.window_order(grids, win)
    assert mg.mgattn_window_segments(grids, win) == cu.tolist()


def test_segment_counts_of_the_workloads(lib):
    assert len(mg.mgattn_window_segments([(64, 64)], 32)) - 1 == 4
    assert len(mg.mgattn_window_segments([(128, 96), (64, 64), (32, 32)], 32)) - 1 == 17
    assert len(mg.mgattn_window_segments([(112, 96), (72, 56), (40, 40)], 32)) - 1 == 22


def _seg(grids, win, max_seg=None, null_grids=False):
    import ctypes
    g, n = mg._grid_array(grids)
    buf = (ctypes.c_int32 * 8)()
    return mg.load_library().mgattn_window_segments(None if null_grids else ctypes.cast(g, ctypes.c_void_p), n, win,
                                                    ctypes.cast(buf, ctypes.c_void_p) if max_seg is not None else None,
                                                    max_seg or 0)


def test_segments_refusals(lib):
    assert _seg([(4, 4)], 2, null_grids=True) == -1
    assert _seg([], 2) == -14
    assert _seg([(4, 4)] * 65, 2) == -14
    assert _seg([(0, 4)], 2) == -14
    assert _seg([(4, 4)], 0) == -14
    assert _seg([(8, 8)], 2, max_seg=7) == -12   # 16 segments do not fit 7
    assert _seg([(8, 8)], 4, max_seg=7) == 4
    assert _seg([(50000, 50000)], 32) == -12     # 2.5e9 tokens


A, B = 0x100000, 0x900000


@pytest.mark.parametrize("kw,status", [
    (dict(src=0), -1), (dict(grids=[]), -14), (dict(win=0), -14), (dict(inverse=2), -14),
    (dict(row_bytes=3000), -13), (dict(row_bytes=8), -13), (dict(src=A + 8), -8),
    (dict(dst=A + 16), -7),
])
def test_permute_refusals(lib, kw, status):
    args = dict(src=A, dst=B, row_bytes=3072, grids=[(16, 16)], win=4, inverse=0)
    args.update(kw)
    assert mg.mgattn_window_permute(args["src"], args["dst"], args["row_bytes"], args["grids"], args["win"],
                                    args["inverse"], None, check=False) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), -1), (dict(dtype=3), -2), (dict(grids=[]), -14), (dict(win=-1), -14), (dict(H=0), -4),
    (dict(d=72), -3), (dict(d=8), -3), (dict(d=144), -3), (dict(theta=1.0), -9), (dict(theta=float("inf")), -9),
    (dict(ldx=1535), -13), (dict(ldx=1540), -13), (dict(x=A + 4), -8),
])
def test_rope_refusals(lib, kw, status):
    args = dict(x=A, ldx=1536, grids=[(16, 16)], win=0, H=16, d=96, theta=10000.0, dtype=1)
    args.update(kw)
    assert mg.mgattn_rope2d(args["x"], args["ldx"], args["grids"], args["win"], args["H"], args["d"], args["theta"],
                            args["dtype"], None, check=False) == status
