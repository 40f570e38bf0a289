"""Pins of the window-order / 2D-RoPE oracle (oracle/window_rope.py) to what the pages
and the mathematics fix, and a mutation battery: each plausible slip in the oracle
(axis swap, 0-based positions, wrong sign or frequency, walk order, missing clip or
image offset, wrong inverse) must fail at least one pin.

Pages: vllm.cpp issue #1545 (second comment: 32x32-patch windows cut by the sparse
permutation; section "Labelled uncertainty": the tower's test images are 12x12 and
8x8 patches), vllm.cpp PR #1579 (body: 12 attention calls over that fixture's
segmentation, 5 window + 2 full + 5 window), vllm.cpp PR #279 (vision-tower commits:
width-first 2D RoPE, 1-based positions, block walk order and within-block order,
inverse permutation before the final LayerNorm).  The unstated orders and the RoPE
formula are readings, stated in oracle/window_rope.py; the pins below check the
oracle against those readings by independent means (hand-derived fixture, geometry
of the segments, closed-form angles via atan2, rotation invariants)."""
from __future__ import annotations

import json
import math
import types
from pathlib import Path

import numpy as np
import pytest

from oracle import window_rope as W

pytestmark = pytest.mark.cpu
ROOT = Path(__file__).resolve().parent.parent
SRC = (ROOT / "oracle" / "window_rope.py").read_text()
GOLDEN = json.loads((ROOT / "tests" / "golden" / "window_order_5x7_win3.json").read_text())
GRIDS = [[(5, 7)], [(12, 12), (8, 8)], [(64, 64)], [(40, 40), (33, 65), (1, 9)], [(112, 96), (72, 56), (40, 40)]]


# ------------------------------------------------------------------ window order pins

def pin_golden_5x7(w):
    perm, cu = w.window_order(GOLDEN["grids"], GOLDEN["win"])
    assert list(perm) == GOLDEN["perm"] and list(cu) == GOLDEN["cu_seqlens"]


def pin_fixture_segment_counts(w):
    """The pages' fixture: images of 12x12 and 8x8 patches; a window layer makes 5
    attention calls and a full layer 2.  Windows of 8..11 give 5; 12 or more give 2."""
    for win in (8, 9, 10, 11):
        assert len(w.window_order([(12, 12), (8, 8)], win)[1]) - 1 == 5
    for win in (12, 32):
        assert len(w.window_order([(12, 12), (8, 8)], win)[1]) - 1 == 2


def pin_segments_are_clipped_blocks(w):
    """Every segment is one win x win block of one image, clipped at the edges, the
    blocks of an image in row-major order, tokens row-major inside; perm is a bijection."""
    for grids in GRIDS:
        for win in (1, 3, 8, 32):
            perm, cu = w.window_order(grids, win)
            T = sum(gh * gw for gh, gw in grids)
            assert sorted(perm.tolist()) == list(range(T))
            blocks = []
            base = 0
            for gh, gw in grids:
                for by in range(math.ceil(gh / win)):
                    for bx in range(math.ceil(gw / win)):
                        ys = range(by * win, min(by * win + win, gh))
                        xs = range(bx * win, min(bx * win + win, gw))
                        blocks.append([base + y * gw + x for y in ys for x in xs])
                base += gh * gw
            assert len(cu) - 1 == len(blocks)
            for g, blk in enumerate(blocks):
                assert perm[cu[g]:cu[g + 1]].tolist() == blk


def pin_identity_cases(w):
    for grids in GRIDS:
        T = sum(gh * gw for gh, gw in grids)
        perm, cu = w.window_order(grids, max(max(g) for g in grids))
        assert perm.tolist() == list(range(T))
        assert cu.tolist() == [0] + list(np.cumsum([gh * gw for gh, gw in grids]))
        perm1, cu1 = w.window_order(grids, 1)
        assert perm1.tolist() == list(range(T)) and cu1.tolist() == list(range(T + 1))


def pin_round_trip(w):
    rng = np.random.default_rng(3)
    for grids in GRIDS[:4]:
        T = sum(gh * gw for gh, gw in grids)
        x = rng.standard_normal((T, 5))
        for win in (3, 32):
            xw = w.to_window_order(x, grids, win)
            assert not np.array_equal(xw, x) or T <= win * win
            assert np.array_equal(w.to_raster_order(xw, grids, win), x)


# ----------------------------------------------------------------------- RoPE pins

H_, D_ = 2, 16


def _rope(w, x, grids, win=0):
    return w.rope2d(x, grids, win, H_, D_, 10000.0)


def pin_rotation_preserves_pair_norms(w):
    rng = np.random.default_rng(5)
    grids = [(6, 9)]
    x = rng.standard_normal((54, H_ * D_))
    y = _rope(w, x, grids)
    nx = np.hypot(x[:, 0::2], x[:, 1::2])
    ny = np.hypot(y[:, 0::2], y[:, 1::2])
    assert np.abs(nx - ny).max() < 1e-12
    assert np.abs(x - y).max() > 0.1


def pin_angles_closed_form(w):
    """A unit vector (1, 0) in pair i of the width half of a patch at column x ends at
    angle (x+1) * theta^(-4i/d); in the height half at (y+1) * theta^(-4i/d)."""
    gh, gw = 4, 7
    x = np.zeros((gh * gw, H_ * D_))
    x[:, 0::2] = 1.0
    y = _rope(w, x, [(gh, gw)])
    for r in range(gh):
        for c in range(gw):
            t = r * gw + c
            for h in range(H_):
                for i in range(D_ // 4):
                    wi = 10000.0 ** (-4.0 * i / D_)
                    for first, pos in ((0, c + 1), (D_ // 2, r + 1)):
                        ch = h * D_ + first + 2 * i
                        got = W.angle_of_pair((y[t, ch], y[t, ch + 1]))
                        want = (pos * wi) % (2 * math.pi)
                        assert min(abs(got - want), 2 * math.pi - abs(got - want)) < 1e-9


def pin_width_first_axis_separation(w):
    rng = np.random.default_rng(7)
    gh, gw = 5, 6
    v = rng.standard_normal(H_ * D_)
    y = _rope(w, np.tile(v, (gh * gw, 1)), [(gh, gw)]).reshape(gh, gw, H_, D_)
    # same column -> same first half; same row -> same second half
    assert np.abs(y[0, 3, :, :D_ // 2] - y[4, 3, :, :D_ // 2]).max() < 1e-12
    assert np.abs(y[2, 0, :, D_ // 2:] - y[2, 5, :, D_ // 2:]).max() < 1e-12
    assert np.abs(y[0, 3, :, D_ // 2:] - y[4, 3, :, D_ // 2:]).max() > 1e-3


def roformer_1d(x, m, base=10000.0):
    """1D rotary position embedding as RoFormer defines it (Su et al., 2021, "RoFormer:
    Enhanced Transformer with Rotary Position Embedding", section 3.4.2, the
    element-wise form of the rotary matrix product): for a vector x of even length n
    at position m, with theta_i = base^(-2(i-1)/n) for i = 1 .. n/2,
        R x = x * (cos m theta_1, cos m theta_1, cos m theta_2, cos m theta_2, ...)
            + (-x_2, x_1, -x_4, x_3, ...) * (sin m theta_1, sin m theta_1, ...).
    RoFormer rotates ADJACENT channel pairs (x_1, x_2), (x_3, x_4), ... (1-based); the
    tower's reading is the same adjacent pairing (not the split-halves pairing of
    x_i with x_(i+n/2)).  Written independently of the oracle: x is [..., n], m is
    broadcast against x's leading axes."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    i = np.arange(1, n // 2 + 1, dtype=np.float64)
    theta = base ** (-2.0 * (i - 1.0) / n)
    ang = np.asarray(m, dtype=np.float64)[..., None] * np.repeat(theta, 2)
    swapped = np.empty_like(x)
    swapped[..., 0::2] = -x[..., 1::2]
    swapped[..., 1::2] = x[..., 0::2]
    return x * np.cos(ang) + swapped * np.sin(ang)


def pin_roformer_per_axis(w):
    """Width-first 2D RoPE = RoFormer's 1D RoPE applied per axis on half the channels:
    channels [0, d/2) of every head are RoFormer-rotated (dimension n = d/2) at
    position column + 1, channels [d/2, d) at row + 1.  So a 1 x W grid's width half is
    exactly the 1D rotation at x + 1, and an H x 1 grid's height half the 1D rotation
    at y + 1.  Pins the frequency schedule, the pairing, the sign and the 1-based
    positions against a published definition."""
    rng = np.random.default_rng(17)
    for gh, gw in ((1, 11), (9, 1), (5, 7)):
        T = gh * gw
        x = rng.standard_normal((T, H_ * D_))
        y = _rope(w, x, [(gh, gw)]).reshape(T, H_, D_)
        xs = x.reshape(T, H_, D_)
        rows = np.repeat(np.arange(gh), gw)[:, None] * np.ones((1, H_))
        cols = np.tile(np.arange(gw), gh)[:, None] * np.ones((1, H_))
        want_w = roformer_1d(xs[:, :, :D_ // 2], cols + 1)
        want_h = roformer_1d(xs[:, :, D_ // 2:], rows + 1)
        assert np.abs(y[:, :, :D_ // 2] - want_w).max() < 1e-12
        assert np.abs(y[:, :, D_ // 2:] - want_h).max() < 1e-12
    # also at the tower's head size (96 channels: 24 frequencies per axis)
    x = rng.standard_normal((6, 96))
    y = w.rope2d(x, [(2, 3)], 0, 1, 96, 10000.0)
    r, c = np.repeat(np.arange(2), 3), np.tile(np.arange(3), 2)
    assert np.abs(y[:, :48] - roformer_1d(x[:, :48], c + 1)).max() < 1e-12
    assert np.abs(y[:, 48:] - roformer_1d(x[:, 48:], r + 1)).max() < 1e-12


def pin_relative_position(w):
    """<R(p1) q, R(p2) k> is unchanged when both patches move by the same offset."""
    rng = np.random.default_rng(11)
    gh, gw = 9, 9
    q, k = rng.standard_normal(H_ * D_), rng.standard_normal(H_ * D_)
    Q = _rope(w, np.tile(q, (gh * gw, 1)), [(gh, gw)])
    K = _rope(w, np.tile(k, (gh * gw, 1)), [(gh, gw)])
    (y1, x1), (y2, x2), (dy, dx) = (1, 2), (4, 0), (3, 5)
    a = Q[y1 * gw + x1] @ K[y2 * gw + x2]
    b = Q[(y1 + dy) * gw + x1 + dx] @ K[(y2 + dy) * gw + x2 + dx]
    assert abs(a - b) < 1e-10


def pin_window_order_positions(w):
    rng = np.random.default_rng(13)
    grids = [(7, 10), (3, 3)]
    x = rng.standard_normal((79, H_ * D_))
    ref = w.to_window_order(_rope(w, x, grids), grids, 4)
    got = _rope(w, w.to_window_order(x, grids, 4), grids, win=4)
    assert np.abs(ref - got).max() < 1e-12


PINS = [pin_golden_5x7, pin_fixture_segment_counts, pin_segments_are_clipped_blocks, pin_identity_cases,
        pin_round_trip, pin_rotation_preserves_pair_norms, pin_angles_closed_form,
        pin_width_first_axis_separation, pin_relative_position, pin_window_order_positions, pin_roformer_per_axis]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(W)


MUTANTS = [
    ("height first", "for first, pos in ((0, cols + 1), (half, rows + 1)):",
     "for first, pos in ((0, rows + 1), (half, cols + 1)):"),
    ("0-based positions", "for first, pos in ((0, cols + 1), (half, rows + 1)):",
     "for first, pos in ((0, cols), (half, rows)):"),
    ("sign of the sine term", "out[:, :, first + 2 * i] = re * c - im * s",
     "out[:, :, first + 2 * i] = re * c + im * s"),
    ("reverse rotation", "re * c - im * s\n            out[:, :, first + 2 * i + 1] = re * s + im * c",
     "re * c + im * s\n            out[:, :, first + 2 * i + 1] = -re * s + im * c"),
    ("frequency exponent", "w = theta ** (-4.0 * i / d)", "w = theta ** (-2.0 * i / d)"),
    ("column-major blocks", "for y0 in range(0, gh, win):              # block rows, top to bottom\n"
     "            for x0 in range(0, gw, win):",
     "for x0 in range(0, gw, win):              # block rows, top to bottom\n"
     "            for y0 in range(0, gh, win):"),
    ("column-major inside a block", "for y in range(y0, min(y0 + win, gh)):      # rows inside the block\n"
     "                    for x in range(x0, min(x0 + win, gw)):",
     "for x in range(x0, min(x0 + win, gw)):      # rows inside the block\n"
     "                    for y in range(y0, min(y0 + win, gh)):"),
    ("no edge clip", "for y in range(y0, min(y0 + win, gh)):", "for y in range(y0, y0 + win):"),
    ("no image offset", "        base += gh * gw\n    return np.array(perm", "    return np.array(perm"),
    ("wrong inverse", "out[perm] = xw", "out = xw[perm]"),
    ("window positions not permuted", "        rows, cols = rows[perm], cols[perm]", "        pass"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(name, old, new):
    assert old in SRC, f"mutation target missing: {name}"
    mod = types.ModuleType(f"mutant_{name}")
    exec(compile(SRC.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:  # any failure, assertion or error, counts as caught
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passes every pin"


def test_roformer_reference_itself():
    """The RoFormer function is checked on its own against the 2x2 rotation it
    stands for: pair i of a vector at position m turns by m * base^(-2(i-1)/n), and
    the first pair (theta_1 = 1) by exactly m radians."""
    x = np.zeros(8)
    x[0] = 1.0
    y = roformer_1d(x, 0.5)
    assert abs(y[0] - math.cos(0.5)) < 1e-15 and abs(y[1] - math.sin(0.5)) < 1e-15
    x = np.zeros(8)
    x[6] = 1.0  # pair 4: theta_4 = 10000^(-6/8)
    y = roformer_1d(x, 3.0)
    ang = 3.0 * 10000.0 ** (-0.75)
    assert abs(y[6] - math.cos(ang)) < 1e-15 and abs(y[7] - math.sin(ang)) < 1e-15


@pytest.mark.parametrize("name", ["frequency exponent", "0-based positions", "height first", "sign of the sine term",
                                  "reverse rotation"])
def test_roformer_pin_alone_catches(name):
    """The RoPE mutants are caught by the RoFormer pin on its own, not only by pins
    that restate the oracle's formula."""
    old, new = next((m[1], m[2]) for m in MUTANTS if m[0] == name)
    mod = types.ModuleType(f"mutant_{name}")
    exec(compile(SRC.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    with pytest.raises(AssertionError):
        pin_roformer_per_axis(mod)
