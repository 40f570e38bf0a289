"""Plain numpy oracle of the perception encoder's token order and 2D rotary
embedding.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with the
HIP library and never imports the ``vit_perception_encoder_amd`` package.

What the pages give, and the readings taken where they are silent:

* Window layers attend inside 32x32 = 1024-patch windows cut by the vision tower's
  sparse permutation (vllm.cpp issue #1545, second comment, "Two of the three
  labelled uncertainties are now resolved"); the tower gathers its tokens window by
  window and applies the inverse permutation before the final LayerNorm, permuting
  the rotary table alongside (vllm.cpp PR #279, vision-tower commit).  The block walk
  order and the order inside a block are mutation-pinned upstream but not stated.
  Reading: row-major over the win x win blocks of each image, edge blocks clipped to
  the grid, row-major inside a block; images of a batch keep their own token ranges.
* 2D RoPE, width-first, 1-based positions (PR #279, vision-tower commits).  No
  formula is printed.  Reading: channels [0, d/2) of a head rotate with the patch's
  column + 1, channels [d/2, d) with its row + 1; inside a half, channel pair
  (2i, 2i+1) is the complex number c_2i + i*c_2i+1 multiplied by exp(i*pos*w_i),
  w_i = theta^(-4i/d).  Evaluated in f64.
"""
from __future__ import annotations

import math

import numpy as np


def window_order(grids, win):
    """(perm, cu_seqlens): perm[p] is the raster index (batch-global) of the token at
    window-order position p; cu_seqlens holds the window segments in that order.
    Written as the nested walk the reading describes."""
    perm, cu, base = [], [0], 0
    for gh, gw in grids:
        for y0 in range(0, gh, win):              # block rows, top to bottom
            for x0 in range(0, gw, win):          # blocks of a row, left to right
                for y in range(y0, min(y0 + win, gh)):      # rows inside the block
                    for x in range(x0, min(x0 + win, gw)):  # columns inside the block
                        perm.append(base + y * gw + x)
                cu.append(len(perm))
        base += gh * gw
    return np.array(perm, dtype=np.int64), np.array(cu, dtype=np.int32)


def to_window_order(x, grids, win):
    """Rows of x (raster order) gathered into window order."""
    perm, _ = window_order(grids, win)
    return x[perm]


def to_raster_order(xw, grids, win):
    """Rows of xw (window order) scattered back into raster order."""
    perm, _ = window_order(grids, win)
    out = np.empty_like(xw)
    out[perm] = xw
    return out


def patch_coords(grids, win=0):
    """(row, col) of every token's patch, 0-based, for tokens in raster order
    (win == 0) or in the window order of window win."""
    rows, cols = [], []
    for gh, gw in grids:
        for y in range(gh):
            for x in range(gw):
                rows.append(y)
                cols.append(x)
    rows, cols = np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)
    if win > 0:
        perm, _ = window_order(grids, win)
        rows, cols = rows[perm], cols[perm]
    return rows, cols


def rope2d(x, grids, win, H, d, theta=10000.0):
    """f64 rotation of x ([T, >= H*d], float values; the first H*d columns are H heads
    of d channels) for tokens in raster (win == 0) or window order."""
    rows, cols = patch_coords(grids, win)
    T = rows.shape[0]
    xf = np.asarray(x, dtype=np.float64)[:, :H * d].reshape(T, H, d)
    out = xf.copy()
    half = d // 2
    for i in range(d // 4):
        w = theta ** (-4.0 * i / d)
        for first, pos in ((0, cols + 1), (half, rows + 1)):  # width half first
            ang = pos.astype(np.float64) * w
            c = np.cos(ang)[:, None]
            s = np.sin(ang)[:, None]
            re = xf[:, :, first + 2 * i]
            im = xf[:, :, first + 2 * i + 1]
            out[:, :, first + 2 * i] = re * c - im * s
            out[:, :, first + 2 * i + 1] = re * s + im * c
    return out.reshape(T, H * d)


def angle_of_pair(vec2):
    """Angle of a 2-vector in [0, 2*pi) (for the pins)."""
    return math.atan2(vec2[1], vec2[0]) % (2 * math.pi)
