"""mgattn_dense_rope2d (q rotated by the 2D RoPE as the attention kernel loads it, k
rotated in place by the RoPE pass) against the unfused path on the same inputs:
mgattn_rope2d on q and on k, then mgattn_dense_strided.  The fused kernel rounds the
rotated q exactly as the pass does, so the outputs and the rotated k are equal bit for
bit; q is left untouched.  One case is also compared with the oracle on the rotated
inputs.  Workloads: the tower's 64x64 grid in window order (full layer and 32x32
window layer), the 16,384-token ragged batch with clipped edge windows, a causal call,
a negative scale, and a merged q|k|v buffer."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle as orc
from tests.gpu_helpers import BF16_TOL, from_device, say, to_device
from vit_perception_encoder_amd import mgattn as mg
from vit_perception_encoder_amd import workloads as wl

pytestmark = pytest.mark.gpu
THETA = 10000.0


@pytest.fixture(scope="module")
def torch():
    import torch as t

    assert t.cuda.is_available()
    mg.load_library()
    return t


def _case(torch, grids, win, layer, causal=0, scale=None, seed=0, merged=False):
    H, d = 16, 96
    row = H * d
    T = sum(gh * gw for gh, gw in grids)
    cu = mg.mgattn_window_segments(grids, win if layer == "window" else 1 << 20)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    say(f"fused rope grids={grids} win={win} layer={layer} causal={causal} scale={scale:.4f} merged={merged}")
    q, k, v = (to_device(wl.f32_to_bf16_bits(wl.normal_f32(seed + i, (T, row))), torch) for i in range(3))
    s = torch.cuda.current_stream()
    if merged:
        qkv = torch.cat([q, k, v], dim=1).contiguous()
        q, k, v = qkv[:, :row], qkv[:, row:2 * row], qkv[:, 2 * row:]
    ld = q.stride(0)
    q0 = q.clone()
    # unfused: rotate copies of q and k in memory, then attend
    qr, kr = q.clone(), k.clone()
    mg.mgattn_rope2d(qr, row, grids, win, H, d, THETA, wl.BF16, s)
    mg.mgattn_rope2d(kr, row, grids, win, H, d, THETA, wl.BF16, s)
    want = torch.empty(T, row, dtype=torch.bfloat16, device="cuda")
    mg.mgattn_dense(qr, kr, v.contiguous(), want, cu, len(cu) - 1, H, d, scale, causal, wl.BF16, s)
    # fused
    got = torch.full((T, row), float("nan"), dtype=torch.bfloat16, device="cuda")
    mg.mgattn_dense_rope2d(q, k, v, got, ld, ld, ld, row, cu, len(cu) - 1, H, d, scale, causal, wl.BF16, grids, win,
                           THETA, s)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "fused output differs from the unfused path"
    assert torch.equal(k.contiguous().view(torch.int16), kr.view(torch.int16)), "k not rotated as mgattn_rope2d does"
    assert torch.equal(q.view(torch.int16), q0.view(torch.int16)), "q was modified"
    return qr, kr, v.contiguous(), got, cu, scale


@pytest.mark.parametrize("layer", ["full", "window"])
def test_tower_grid_window_order(torch, layer):
    _case(torch, [(64, 64)], 32, layer, seed=900)


def test_ragged_batch_with_clipped_windows(torch):
    _case(torch, [(112, 96), (72, 56), (40, 40)], 32, "window", seed=910)


def test_causal_negative_scale_merged_qkv(torch):
    _case(torch, [(24, 40), (7, 9)], 8, "full", causal=1, scale=-0.07, seed=920, merged=True)


@pytest.mark.parametrize("grid,bm", [((32, 32), 64), ((32, 64), 128)])
def test_key_split_shapes(torch, grid, bm):
    """A 448x448 image (one 1024-token segment: 64-query tiles, keys split between two
    wave groups) and a 2048-token one (128-query key-split tiles), full attention."""
    T = grid[0] * grid[1]
    assert mg.mgattn_dense_plan_block_m([0, T], 1, 16, 96, wl.BF16, 0) == bm
    _case(torch, [grid], 32, "full", seed=940 + bm)


def test_raster_order_against_oracle(torch):
    """Tokens in raster order (win = 0), 64-query key-split tiles (a short call); the
    fused output against the oracle on the rotated bf16 q and k the RoPE pass stores."""
    grids = [(20, 30)]
    qr, kr, v, got, cu, scale = _case(torch, grids, 0, "full", seed=930)
    assert mg.mgattn_dense_plan_block_m(cu, len(cu) - 1, 16, 96, wl.BF16, 0) == 64
    T = 600
    qh, kh, vh = (from_device(x, torch).astype(np.float32) for x in (qr, kr, v))
    to_bits = wl.f32_to_bf16_bits  # exact: the values are bf16 already
    want = orc.attention(*(to_bits(x).reshape(T, 16, 96) for x in (qh, kh, vh)), cu, 16, 96, scale)
    err = np.abs(from_device(got, torch).reshape(T, 16, 96) - want).max()
    assert err <= BF16_TOL, f"max err {err:.3e}"
