"""GPU parity of the token-order entry points against the numpy oracle
(oracle/window_rope.py, pinned in tests/test_window_rope_oracle.py):

* mgattn_window_permute: gather into window order and scatter back, bit-exact;
* mgattn_rope2d: f32 and bf16, raster and window order, contiguous and in place on the
  q and k columns of a merged qkv buffer (v untouched), within the error bound of
  f32 angles (|angle error| <= pos * 2^-23 with pos <= 129 here) plus the bf16 rounding
  of the output (unit roundoff 2^-8: bf16 carries 8 significant bits);
* the tower's token path end to end: raster-order q, k, v -> window order -> RoPE ->
  window-segment attention -> raster order, against attention written directly over
  window membership in raster order (no permutation on the oracle side)."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import window_rope as W
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


def _tokens(grids):
    return sum(gh * gw for gh, gw in grids)


@pytest.mark.parametrize("grids,win", [([(5, 7)], 3), ([(64, 64)], 32), ([(128, 96), (64, 64), (32, 32)], 32),
                                       ([(112, 96), (72, 56), (40, 40)], 32), ([(12, 12), (8, 8)], 8),
                                       ([(33, 65), (1, 9), (40, 40)], 32)])
@pytest.mark.parametrize("row_bytes", [16, 3072])
def test_window_permute_bit_exact(torch, grids, win, row_bytes):
    T = _tokens(grids)
    say(f"window permute grids={grids} win={win} row_bytes={row_bytes}")
    rng = np.random.default_rng(T + row_bytes)
    x = rng.integers(0, 256, size=(T, row_bytes), dtype=np.uint8)
    src = torch.from_numpy(x).cuda()
    dst = torch.zeros_like(src)
    back = torch.zeros_like(src)
    mg.mgattn_window_permute(src, dst, row_bytes, grids, win, 0, torch.cuda.current_stream())
    mg.mgattn_window_permute(dst, back, row_bytes, grids, win, 1, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), W.to_window_order(x, grids, win))
    assert np.array_equal(back.cpu().numpy(), x)


def _random_grids(rng, win):
    """1-5 images with sides 1..80 (most not multiples of the window)."""
    return [(int(rng.integers(1, 81)), int(rng.integers(1, 81))) for _ in range(int(rng.integers(1, 6)))], win


@pytest.mark.parametrize("case_seed,win", [(2701, 1), (2702, 3), (2703, 8), (2704, 16), (2705, 32), (2706, 32)])
def test_random_grids_permute_and_rope(torch, case_seed, win):
    """Seeded random image batches: the gather into window order and back is bit exact,
    and RoPE in window order (head_dim 64/96/128, bf16 or f32) matches the oracle."""
    rng = np.random.Generator(np.random.PCG64(case_seed))
    grids, win = _random_grids(rng, win)
    T = _tokens(grids)
    row_bytes = int(rng.choice([16, 48, 3072]))
    say(f"random grids={grids} win={win} row_bytes={row_bytes}")
    x = rng.integers(0, 256, size=(T, row_bytes), dtype=np.uint8)
    src = torch.from_numpy(x).cuda()
    dst = torch.zeros_like(src)
    back = torch.zeros_like(src)
    mg.mgattn_window_permute(src, dst, row_bytes, grids, win, 0, torch.cuda.current_stream())
    mg.mgattn_window_permute(dst, back, row_bytes, grids, win, 1, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), W.to_window_order(x, grids, win))
    assert np.array_equal(back.cpu().numpy(), x)
    H, d = int(rng.choice([1, 4, 16])), int(rng.choice([64, 96, 128]))
    dtype = wl.BF16 if rng.random() < 0.6 else wl.F32
    xr = wl.normal_f32(case_seed, (T, H * d))
    if dtype == wl.BF16:
        xr = wl.f32_to_bf16_bits(xr)
        xin = wl.bf16_bits_to_f32(xr)
    else:
        xin = xr
    xd = to_device(xr, torch)
    mg.mgattn_rope2d(xd, H * d, grids, win, H, d, THETA, dtype, torch.cuda.current_stream())
    torch.cuda.synchronize()
    _check_rope(from_device(xd, torch), W.rope2d(xin, grids, win, H, d, THETA), H, d, dtype)


def _rope_bound(want_pairs_norm, dtype):
    angle = 129 * 2.0 ** -23 + 2e-7
    return want_pairs_norm * (angle + (2.0 ** -8 if dtype == wl.BF16 else 0.0)) + 1e-7


def _check_rope(got, want, H, d, dtype):
    norms = np.repeat(np.hypot(want[:, 0::2], want[:, 1::2]), 2, axis=1)
    err = np.abs(got - want)
    bound = _rope_bound(norms, dtype)
    worst = np.unravel_index(int(np.argmax(err - bound)), err.shape)
    assert np.all(err <= bound), f"rope error {err[worst]:.3e} > bound {bound[worst]:.3e} at {worst}"


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
@pytest.mark.parametrize("grids,win", [([(64, 64)], 0), ([(64, 64)], 32), ([(112, 96), (72, 56), (40, 40)], 32),
                                       ([(7, 5)], 0)])
def test_rope2d_matches_oracle(torch, dtype, grids, win):
    H, d = 16, 96
    T = _tokens(grids)
    say(f"rope2d dtype={dtype} grids={grids} win={win}")
    x = wl.normal_f32(700 + T + win, (T, H * d))
    if dtype == wl.BF16:
        x = wl.f32_to_bf16_bits(x)
        xin = wl.bf16_bits_to_f32(x)
    else:
        xin = x
    xd = to_device(x, torch)
    mg.mgattn_rope2d(xd, H * d, grids, win, H, d, THETA, dtype, torch.cuda.current_stream())
    torch.cuda.synchronize()
    _check_rope(from_device(xd, torch), W.rope2d(xin, grids, win, H, d, THETA), H, d, dtype)


@pytest.mark.parametrize("d", [64, 128])
def test_rope2d_other_head_dims(torch, d):
    grids, H = [(20, 13)], 3
    T = _tokens(grids)
    say(f"rope2d d={d}")
    x = wl.f32_to_bf16_bits(wl.normal_f32(730 + d, (T, H * d)))
    xd = to_device(x, torch)
    mg.mgattn_rope2d(xd, H * d, grids, 4, H, d, THETA, wl.BF16, torch.cuda.current_stream())
    torch.cuda.synchronize()
    _check_rope(from_device(xd, torch), W.rope2d(wl.bf16_bits_to_f32(x), grids, 4, H, d, THETA), H, d, wl.BF16)


@pytest.mark.parametrize("dtype,d,H", [(wl.BF16, 16, 37), (wl.BF16, 32, 5), (wl.BF16, 48, 11), (wl.F32, 16, 9),
                                       (wl.F32, 64, 3), (wl.F32, 128, 5)])
def test_rope2d_piece_groups(torch, dtype, d, H):
    """The pass gives each lane one 16-byte piece position of a head (P = d*elem/16
    pieces per head, 64/P heads per group of lanes).  Every head dim's layout, from 2
    pieces and 32 heads per group to 32 pieces and 2 heads, with head counts that leave
    the last group partial, on rows padded past H*d: the heads match the oracle and the
    padding is left untouched."""
    grids, win = [(9, 11)], 4
    T = _tokens(grids)
    elem = 2 if dtype == wl.BF16 else 4
    ld = H * d + 3 * (16 // elem)  # three 16-byte pieces of padding per row
    say(f"rope2d piece groups dtype={dtype} d={d} H={H}")
    x = wl.normal_f32(760 + d + H, (T, ld))
    if dtype == wl.BF16:
        x = wl.f32_to_bf16_bits(x)
        xin = wl.bf16_bits_to_f32(x).astype(np.float64)
    else:
        xin = x.astype(np.float64)
    xd = to_device(x, torch)
    mg.mgattn_rope2d(xd, ld, grids, win, H, d, THETA, dtype, torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = from_device(xd, torch)
    _check_rope(got[:, :H * d], W.rope2d(xin[:, :H * d], grids, win, H, d, THETA), H, d, dtype)
    assert np.array_equal(got[:, H * d:], xin[:, H * d:]), "the pass wrote into the row padding"


def test_rope2d_in_place_on_merged_qkv(torch):
    H, d, grids, win = 16, 96, [(40, 40), (9, 33)], 32
    T, row = _tokens(grids), H * d
    say("rope2d on merged qkv columns")
    qkv = wl.f32_to_bf16_bits(wl.normal_f32(741, (T, 3 * row)))
    buf = to_device(qkv, torch)
    for part in (0, 1):  # q, then k
        mg.mgattn_rope2d(buf[:, part * row:(part + 1) * row], buf.stride(0), grids, win, H, d, THETA, wl.BF16,
                         torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = from_device(buf, torch)
    ref = wl.bf16_bits_to_f32(qkv).astype(np.float64)
    assert np.array_equal(got[:, 2 * row:], ref[:, 2 * row:]), "v columns were written"
    for part in (0, 1):
        _check_rope(got[:, part * row:(part + 1) * row], W.rope2d(ref[:, part * row:(part + 1) * row], grids, win,
                                                                   H, d, THETA), H, d, wl.BF16)


def test_rope2d_q_and_k_in_one_call(torch):
    """q and k are adjacent in a merged qkv row, so one call over 2H heads with the
    merged row stride rotates both: the same result as the oracle on each part."""
    H, d, grids, win = 16, 96, [(40, 40), (9, 33)], 32
    T, row = _tokens(grids), H * d
    say("rope2d on q and k of merged qkv in one call (2H heads)")
    qkv = wl.f32_to_bf16_bits(wl.normal_f32(743, (T, 3 * row)))
    buf = to_device(qkv, torch)
    mg.mgattn_rope2d(buf[:, :2 * row], buf.stride(0), grids, win, 2 * H, d, THETA, wl.BF16,
                     torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = from_device(buf, torch)
    ref = wl.bf16_bits_to_f32(qkv).astype(np.float64)
    assert np.array_equal(got[:, 2 * row:], ref[:, 2 * row:]), "v columns were written"
    for part in (0, 1):
        _check_rope(got[:, part * row:(part + 1) * row], W.rope2d(ref[:, part * row:(part + 1) * row], grids, win,
                                                                   H, d, THETA), H, d, wl.BF16)


def _window_attention_rows(q, k, v, grids, win, scale, rows):
    """f64 attention of raster-order tokens `rows` over the keys of their window, with
    window membership computed from patch coordinates (no permutation)."""
    coords, base = [], 0
    for img, (gh, gw) in enumerate(grids):
        for y in range(gh):
            for x in range(gw):
                coords.append((img, y // win, x // win))
    coords = np.array(coords)
    out = []
    for t in rows:
        keys = np.nonzero(np.all(coords == coords[t], axis=1))[0]
        s = np.einsum("hc,khc->hk", q[t], k[keys]) * scale
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out.append(np.einsum("hk,khc->hc", p / p.sum(axis=1, keepdims=True), v[keys]))
    return np.array(out)


def test_tower_token_path_end_to_end(torch):
    """raster q,k,v -> window order -> RoPE on q,k -> attention over the window
    segments -> output back in raster order, against the raster-order oracle."""
    H, d, win = 16, 96, 32
    grids = [(40, 40), (33, 65)]
    T, row = _tokens(grids), H * d
    scale = 1.0 / np.sqrt(d)
    say(f"tower token path grids={grids}")
    q, k, v = (wl.f32_to_bf16_bits(wl.normal_f32(750 + i, (T, row))) for i in range(3))
    s = torch.cuda.current_stream()
    dev = [to_device(x, torch) for x in (q, k, v)]
    win_order = [torch.empty_like(x) for x in dev]
    for a, b in zip(dev, win_order):
        mg.mgattn_window_permute(a, b, row * 2, grids, win, 0, s)
    for x in win_order[:2]:
        mg.mgattn_rope2d(x, row, grids, win, H, d, THETA, wl.BF16, s)
    cu = mg.mgattn_window_segments(grids, win)
    out_w = torch.empty_like(dev[0])
    mg.mgattn_dense(win_order[0], win_order[1], win_order[2], out_w, cu, len(cu) - 1, H, d, scale, 0, wl.BF16, s)
    out = torch.empty_like(dev[0])
    mg.mgattn_window_permute(out_w, out, row * 2, grids, win, 1, s)
    torch.cuda.synchronize()
    got = from_device(out, torch).reshape(T, H, d)
    # oracle: RoPE in raster order (positions of the patches), rounded to bf16 as the
    # stored q and k are, then attention over window membership
    qr, kr = (wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(
        W.rope2d(wl.bf16_bits_to_f32(x), grids, 0, H, d, THETA).astype(np.float32))).astype(np.float64)
              for x in (q, k))
    vf = wl.bf16_bits_to_f32(v).astype(np.float64)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 31, 32, 1599, 1600, T - 1], rng.integers(0, T, 60)]))
    want = _window_attention_rows(qr.reshape(T, H, d), kr.reshape(T, H, d), vf.reshape(T, H, d), grids, win,
                                  scale, rows)
    err = np.abs(got[rows] - want).max()
    assert err <= BF16_TOL, f"max err {err:.3e}"
