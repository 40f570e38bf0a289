"""GPU parity of mgattn_attention_kv (causal sliding-window attention with grouped
key/value heads over a KV cache, the text decoder's attention) against the numpy f64
oracle (oracle/gqa_window.py, pinned in tests/test_gqa_window_oracle.py), on the same
seeded inputs, to the tolerances of the dense tests (bf16 2e-2, f32 1e-4).

Shapes: the text decoder's heads (32 query heads, 2 key/value heads, head size 128,
window 2048) in prefill longer than the window, a cache with new queries, and
one-token decoding; plus small windows, other head groupings and head sizes, ragged
and empty sequences, and the merged q|k|v projection layout."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import gqa_window as G
from tests.gpu_helpers import BF16_TOL, F32_TOL, from_device, say, to_device
from vit_perception_encoder_amd import mgattn as mg
from vit_perception_encoder_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t

    assert t.cuda.is_available()
    mg.load_library()
    return t


def _arr(seed, shape, dtype):
    x = wl.normal_f32(seed, shape)
    if dtype == wl.BF16:
        bits = wl.f32_to_bf16_bits(x)
        return bits, wl.bf16_bits_to_f32(bits)
    return x, x


def _check(torch, name, lq, lk, Hq, Hkv, d, window, dtype, seed, scale=None):
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    Tq, Tk = int(cq[-1]), int(ck[-1])
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    say(f"{name}: lq={lq} lk={lk} Hq={Hq} Hkv={Hkv} d={d} window={window} dtype={dtype}")
    q, qf = _arr(seed, (Tq, Hq * d), dtype)
    k, kf = _arr(seed + 1, (Tk, Hkv * d), dtype)
    v, vf = _arr(seed + 2, (Tk, Hkv * d), dtype)
    qd, kd, vd = (to_device(x, torch) for x in (q, k, v))
    out = torch.full_like(qd, -777.0)
    mg.mgattn_attention_kv(qd, kd, vd, out, Hq * d, Hkv * d, Hkv * d, Hq * d, cq, ck, len(lq), Hq, Hkv, d, scale,
                           window, dtype, torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = from_device(out, torch).reshape(Tq, Hq, d)
    want = G.attention_kv(qf, kf, vf, cq, ck, Hq, Hkv, d, scale, window)
    err = np.abs(got - want)
    tol = BF16_TOL if dtype == wl.BF16 else F32_TOL
    worst = np.unravel_index(int(np.argmax(err)), err.shape)
    assert err.max() <= tol, f"max err {err.max():.3e} at (t,h,c)={worst}"


@pytest.mark.parametrize("case_seed", list(range(1701, 1717)))
def test_random_caches(torch, case_seed):
    """Seeded random combinations: 1-6 sequences, each a prefill (as many queries as
    keys), a one-token decode or new queries over a longer cache; 1-4 key/value heads of
    1-16 query heads each; head_dim 64/96/128; no window or a random one; bf16 or f32;
    scale of either sign.  Whole outputs against the oracle."""
    rng = np.random.Generator(np.random.PCG64(case_seed))
    n = int(rng.integers(1, 7))
    lk = [int(rng.choice([1, 2, 63, 64, 65, 255, 256, 257])) if rng.random() < 0.4 else int(rng.integers(1, 1200))
          for _ in range(n)]
    lq = []
    for L in lk:
        r = rng.random()
        lq.append(L if r < 0.4 else (1 if r < 0.7 else int(rng.integers(0, L + 1))))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8, 16] if Hkv < 4 else [1, 2, 4]))
    d = int(rng.choice([64, 96, 128]))
    window = 0 if rng.random() < 0.4 else int(rng.integers(1, 1300))
    dtype = wl.BF16 if rng.random() < 0.75 else wl.F32
    scale = float(rng.choice([-1.0, 1.0]) * rng.uniform(0.02, 0.25))
    _check(torch, f"random{case_seed}", lq, lk, Hq, Hkv, d, window, dtype, seed=case_seed, scale=scale)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_text_decoder_prefill_longer_than_window(torch, dtype):
    _check(torch, "prefill", [2600], [2600], 32, 2, 128, 2048, dtype, seed=801)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_text_decoder_cache_with_new_queries(torch, dtype):
    _check(torch, "cache", [300, 45], [2500, 45], 32, 2, 128, 2048, dtype, seed=811)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_text_decoder_one_token_decode(torch, dtype):
    lk = [1, 17, 2047, 2048, 2049, 3000]
    _check(torch, "decode", [1] * len(lk), lk, 32, 2, 128, 2048, dtype, seed=821)


@pytest.mark.parametrize("window", [0, 1, 2, 7, 64, 200, 257])
def test_small_windows(torch, window):
    _check(torch, f"window{window}", [300, 1, 77], [300, 9, 600], 4, 1, 64, window, wl.BF16, seed=831)


def test_window_wider_than_every_cache_is_no_window(torch):
    """A window beyond every sequence's keys (up to 2^31 - 1) masks nothing: bit for bit
    the plain causal call (window 0), prefill and cache rows alike."""
    Hq, Hkv, d = 8, 2, 128
    lq, lk = [300, 1, 77], [300, 9, 600]
    cq = [0] + list(np.cumsum(lq))
    ck = [0] + list(np.cumsum(lk))
    q = to_device(_arr(961, (cq[-1], Hq * d), wl.BF16)[0], torch)
    k = to_device(_arr(962, (ck[-1], Hkv * d), wl.BF16)[0], torch)
    v = to_device(_arr(963, (ck[-1], Hkv * d), wl.BF16)[0], torch)
    s = torch.cuda.current_stream()
    outs = []
    for window in (0, 600, 2 ** 31 - 1):
        say(f"wide window {window}")
        o = torch.empty_like(q)
        mg.mgattn_attention_kv(q, k, v, o, Hq * d, Hkv * d, Hkv * d, Hq * d, cq, ck, 3, Hq, Hkv, d, 0.09, window,
                               wl.BF16, s)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("d,Hq,Hkv", [(64, 8, 8), (96, 16, 4), (128, 6, 3), (96, 3, 1)])
@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_groupings_and_head_dims(torch, d, Hq, Hkv, dtype):
    _check(torch, "groups", [513, 0, 130], [700, 5, 130], Hq, Hkv, d, 300, dtype, seed=841)


def test_merged_qkv_text_layout(torch):
    """The decoder's merged projection [T, (Hq + 2*Hkv)*d]: q, k, v column views of one
    buffer (prefill, so the cache is the same tokens)."""
    Hq, Hkv, d, T, W = 32, 2, 128, 700, 256
    say("merged qkv, text layout")
    wide = (Hq + 2 * Hkv) * d
    bits, vals = _arr(851, (T, wide), wl.BF16)
    buf = to_device(bits, torch)
    out = torch.empty(T, Hq * d, dtype=torch.bfloat16, device="cuda")
    qv, kv, vv = buf[:, :Hq * d], buf[:, Hq * d:(Hq + Hkv) * d], buf[:, (Hq + Hkv) * d:]
    mg.mgattn_attention_kv(qv, kv, vv, out, wide, wide, wide, Hq * d, [0, T], [0, T], 1, Hq, Hkv, d, 0.0883883,
                           W, wl.BF16, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = G.attention_kv(vals[:, :Hq * d], vals[:, Hq * d:(Hq + Hkv) * d], vals[:, (Hq + Hkv) * d:], [0, T], [0, T],
                          Hq, Hkv, d, np.float32(0.0883883), W)
    assert np.abs(from_device(out, torch).reshape(T, Hq, d) - want).max() <= BF16_TOL


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_dense_path_unchanged_by_the_generalisation(torch, dtype, d):
    """mgattn_attention_kv with keys = queries, Hkv = Hq and no window equals the causal
    dense call bit for bit (the same arithmetic, from the general and the dense
    instantiation of one kernel template)."""
    H, lens = 4, [333, 64, 1]
    cu = [0] + list(np.cumsum(lens))
    T = cu[-1]
    say(f"kv entry vs dense causal, dtype={dtype} d={d}")
    q, k, v = (to_device(_arr(861 + i, (T, H * d), dtype)[0], torch) for i in range(3))
    a, b = torch.empty_like(q), torch.empty_like(q)
    s = torch.cuda.current_stream()
    mg.mgattn_attention_kv(q, k, v, a, H * d, H * d, H * d, H * d, cu, cu, 3, H, H, d, 0.1, 0, dtype, s)
    mg.mgattn_dense(q, k, v, b, cu, 3, H, d, 0.1, 1, dtype, s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("d,Hq,Hkv,window", [(64, 16, 2, 0), (96, 8, 1, 100), (128, 32, 2, 2048), (128, 4, 4, 33),
                                            (64, 32, 1, 1)])
def test_decode_kernel_shapes(torch, d, Hq, Hkv, window):
    """One-token decoding (the key-split decode kernel): groupings up to 32 query heads
    per key/value head, head sizes, windows, caches from 1 to beyond the window."""
    lk = [1, 2, 31, 32, 33, 255, 700, 2100]
    _check(torch, "decode kernel", [1] * len(lk), lk, Hq, Hkv, d, window, wl.BF16, seed=871 + d + window)


def test_decode_many_sequences_and_scales(torch):
    """More sequences than one launch holds (150 > 120), empty query rows in between,
    and negative / zero scale."""
    rng = np.random.default_rng(881)
    lk = rng.integers(1, 600, size=150).tolist()
    lq = [1] * 150
    lq[3] = 0
    for scale in (-0.2, 0.0):
        _check(torch, f"decode 150 seqs scale {scale}", lq, lk, 16, 2, 128, 300, wl.BF16, seed=883, scale=scale)


# ------------------------------------------------ one-token decoding with a workspace

def _check_ws(torch, name, lk, Hq, Hkv, d, window, seed, ws_frac=1.0, scale=None, expect_split=True, ws=None):
    """mgattn_attention_kv_ws on one-token decoding against the oracle, with a workspace
    of ws_frac times the full-split size (in the tensor ws when given)."""
    n = len(lk)
    cq = np.arange(n + 1, dtype=np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    full = mg.mgattn_attention_kv_workspace(list(cq), list(ck), n, Hq, Hkv, d, window, wl.BF16)
    assert (full > 0) == expect_split, full
    nbytes = int(full * ws_frac) // 256 * 256
    say(f"{name}: n={n} lk[:8]={lk[:8]} Hq={Hq} Hkv={Hkv} d={d} window={window} workspace={nbytes}/{full}")
    q, qf = _arr(seed, (n, Hq * d), wl.BF16)
    k, kf = _arr(seed + 1, (int(ck[-1]), Hkv * d), wl.BF16)
    v, vf = _arr(seed + 2, (int(ck[-1]), Hkv * d), wl.BF16)
    qd, kd, vd = (to_device(x, torch) for x in (q, k, v))
    out = torch.full_like(qd, -777.0)
    if ws is None:
        ws = torch.full((max(nbytes, 256),), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-patterned scratch
    assert ws.numel() >= nbytes
    mg.mgattn_attention_kv_ws(qd, kd, vd, out, Hq * d, Hkv * d, Hkv * d, Hq * d, list(cq), list(ck), n, Hq, Hkv, d,
                              scale, window, wl.BF16, ws, nbytes, torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = from_device(out, torch).reshape(n, Hq, d)
    want = G.attention_kv(qf, kf, vf, cq, ck, Hq, Hkv, d, scale, window)
    err = np.abs(got - want)
    worst = np.unravel_index(int(np.argmax(err)), err.shape)
    assert np.all(np.isfinite(got))
    assert err.max() <= BF16_TOL, f"max err {err.max():.3e} at (seq,h,c)={worst}"
    return got


def test_decode_split_text_decoder_batch(torch):
    """The text decoder's decoding step at batch 32 over 4096 cached keys (window 2048):
    64 (sequence, key/value head) pairs, each split over 4 workgroups."""
    _check_ws(torch, "decode split 32x4096", [4096] * 32, 32, 2, 128, 2048, seed=891)


@pytest.mark.parametrize("d,Hq,Hkv,window", [(64, 16, 2, 0), (96, 8, 1, 100), (128, 32, 2, 2048), (128, 4, 4, 33),
                                            (64, 32, 1, 1), (128, 32, 2, 0)])
def test_decode_split_shapes(torch, d, Hq, Hkv, window):
    """Split decoding with caches from 1 key (splits without keys) to beyond the
    window, every grouping and head size of the unsplit kernel's test."""
    lk = [1, 2, 31, 33, 255, 700, 2100, 5000]
    _check_ws(torch, "decode split", lk, Hq, Hkv, d, window, seed=901 + d + window,
              expect_split=window in (0, 2048))  # smaller windows leave < 16 blocks: no split


@pytest.mark.parametrize("frac", [0.0, 0.3, 0.5, 1.0])
def test_decode_split_partial_workspace(torch, frac):
    """A workspace below the full size gives fewer splits (none at 0 bytes), same result."""
    _check_ws(torch, f"decode workspace x{frac}", [3000, 17, 900], 32, 2, 128, 0, seed=911, ws_frac=frac)


def test_decode_split_scales_and_reuse(torch):
    """Negative and zero scale, and two calls in a row sharing one workspace (the second
    with fewer, shorter sequences)."""
    for scale in (-0.2, 0.0):
        _check_ws(torch, f"decode split scale {scale}", [1500, 2500, 64], 16, 2, 128, 2048, seed=921, scale=scale)
    ws = torch.full((8 << 20,), 0xFF, dtype=torch.uint8, device="cuda")
    _check_ws(torch, "decode split reuse 1", [4000] * 6, 32, 2, 128, 0, seed=923, ws=ws)
    _check_ws(torch, "decode split reuse 2", [700, 1200], 32, 2, 128, 0, seed=925, ws=ws)


def test_decode_split_repeated_calls_one_workspace(torch):
    """Three calls in a row on one zero-filled workspace, which each call leaves holding
    its partial results: every result matches the oracle and the first bit for bit."""
    ws = torch.zeros((4 << 20,), dtype=torch.uint8, device="cuda")
    first = _check_ws(torch, "decode split repeat 1", [2500] * 4, 32, 2, 128, 0, seed=931, ws=ws)
    for i in (2, 3):
        again = _check_ws(torch, f"decode split repeat {i}", [2500] * 4, 32, 2, 128, 0, seed=931, ws=ws)
        assert np.array_equal(again, first)


def test_decode_split_graph_capture_replays_match_eager(torch):
    """One-token decoding with a workspace (decode kernel + merge kernel, no allocation,
    no memset) captured into a HIP graph replays to the eager result bit for bit, with
    unrelated eager work and synchronisations between the replays."""
    n, Hq, Hkv, d, W = 8, 32, 2, 128, 2048
    lk = [3000, 17, 900, 2048, 64, 4000, 1, 700]
    cq = list(range(n + 1))
    ck = [int(x) for x in np.concatenate([[0], np.cumsum(lk)])]
    nbytes = mg.mgattn_attention_kv_workspace(cq, ck, n, Hq, Hkv, d, W, wl.BF16)
    assert nbytes > 0
    q, _ = _arr(961, (n, Hq * d), wl.BF16)
    k, _ = _arr(962, (ck[-1], Hkv * d), wl.BF16)
    v, _ = _arr(963, (ck[-1], Hkv * d), wl.BF16)
    qd, kd, vd = (to_device(x, torch) for x in (q, k, v))
    out = torch.zeros_like(qd)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")

    def call(stream):
        mg.mgattn_attention_kv_ws(qd, kd, vd, out, Hq * d, Hkv * d, Hkv * d, Hq * d, cq, ck, n, Hq, Hkv, d,
                                  d ** -0.5, W, wl.BF16, ws, nbytes, stream)

    call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = from_device(out, torch)
    say("decode split graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_device(out, torch), want), f"replay {rep}"
        junk.mul_(1.0001)  # unrelated eager work between replays
        torch.cuda.synchronize()


def test_decode_split_across_launches(torch):
    """More sequences than one launch holds: 150 one-token rows (and empty rows) go to
    a launch of 120 sequences (240 pairs, unsplit) and one of 30 (60 pairs, split 4
    ways), both through one workspace in stream order."""
    rng = np.random.default_rng(941)
    lk = rng.integers(1, 3000, size=150).tolist()
    lq = [1] * 150
    lq[7] = 0
    lq[130] = 0
    n, Hq, Hkv, d, W = 150, 32, 2, 128, 2048
    cq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    nbytes = mg.mgattn_attention_kv_workspace(list(cq), list(ck), n, Hq, Hkv, d, W, wl.BF16)
    assert nbytes > 0
    say(f"decode split across launches: n={n} workspace={nbytes}")
    q, qf = _arr(951, (int(cq[-1]), Hq * d), wl.BF16)
    k, kf = _arr(952, (int(ck[-1]), Hkv * d), wl.BF16)
    v, vf = _arr(953, (int(ck[-1]), Hkv * d), wl.BF16)
    qd, kd, vd = (to_device(x, torch) for x in (q, k, v))
    out = torch.full_like(qd, -777.0)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    mg.mgattn_attention_kv_ws(qd, kd, vd, out, Hq * d, Hkv * d, Hkv * d, Hq * d, list(cq), list(ck), n, Hq, Hkv, d,
                              d ** -0.5, W, wl.BF16, ws, nbytes, torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = from_device(out, torch).reshape(int(cq[-1]), Hq, d)
    want = G.attention_kv(qf, kf, vf, cq, ck, Hq, Hkv, d, d ** -0.5, W)
    assert np.abs(got - want).max() <= BF16_TOL


def test_decode_without_workspace_is_the_plain_entry(torch):
    """workspace_bytes = 0 runs exactly mgattn_attention_kv (bit for bit)."""
    lk = [4096] * 4
    n, Hq, Hkv, d = 4, 32, 2, 128
    cq, ck = list(range(n + 1)), [4096 * i for i in range(n + 1)]
    q = to_device(_arr(931, (n, Hq * d), wl.BF16)[0], torch)
    k = to_device(_arr(932, (sum(lk), Hkv * d), wl.BF16)[0], torch)
    v = to_device(_arr(933, (sum(lk), Hkv * d), wl.BF16)[0], torch)
    a, b = torch.empty_like(q), torch.empty_like(q)
    s = torch.cuda.current_stream()
    say("decode ws=0 vs plain")
    mg.mgattn_attention_kv(q, k, v, a, Hq * d, Hkv * d, Hkv * d, Hq * d, cq, ck, n, Hq, Hkv, d, 0.09, 2048, wl.BF16, s)
    mg.mgattn_attention_kv_ws(q, k, v, b, Hq * d, Hkv * d, Hkv * d, Hq * d, cq, ck, n, Hq, Hkv, d, 0.09, 2048, wl.BF16,
                              None, 0, s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
