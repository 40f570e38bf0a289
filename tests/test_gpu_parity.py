"""GPU parity: the HIP path (through the C ABI) against the f64 oracle on the same
seeded inputs.  Tolerances: max |GPU - oracle| <= 2e-2 for bf16 inputs (f32
accumulation) and <= 1e-4 for f32 inputs.

Small cases are compared element by element over the whole output.  Full-size cases
(the 50-layer tower at 4096 tokens, the ragged 16k/17k-token batches) run in the
same launch configuration as the benchmark: every layer on sampled rows the oracle
computes one by one (every segment's first and last rows, rows on both sides of each
q-tile edge, and random rows), and the largest layers (tower layers 3 and 0, both
ragged batches' full and window layers) on the whole output."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle as orc
from tests.gpu_helpers import BF16_TOL, F32_TOL, run, say
from vit_perception_encoder_amd import mgattn as mg
from vit_perception_encoder_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t

    assert t.cuda.is_available()
    mg.load_library()
    return t


def _tol(dtype):
    return BF16_TOL if dtype == wl.BF16 else F32_TOL


def _full_check(torch, case: wl.Case, guard_rows=3):
    say(f"{case.name}: T={case.T} n_seg={case.n_seg} H={case.H} d={case.d} dtype={case.dtype} causal={case.causal}")
    got, guards = run(torch, case.q, case.k, case.v, case.cu_seqlens, case.H, case.d, case.scale,
                      case.causal, case.dtype, guard_rows=guard_rows)
    q, k, v = (x.reshape(case.T, case.H, case.d) for x in (case.q, case.k, case.v))
    want = orc.attention(q, k, v, case.cu_seqlens, case.H, case.d, case.scale, causal=bool(case.causal))
    err = np.abs(got - want)
    worst = np.unravel_index(int(np.argmax(err)), err.shape)
    assert guards, "kernel wrote outside out"
    assert np.all(np.isfinite(got))
    assert err.max() <= _tol(case.dtype), f"max err {err.max():.3e} at (t,h,c)={worst}"
    return got, want


def _sampled_check(torch, case: wl.Case, n_random=256, seed=0):
    say(f"{case.name} (sampled): T={case.T} n_seg={case.n_seg}")
    got, guards = run(torch, case.q, case.k, case.v, case.cu_seqlens, case.H, case.d, case.scale,
                      case.causal, case.dtype, guard_rows=2)
    assert guards
    assert np.all(np.isfinite(got))
    toks, heads = wl.sample_rows(case.cu_seqlens, case.H, n_random, seed)
    q, k, v = (x.reshape(case.T, case.H, case.d) for x in (case.q, case.k, case.v))
    want = orc.attention_rows(q, k, v, case.cu_seqlens, case.H, case.d, case.scale, toks, heads,
                              causal=bool(case.causal))
    err = np.abs(got[toks, heads] - want)
    i = int(np.argmax(err.max(axis=1)))
    assert err.max() <= _tol(case.dtype), f"max err {err.max():.3e} at token {toks[i]} head {heads[i]}"
    return err.max()


# ------------------------------------------------------------------ the five workloads

def test_config1_tiny_f32(torch):
    _full_check(torch, wl.config_tiny())


def test_config2_full_1024(torch):
    _full_check(torch, wl.config_full448())


def test_config3_window_4x1024(torch):
    _full_check(torch, wl.config_window896())


def test_config4_tower_50_layers(torch):
    """All 50 layers at 4096 tokens, fresh inputs per layer, sampled rows per layer."""
    worst = 0.0
    for layer in range(wl.N_LAYERS):
        worst = max(worst, _sampled_check(torch, wl.tower_layer(layer), n_random=48, seed=layer))
    say(f"tower worst sampled error {worst:.3e}")


@pytest.mark.parametrize("which", ["5a", "5b"])
def test_config5_ragged(torch, which):
    qkv = wl.ragged_inputs(which)
    for kind in ("full", "window"):
        _sampled_check(torch, wl.ragged_case(which, kind, qkv), n_random=256, seed=7)


# ------------------------------------------------- whole outputs at the full sizes
# The sampled checks above run every layer; these compare every element of the
# largest layers against the oracle (about a minute of oracle time on 16 host cores).

@pytest.mark.parametrize("layer", [3, 0])
def test_config4_tower_layers_whole_output(torch, layer):
    """Tower layer 3 (one 4096-token segment) and layer 0 (four 1024-token windows),
    every element, in the benchmark's launch configuration."""
    _full_check(torch, wl.tower_layer(layer), guard_rows=2)


@pytest.mark.parametrize("which,kind", [("5a", "full"), ("5a", "window"), ("5b", "full"), ("5b", "window")])
def test_config5_ragged_whole_output(torch, which, kind):
    """The ragged multi-image batches (segments of 12,288 / 10,752 tokens and clipped
    windows, 5% of Q and K rows scaled x8), every element."""
    _full_check(torch, wl.ragged_case(which, kind, wl.ragged_inputs(which)), guard_rows=2)


# ------------------------------------------------------------------------ edge cases

def _rand_case(name, lens, H=16, d=96, dtype=wl.BF16, causal=0, scale=None, seed=0, qscale=1.0, kscale=1.0):
    T = int(sum(lens))
    q = wl.normal_f32(seed, (T, H * d)) * np.float32(qscale)
    k = wl.normal_f32(seed + 1, (T, H * d)) * np.float32(kscale)
    v = wl.normal_f32(seed + 2, (T, H * d))
    if dtype == wl.BF16:
        q, k, v = (wl.f32_to_bf16_bits(x) for x in (q, k, v))
    return wl.Case(name, q, k, v, wl.cu_from_lengths(lens), dtype, H=H, d=d,
                   scale=(1.0 / np.sqrt(d)) if scale is None else scale, causal=causal)


RAGGED = [1, 2, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 600]


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
@pytest.mark.parametrize("causal", [0, 1])
def test_ragged_lengths(torch, dtype, causal):
    _full_check(torch, _rand_case(f"ragged_{dtype}_{causal}", RAGGED, H=4, dtype=dtype, causal=causal, seed=11))


SPLIT_EDGES = [1, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 1023, 1024, 1025]


def test_key_split_tile_edges(torch):
    """Launches too small to fill the chip split each tile's keys between two wave
    groups (64 keys of every 128 each) and merge their (m, l, O): segments ending on
    both sides of every half-tile edge, including ones where the second group sees no
    key at all."""
    case = _rand_case("split_edges", SPLIT_EDGES, H=2, seed=15)
    assert mg.mgattn_dense_plan_block_m(case.cu_seqlens, case.n_seg, 2, 96, wl.BF16, 0) == 64
    _full_check(torch, case)


def test_key_split_large_logits(torch):
    """Key-split merge with maxima far apart: keys scaled x8 (scores with a standard
    deviation near 8), so the two groups' running maxima differ by several units and
    each group's lazy rescaling fires on its own."""
    case = _rand_case("split_logits", [1024, 700], H=4, seed=16, kscale=8.0)
    assert mg.mgattn_dense_plan_block_m(case.cu_seqlens, case.n_seg, 4, 96, wl.BF16, 0) == 64
    _full_check(torch, case)


@pytest.mark.parametrize("H,bm", [(8, 32), (2, 16)])
def test_f32_key_split_long_segments(torch, H, bm):
    """f32 calls too short to fill the chip run 32-query blocks (eight heads: 552 of
    them) or, when those leave CUs idle too, 16-query blocks (two heads: 138 blocks of
    32) with the keys split over eight waves (four at head_dim 128 with 32-query
    blocks): long segments give every wave several 32-key tiles, short ones leave waves
    without tiles; keys scaled x4 so the waves' maxima differ.  Tolerance 1e-4 (f32)."""
    for d in (64, 96, 128):
        case = _rand_case(f"f32_split{bm}_d{d}", [2047, 33, 1, 0, 64], H=H, d=d, dtype=wl.F32, seed=18, kscale=4.0)
        assert mg.mgattn_dense_plan_block_m(case.cu_seqlens, case.n_seg, H, d, wl.F32, 0) == bm
        _full_check(torch, case)


def test_key_split_128_query_tiles(torch):
    """One 2048-token segment of 16 heads: 128 units of 256 queries, 256 of 128, so
    128-query tiles with the keys split between two groups of four waves."""
    case = _rand_case("split_2048", [2048], H=16, seed=17)
    assert mg.mgattn_dense_plan_block_m(case.cu_seqlens, case.n_seg, 16, 96, wl.BF16, 0) == 128
    _full_check(torch, case)


@pytest.mark.parametrize("d", [64, 96, 128])
@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_head_dims(torch, d, dtype):
    _full_check(torch, _rand_case(f"d{d}", [300, 77, 513], H=2, d=d, dtype=dtype, seed=21))


@pytest.mark.parametrize("H", [1, 3, 8, 16])
def test_head_counts(torch, H):
    _full_check(torch, _rand_case(f"H{H}", [257, 100], H=H, seed=31))


def test_empty_segments(torch):
    _full_check(torch, _rand_case("empties", [0, 40, 0, 0, 300, 0], H=3, seed=41))


@pytest.mark.parametrize("scale", [0.0, -0.3, 1.7])
def test_scales(torch, scale):
    _full_check(torch, _rand_case(f"scale{scale}", [130, 270], H=2, scale=scale, seed=51))


@pytest.mark.parametrize("case_seed", list(range(701, 713)))
def test_random_segment_tables(torch, case_seed):
    """Seeded random combinations of every parameter at once: 1-10 segments whose
    lengths mix empty, single-token, tile-edge (63..65, 255..257) and ragged ones;
    1-16 heads; head_dim 64/96/128; bf16 or f32; causal or not; scale of either sign.
    Whole outputs against the oracle."""
    rng = np.random.Generator(np.random.PCG64(case_seed))
    pool = [0, 1, 2, 31, 63, 64, 65, 255, 256, 257, 511, 777, 1024, 1300]
    lens = [int(rng.choice(pool)) if rng.random() < 0.6 else int(rng.integers(1, 1400))
            for _ in range(int(rng.integers(1, 11)))]
    while sum(lens) > 2600:
        lens.pop()
    if sum(lens) == 0:
        lens.append(97)
    H = int(rng.choice([1, 2, 3, 5, 8, 16]))
    d = int(rng.choice([64, 96, 128]))
    dtype = wl.BF16 if rng.random() < 0.75 else wl.F32
    causal = int(rng.random() < 0.4)
    scale = float(rng.choice([-1.0, 1.0]) * rng.uniform(0.02, 0.25))
    _full_check(torch, _rand_case(f"random{case_seed}", lens, H=H, d=d, dtype=dtype, causal=causal, scale=scale,
                                  seed=case_seed))


def test_many_segments_split_over_launches(torch):
    lens = np.random.Generator(np.random.PCG64(61)).integers(0, 90, size=300).tolist()
    case = _rand_case("300_segments", lens, H=2, seed=61)
    assert len(mg.mgattn_dense_plan(case.cu_seqlens, case.n_seg, 2, 96, wl.BF16)) == 3
    _full_check(torch, case)


def test_large_logits(torch):
    """Rows scaled by 8 on both Q and K: logits with std ~64, sharp softmax."""
    _full_check(torch, _rand_case("sharp", [700, 300], H=2, seed=71, qscale=8.0, kscale=8.0))


def test_single_key_segments_return_v_exactly(torch):
    case = _rand_case("single_keys", [1, 1, 5, 1], H=4, seed=81, qscale=4.0, kscale=4.0)
    got, _ = run(torch, case.q, case.k, case.v, case.cu_seqlens, 4, 96, case.scale, 0, wl.BF16)
    v = wl.bf16_bits_to_f32(case.v).reshape(case.T, 4, 96).astype(np.float64)
    for t in (0, 1, 7):
        assert np.array_equal(got[t], v[t])


def test_identical_keys_give_mean_of_v(torch):
    H, d, lens = 2, 96, [200, 333]
    case = _rand_case("identical_keys", lens, H=H, seed=91)
    k = case.k.reshape(case.T, H * d).copy()
    k[:200] = k[0]
    k[200:] = k[200]
    got, _ = run(torch, case.q, k, case.v, case.cu_seqlens, H, d, case.scale, 0, wl.BF16)
    v = wl.bf16_bits_to_f32(case.v).reshape(case.T, H, d).astype(np.float64)
    for a, b in ((0, 200), (200, 533)):
        assert np.abs(got[a:b] - v[a:b].mean(axis=0)).max() <= BF16_TOL


def test_key_shift_invariance_stress(torch):
    """Keys shifted by a large common vector (max-subtraction stress): the GPU still
    matches the oracle on the same stored keys."""
    H, d = 2, 96
    case = _rand_case("shifted", [512, 129], H=H, seed=101)
    kf = wl.bf16_bits_to_f32(case.k).reshape(case.T, H * d) + wl.normal_f32(102, (1, H * d)) * np.float32(6.0)
    case.k = wl.f32_to_bf16_bits(kf)
    _full_check(torch, case)


def test_segment_independence_and_determinism(torch):
    """A segment's output does not depend on the other segments of the call, bit for
    bit, among calls that run the same workgroup shape.  The shape follows the call's
    size (four 1024-token windows of 16 heads run 256-query tiles, one window alone
    runs 64-query key-split tiles), and across shapes the sums are taken in another
    order, so the outputs agree to rounding (each is checked against the oracle
    elsewhere).  256-query shape: the window layer against its windows in reverse
    order; key-split shape: four heads, each window alone against the four together."""
    case = wl.config_window896()
    say("segment independence")
    cu = [int(x) for x in case.cu_seqlens]
    got, _ = run(torch, case.q, case.k, case.v, cu, 16, 96, case.scale, 0, wl.BF16)
    again, _ = run(torch, case.q, case.k, case.v, cu, 16, 96, case.scale, 0, wl.BF16)
    assert np.array_equal(got, again)
    assert mg.mgattn_dense_plan_block_m(cu, 4, 16, 96, wl.BF16, 0) == 256
    order = [3, 2, 1, 0]
    rq, rk, rv = (np.concatenate([x[cu[g]:cu[g + 1]] for g in order]) for x in (case.q, case.k, case.v))
    rev, _ = run(torch, rq, rk, rv, cu, 16, 96, case.scale, 0, wl.BF16)
    for i, g in enumerate(order):
        assert np.array_equal(rev[cu[i]:cu[i + 1]], got[cu[g]:cu[g + 1]])
    # four heads: every call below runs the key-split shape
    q4, k4, v4 = (np.ascontiguousarray(x.reshape(case.T, 16, 96)[:, :4, :].reshape(case.T, 4 * 96))
                  for x in (case.q, case.k, case.v))
    assert mg.mgattn_dense_plan_block_m(cu, 4, 4, 96, wl.BF16, 0) == 64
    assert mg.mgattn_dense_plan_block_m([0, 1024], 1, 4, 96, wl.BF16, 0) == 64
    all4, _ = run(torch, q4, k4, v4, cu, 4, 96, case.scale, 0, wl.BF16)
    for g in range(4):
        a, b = cu[g], cu[g + 1]
        one, _ = run(torch, q4[a:b], k4[a:b], v4[a:b], [0, b - a], 4, 96, case.scale, 0, wl.BF16)
        assert np.array_equal(one, all4[a:b])


def test_runtime_refusals_on_device(torch):
    q = torch.zeros(64 * 1536 + 8, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(64 * 1536, dtype=torch.bfloat16, device="cuda")
    st = mg.mgattn_dense(q[1:], q, q, o, [0, 64], 1, 16, 96, 0.1, 0, wl.BF16, check=False)
    assert st == -8
    st = mg.mgattn_dense(q, q, q, q, [0, 64], 1, 16, 96, 0.1, 0, wl.BF16, check=False)
    assert st == -7
    with pytest.raises(mg.MgattnError):
        mg.mgattn_dense(q, q, q, o, [0, 64, 10], 2, 16, 96, 0.1, 0, wl.BF16)


def test_graph_capture_replays_match_eager(torch):
    """mgattn_dense captured into a HIP graph (three launches: 300 segments) replays
    to the eager result, bit for bit, with unrelated eager work and synchronisations
    between the replays."""
    from tests.gpu_helpers import to_device

    lens = np.random.Generator(np.random.PCG64(111)).integers(0, 200, size=300).tolist()
    case = _rand_case("graph", lens, H=2, seed=111)
    want, _ = run(torch, case.q, case.k, case.v, case.cu_seqlens, 2, 96, case.scale, 0, wl.BF16)
    qd, kd, vd = (to_device(x, torch) for x in (case.q, case.k, case.v))
    out = torch.zeros(case.T, 2 * 96, dtype=torch.bfloat16, device="cuda")
    cu = [int(x) for x in case.cu_seqlens]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mg.mgattn_dense(qd, kd, vd, out, cu, case.n_seg, 2, 96, case.scale, 0, wl.BF16, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.mgattn_dense(qd, kd, vd, out, cu, case.n_seg, 2, 96, case.scale, 0, wl.BF16,
                        torch.cuda.current_stream())
    other = wl.config_full448()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        from tests.gpu_helpers import from_device
        got = from_device(out, torch).reshape(case.T, 2, 96)
        assert np.array_equal(got, want), f"replay {rep} differs from eager"
        # eager work between replays
        run(torch, other.q, other.k, other.v, other.cu_seqlens, 16, 96, other.scale, 0, wl.BF16)


def test_graph_capture_f32_key_split(torch):
    """The f32 workload (one 256-token segment of 16 heads: 16-query key-split blocks)
    captured into a HIP graph replays to the eager result bit for bit."""
    from tests.gpu_helpers import from_device, to_device

    case = wl.config_tiny()
    assert mg.mgattn_dense_plan_block_m(case.cu_seqlens, case.n_seg, 16, 96, wl.F32, 0) == 16
    want, _ = run(torch, case.q, case.k, case.v, case.cu_seqlens, 16, 96, case.scale, 0, wl.F32)
    qd, kd, vd = (to_device(x, torch) for x in (case.q, case.k, case.v))
    out = torch.zeros(case.T, 16 * 96, dtype=torch.float32, device="cuda")
    cu = [int(x) for x in case.cu_seqlens]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mg.mgattn_dense(qd, kd, vd, out, cu, case.n_seg, 16, 96, case.scale, 0, wl.F32, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph capture, f32 key split")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.mgattn_dense(qd, kd, vd, out, cu, case.n_seg, 16, 96, case.scale, 0, wl.F32, torch.cuda.current_stream())
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_device(out, torch).reshape(want.shape), want), f"replay {rep} differs from eager"


def test_graph_capture_key_split_shapes(torch):
    """Both key-split shapes captured into one HIP graph (a 1024-token segment of 16
    heads: 64-query tiles; a 2048-token one: 128-query tiles) replay to the eager
    results bit for bit, with eager work between the replays."""
    from tests.gpu_helpers import from_device, to_device

    cases = [_rand_case("graph_split64", [1024], H=16, seed=121), _rand_case("graph_split128", [2048], H=16, seed=122)]
    for c, bm in zip(cases, (64, 128)):
        assert mg.mgattn_dense_plan_block_m(c.cu_seqlens, 1, 16, 96, wl.BF16, 0) == bm
    wants = [run(torch, c.q, c.k, c.v, c.cu_seqlens, 16, 96, c.scale, 0, wl.BF16)[0] for c in cases]
    dev = [tuple(to_device(x, torch) for x in (c.q, c.k, c.v)) for c in cases]
    outs = [torch.zeros(c.T, 16 * 96, dtype=torch.bfloat16, device="cuda") for c in cases]
    cus = [[int(x) for x in c.cu_seqlens] for c in cases]

    def launch(stream):
        for (q, k, v), o, cu, c in zip(dev, outs, cus, cases):
            mg.mgattn_dense(q, k, v, o, cu, 1, 16, 96, c.scale, 0, wl.BF16, stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    say("graph capture, key-split shapes")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(torch.cuda.current_stream())
    other = wl.config_window896()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, c, want in zip(outs, cases, wants):
            got = from_device(o, torch).reshape(c.T, 16, 96)
            assert np.array_equal(got, want), f"{c.name}: replay {rep} differs from eager"
        run(torch, other.q, other.k, other.v, other.cu_seqlens, 16, 96, other.scale, 0, wl.BF16)
