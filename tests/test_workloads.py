"""CPU tests of the seeded input generator and workload shapes, pinned to the pages'
printed numbers (tests/golden/pages_numbers.json) and to torch's bf16 rounding."""
from __future__ import annotations

import hashlib
import json
from pathlib import Path

import numpy as np
import pytest

from vit_perception_encoder_amd import workloads as wl

pytestmark = pytest.mark.cpu
GOLD = json.loads((Path(__file__).parent / "golden" / "pages_numbers.json").read_text())


def test_bf16_rne_matches_torch_and_hand_cases():
    torch = pytest.importorskip("torch")
    x = np.concatenate([
        wl.normal_f32(7, 200_000) * np.float32(3.0),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 1e-40, -1e-40, np.inf, -np.inf], np.float32),
        # exact ties: 1 + 2^-8 (rounds down to even 1.0), 1 + 3*2^-8 (rounds up to 1 + 2^-6)
        np.array([1.00390625, 1.01171875], np.float32),
    ])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert ours[-2] == 0x3F80 and ours[-1] == 0x3F82
    assert wl.f32_to_bf16_bits(np.array([np.nan], np.float32))[0] == 0x7FC0
    # widening is exact and inverts rounding of already-bf16 values
    assert np.array_equal(wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(ours)), ours)


def test_seeded_generation_is_deterministic():
    a = wl.normal_stored(201, 64, wl.BF16)
    b = wl.normal_stored(201, 64, wl.BF16)
    assert a.dtype == np.uint16 and a.shape == (64, 1536)
    assert hashlib.sha256(a.tobytes()).hexdigest() == hashlib.sha256(b.tobytes()).hexdigest()
    assert not np.array_equal(a, wl.normal_stored(202, 64, wl.BF16))
    f = wl.bf16_bits_to_f32(wl.normal_stored(201, 4096, wl.BF16))
    assert abs(float(f.mean())) < 0.01 and abs(float(f.std()) - 1.0) < 0.01


def test_layer_schedule_matches_pages():
    kinds = wl.tower_layer_kinds()
    full = [i for i, k in enumerate(kinds) if k == "full"]
    assert len(kinds) == GOLD["layers"]["value"]
    assert full == GOLD["full_attention_layers"]["value"]
    assert len(full) == GOLD["full_attention_layers"]["count_full"]
    assert kinds.count("window") == GOLD["full_attention_layers"]["count_window"]


def _iterations(case_lens_per_layer, H):
    return sum(H * sum(n * n for n in lens) for lens in case_lens_per_layer)


@pytest.mark.parametrize("reading", ["reading_A", "reading_B"])
def test_cost_model_iterations_match_pages(reading):
    """Q*H*K iteration counts of the 50-layer schedule at the pages' two grids."""
    g = GOLD[reading]
    gh, gw = g["grid"]
    H = GOLD["heads"]["value"]
    win = wl.window_lengths(gh, gw, GOLD["window_side"]["value"])
    assert len(win) == g["windows"]
    per_layer = [[gh * gw] if k == "full" else win for k in wl.tower_layer_kinds()]
    it = _iterations(per_layer, H)
    assert it == pytest.approx(g["iterations"], rel=5e-4)
    assert it * GOLD["naive_ns_per_iteration"]["value"] * 1e-9 == pytest.approx(g["seconds"], rel=5e-3)


def test_cost_table_rows():
    ns = GOLD["naive_ns_per_iteration"]["value"] * 1e-9
    H = GOLD["heads"]["value"]
    r1024 = GOLD["cost_table"]["rows"][0]
    assert 1024 * H * 1024 * ns * 1e3 == pytest.approx(r1024["per_call_ms"], rel=1e-3)
    assert 50 * 1024 * H * 1024 * ns == pytest.approx(r1024["per_tower_s"], rel=1e-2)
    r4096 = GOLD["cost_table"]["rows"][1]
    assert 4096 * H * 4096 * ns == pytest.approx(r4096["per_call_s"], rel=3e-2)
    # the tower figure at 4096 is the window-aware total (reading B)
    assert r4096["per_tower_s"] == pytest.approx(GOLD["reading_B"]["seconds"], rel=1e-2)


def test_tower_layer_cases():
    full = wl.tower_layer(3)
    win = wl.tower_layer(0)
    assert list(full.cu_seqlens) == [0, 4096]
    assert list(win.cu_seqlens) == [0, 1024, 2048, 3072, 4096]
    assert full.flops() == pytest.approx(103.079e9, rel=1e-4)
    assert win.flops() == pytest.approx(25.770e9, rel=1e-4)
    total = sum(4.0 * 16 * 96 * sum(n * n for n in np.diff(wl.tower_layer(l).cu_seqlens.astype(np.int64)))
                for l in (0, 3))
    assert total == pytest.approx(103.079e9 + 25.770e9, rel=1e-4)


def test_ragged_segments():
    a_full = wl.ragged_case("5a", "full", qkv=(None, None, None))
    assert list(np.diff(a_full.cu_seqlens)) == [12288, 4096, 1024]
    a_win = wl.ragged_case("5a", "window", qkv=(None, None, None))
    assert a_win.n_seg == 17 and set(np.diff(a_win.cu_seqlens)) == {1024}
    b_full = wl.ragged_case("5b", "full", qkv=(None, None, None))
    assert list(np.diff(b_full.cu_seqlens)) == [10752, 4032, 1600] and b_full.T == 16384
    b_win = wl.ragged_case("5b", "window", qkv=(None, None, None))
    assert b_win.n_seg == 22 and b_win.T == 16384
    assert set(np.diff(b_win.cu_seqlens)) == {1024, 768, 512, 256, 192, 64}


def test_row_scaling_is_exact_and_counted():
    x = wl.normal_stored(504, 1000, wl.BF16)
    y = wl.scale_rows_by_8(x, 9)
    changed = np.where((x != y).any(axis=1))[0]
    assert len(changed) == 50
    assert np.array_equal(wl.bf16_bits_to_f32(y[changed]), wl.bf16_bits_to_f32(x[changed]) * 8)


def test_sample_rows_cover_edges():
    cu = wl.cu_from_lengths([300, 1, 1024])
    toks, heads = wl.sample_rows(cu, 16, 10, 3)
    s = set(toks.tolist())
    for t in (0, 299, 300, 301, 1324, 255, 256, 301 + 255, 301 + 256):
        assert t in s
    assert heads.min() >= 0 and heads.max() < 16 and len(set(heads.tolist())) == 16
