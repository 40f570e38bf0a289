"""CPU tests of the C-ABI library: it loads, exports every function include/mgattn.h
declares, answers its pure host queries, refuses malformed calls by name before
touching a GPU, and splits work so that every (segment, head, q-tile) is computed
exactly once.  No compute call is made here (no GPU)."""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

from vit_perception_encoder_amd import mgattn as mg

pytestmark = pytest.mark.cpu
ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "mgattn.h"


@pytest.fixture(scope="module")
def lib():
    return mg.load_library()


def test_exports_every_declared_function(lib):
    decls = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(mgattn_[a-z_0-9]+)\s*\(", HEADER.read_text(), re.M))
    assert decls == set(mg.EXPORTS)
    for name in decls:
        assert hasattr(lib, name), name


def test_status_codes_match_header(lib):
    text = HEADER.read_text()
    for code, name in mg.STATUS_NAMES.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text), name
        s = mg.mgattn_strerror(code)
        assert s and s != "unknown mgattn status"
    assert mg.mgattn_strerror(12345) == "unknown mgattn status"


def test_supported_domain(lib):
    for d in (64, 96, 128):
        for dt in (mg.MGATTN_F32, mg.MGATTN_BF16):
            assert mg.mgattn_dense_supported(16, d, dt) == 1
            assert mg.mgattn_dense_supported(1, d, dt) == 1
    for d in (0, 32, 80, 95, 97, 160, 192, 256):
        assert mg.mgattn_dense_supported(16, d, mg.MGATTN_BF16) == 0
    assert mg.mgattn_dense_supported(0, 96, mg.MGATTN_BF16) == 0
    assert mg.mgattn_dense_supported(16, 96, 2) == 0


def test_lds_bytes_arithmetic(lib):
    """The LDS a workgroup asks for.  bf16: S stages of a 128-key K tile (pitch d+8)
    and a row-major 128-key V tile (pitch d), S = 3 when three stages fit the 160 KiB
    of one CU, else 2; at d=96 (the pipelined kernel) the 256-row Q tile, padded to
    pitch d+8, starts at the third stage and runs past it.  f32: two stages of 32-key K
    and V tiles (pitch d+4).  The bound is inclusive: d=96 bf16 asks for 155,648 bytes,
    inside 163,840."""
    for d in (64, 96, 128):
        stage = (128 * (d + 8) + 128 * d) * 2
        stages = 3 if 3 * stage <= 160 * 1024 else 2
        want_bf16 = stages * stage if d != 96 else max(3 * stage, 2 * stage + 256 * (d + 8) * 2)
        # f32: the largest of 128-query tiles (two stages of 32-key K and V tiles, pitch
        # d+4), the key-split 32-query blocks ((W-1) waves' partial results of d/32*4+1
        # float4 per lane, W = 8, or 4 at d = 128) and the key-split 16-query blocks
        # (7 waves' partial results of d/16+1 float4 per lane)
        want_f32 = max(2 * 2 * 32 * (d + 4) * 4, ((4 if d == 128 else 8) - 1) * (d // 32 * 4 + 1) * 64 * 16,
                       7 * (d // 16 + 1) * 64 * 16)
        assert mg.mgattn_dense_lds_bytes(d, mg.MGATTN_BF16) == want_bf16
        assert mg.mgattn_dense_lds_bytes(d, mg.MGATTN_F32) == want_f32
        assert want_bf16 <= 160 * 1024 and want_f32 <= 160 * 1024
    assert mg.mgattn_dense_lds_bytes(96, mg.MGATTN_BF16) == 155648
    assert mg.mgattn_dense_lds_bytes(128, mg.MGATTN_BF16) == 135168
    assert mg.mgattn_dense_lds_bytes(80, mg.MGATTN_BF16) == -3
    assert mg.mgattn_dense_lds_bytes(96, 7) == -2
    assert mg.mgattn_dense_block_m(96, mg.MGATTN_BF16) == 256
    assert mg.mgattn_dense_block_m(96, mg.MGATTN_F32) == 128


# Fake, aligned, non-overlapping "device" addresses: every call below is refused
# during argument checking, before any HIP call.
Q, K, V, O = 0x100000, 0x200000, 0x300000, 0x400000


def _call(cu, n_seg=None, H=16, d=96, scale=0.1, causal=0, dtype=1, q=Q, k=K, v=V, o=O):
    return mg.mgattn_dense(q, k, v, o, cu, len(cu) - 1 if n_seg is None else n_seg, H, d, scale,
                           causal, dtype, None, check=False)


@pytest.mark.parametrize("kwargs,status", [
    (dict(dtype=2), -2),
    (dict(q=0), -1), (dict(k=0), -1), (dict(v=0), -1), (dict(o=0), -1),
    (dict(n_seg=0), -6),
    (dict(H=0), -4),
    (dict(d=80), -3), (dict(d=256), -3),
    (dict(scale=float("nan")), -9), (dict(scale=float("inf")), -9), (dict(causal=2), -9),
    (dict(q=Q + 2), -8), (dict(o=O + 8), -8),
    (dict(o=Q + 16), -7), (dict(o=V - 16), -7),
])
def test_refusals(lib, kwargs, status):
    cu = [0, 64, 64, 200]
    assert _call(cu, **kwargs) == status


@pytest.mark.parametrize("cu", [[1, 10], [0, 10, 5], [0, 0], [0, 0, 0], [0, -5]])
def test_bad_seqlens(lib, cu):
    assert _call(cu) == -5


def test_null_seqlens(lib):
    st = lib.mgattn_dense(Q, K, V, O, None, 1, 16, 96, 0.1, 0, 1, None)
    assert st == -1


def test_segment_too_large(lib):
    # a 2^21-token segment of 16*96 bf16 spans 6 GiB: refused by name
    assert _call([0, 1 << 21], o=0x10_0000_0000) == -12


def _call_strided(ld, cu=(0, 64, 200), H=16, d=96, dtype=1, q=Q, k=K, v=V, o=O):
    ldq, ldk, ldv, ldo = ld
    return mg.mgattn_dense_strided(q, k, v, o, ldq, ldk, ldv, ldo, list(cu), len(cu) - 1, H, d, 0.1, 0, dtype,
                                   None, check=False)


@pytest.mark.parametrize("ld,dtype", [
    ((1535, 1536, 1536, 1536), 1),           # below H*d
    ((1536, 1536, 1536, 1540), 1),           # 1540 bf16 = 3080 bytes: not a multiple of 16
    ((1536, 1536, 1538, 1536), 0),           # f32: 1538 * 4 bytes is not a multiple of 16
    ((1536, 1536, 1536, 1 << 31), 1),        # above 2^31 - 1
])
def test_stride_refusals(lib, ld, dtype):
    assert _call_strided(ld, dtype=dtype) == -13


def test_strided_alias_spans(lib):
    """Merged q|k|v views of one [T, 3*H*d] buffer may overlap each other; out may
    not reach into any input's span [x, x + ((T-1)*ld + H*d) elements)."""
    T, row = 200, 1536
    base = 0x1000000
    ld3 = 3 * row
    q, k, v = base, base + 2 * row, base + 4 * row
    span = ((T - 1) * ld3 + row) * 2
    # (an out placed past every span is accepted: covered by the GPU merged-QKV test,
    # since an accepted call here would launch on these fake addresses)
    for o in (v + span - 16, q + 2 * row * 3, k + 16):
        assert mg.mgattn_dense_strided(q, k, v, o, ld3, ld3, ld3, row, [0, 64, T], 2, 16, 96, 0.1, 0, 1,
                                       None, check=False) == -7


def test_strided_segment_too_large(lib):
    # 2^19 tokens at a leading dimension of 3*1536 bf16 spans 4.5 GiB: refused by name
    ld3 = 3 * 1536
    assert _call_strided((ld3, ld3, ld3, 1536), cu=(0, 1 << 19), o=0x100_0000_0000) == -12


def _expected_tiles(cu, H, bm):
    out = set()
    for g in range(len(cu) - 1):
        L = cu[g + 1] - cu[g]
        for h in range(H):
            for q0 in range(0, L, bm):
                out.add((g, h, q0))
    return out


@pytest.mark.parametrize("cu,H,dtype,causal", [
    ([0, 4096], 16, 1, 0),
    ([0, 1024], 16, 1, 0),
    ([0, 1024, 2048], 16, 1, 1),
    ([0, 1024, 2048, 3072, 4096], 16, 1, 0),
    ([0, 12288, 16384, 17408], 16, 1, 0),
    ([0, 1, 1, 300, 557, 557, 1000], 3, 1, 1),
    ([0, 256], 16, 0, 0),
    ([0, 100, 357], 8, 0, 1),
])
def test_plan_is_a_bijection(lib, cu, H, dtype, causal):
    bm = mg.mgattn_dense_plan_block_m(cu, len(cu) - 1, H, 96, dtype, causal)
    grids = mg.mgattn_dense_plan(cu, len(cu) - 1, H, 96, dtype, causal)
    seen = []
    for li, grid in enumerate(grids):
        for b in range(grid):
            t = mg.mgattn_dense_tile(cu, len(cu) - 1, H, 96, dtype, causal, li, b)
            assert t is not None
            seen.append(t)
            if H % 8 == 0:
                assert t[1] % 8 == b % 8  # head dealt to XCD b % 8
    assert len(seen) == len(set(seen))
    assert set(seen) == _expected_tiles(cu, H, bm)


@pytest.mark.parametrize("cu,H,want,want_causal,want_f32", [
    ([0, 4096], 16, 256, 256, 128),       # the tower's full layer: 256 workgroups of 256 queries
    ([0, 1024, 2048, 3072, 4096], 16, 256, 256, 128),  # its window layer
    ([0, 1024], 16, 64, 128, 32),         # one 448x448 image: 64 units of 256, 256 of 64 (key-split)
    ([0, 2048], 16, 128, 128, 128),       # 128 units of 256, 256 of 128 (key-split)
    ([0, 256], 16, 64, 128, 16),          # the f32 workload: 32 units of 128, 128 of 32 (f32 key split)
    ([0, 100], 1, 64, 128, 16),           # nothing fills the chip: the shortest tile
    ([0, 1024] + [1024 + 64 * i for i in range(1, 49)], 16, 256, 256, 128),  # 49 segments x 16 heads
])
def test_plan_block_m_fills_the_chip(lib, cu, H, want, want_causal, want_f32):
    n = len(cu) - 1
    for causal, bm in ((0, want), (1, want_causal)):
        assert mg.mgattn_dense_plan_block_m(cu, n, H, 96, 1, causal) == bm
        assert mg.mgattn_dense_plan_block_m(cu, n, H, 64, 1, causal) == 256  # one tile height at d = 64
        # f32: 128-query tiles, or 32- or 16-query key-split blocks for a short non-causal call
        assert mg.mgattn_dense_plan_block_m(cu, n, H, 96, 0, causal) == (want_f32 if not causal else 128)
        assert sum(mg.mgattn_dense_plan(cu, n, H, 96, 1, causal)) == H * sum(
            -(-(cu[g + 1] - cu[g]) // bm) for g in range(n))


def test_plan_orders_longest_first_and_splits(lib):
    lens = list(np.random.Generator(np.random.PCG64(5)).integers(0, 700, size=300))
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    grids = mg.mgattn_dense_plan(cu, 300, 16, 96, 1, 0)
    nonempty = sum(1 for x in lens if x > 0)
    assert len(grids) == -(-nonempty // 120)
    assert sum(grids) == 16 * sum(-(-x // 256) for x in lens)
    # within XCD 0 of the first launch, segment lengths never increase
    prev = None
    for b in range(0, grids[0], 8):
        g, _, _ = mg.mgattn_dense_tile(cu, 300, 16, 96, 1, 0, 0, b)
        if prev is not None:
            assert lens[g] <= prev
        prev = lens[g]


def test_plan_causal_puts_last_qtile_first(lib):
    cu = [0, 1000]
    first = mg.mgattn_dense_tile(cu, 1, 1, 96, 1, 1, 0, 0)
    bm = mg.mgattn_dense_plan_block_m(cu, 1, 1, 96, 1, 1)
    assert bm == 128  # one head of 1000 tokens fills nothing: the shorter tile
    assert first == (0, 0, (999 // bm) * bm)
    assert mg.mgattn_dense_tile(cu, 1, 64, 96, 1, 1, 0, 0) == (0, 0, 768)  # 64 heads: tiles of 256


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        mg.load_library(tmp_path / "missing.so")


def _call_kv(cq=(0, 10, 30), ck=(0, 20, 50), Hq=32, Hkv=2, d=128, window=2048, dtype=1, ld=None,
             q=Q, k=K, v=V, o=O):
    ldq, ldk, ldv, ldo = ld or (Hq * d, Hkv * d, Hkv * d, Hq * d)
    return mg.mgattn_attention_kv(q, k, v, o, ldq, ldk, ldv, ldo, list(cq), list(ck), len(cq) - 1, Hq, Hkv, d, 0.1,
                                  window, dtype, None, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=3), -4), (dict(Hkv=0), -4), (dict(Hq=0), -4),
    (dict(window=-1), -15),
    (dict(ck=(0, 5, 50)), -5),                     # 5 keys for 10 queries
    (dict(ck=(1, 20, 50)), -5), (dict(ck=(0, 20, 0)), -5),
    (dict(ld=(4096, 255, 256, 4096)), -13),        # ldk below Hkv*d
    (dict(ld=(4095, 256, 256, 4096)), -13),
    (dict(d=80), -3), (dict(dtype=4), -2),
    (dict(o=K + 16), -7),                          # out inside k's span
])
def test_attention_kv_refusals(lib, kw, status):
    assert _call_kv(**kw) == status


def test_attention_kv_null_key_seqlens(lib):
    st = lib.mgattn_attention_kv(Q, K, V, O, 4096, 256, 256, 4096, (ctypes.c_int32 * 2)(0, 10), None, 1, 32, 2, 128,
                                 0.1, 2048, 1, None)
    assert st == -1


# ------------------------------------------------- decode workspace (host arithmetic)

def _dec_cu(n, lk):
    return list(range(n + 1)), [lk * i for i in range(n + 1)]


def test_workspace_bytes_of_the_text_decode_shape(lib):
    """32 sequences decoding one token over 4096 cached keys (32 query, 2 key/value
    heads, head size 128, window 2048): 64 (sequence, key/value head) pairs split 4
    ways fill the 256 CUs once; each split holds 32 columns of 128 floats + (M, den)."""
    cq, ck = _dec_cu(32, 4096)
    assert mg.mgattn_attention_kv_workspace(cq, ck, 32, 32, 2, 128, 2048, 1) == 32 * 2 * 4 * 32 * (128 + 2) * 4


@pytest.mark.parametrize("what,args,want", [
    ("prefill is not decoding", ([0, 10], [0, 10], 1, 32, 2, 128, 0, 1), 0),
    ("f32 has no split path", ([0, 1], [0, 4096], 1, 32, 2, 128, 0, 0), 0),
    # 120 sequences (one launch) x 4 key/value heads = 480 pairs: already one per CU
    ("enough pairs already", (list(range(121)), [4096 * i for i in range(121)], 120, 32, 4, 128, 0, 1), 0),
    # 128 sequences: launches of 120 and 8; the 8-sequence launch (16 pairs) is split
    ("a small second launch is split", (list(range(129)), [4096 * i for i in range(129)], 128, 32, 2, 128, 0, 1),
     8 * 2 * 16 * 32 * 130 * 4),
    ("under 8 blocks per split", ([0, 1], [0, 255], 1, 32, 2, 128, 0, 1), 0),
    ("window caps the visible keys", ([0, 1], [0, 100000], 1, 32, 2, 128, 256, 1), 0),
    # one pair, 2048 visible keys = 64 blocks: min(256, 64 / 8) = 8 splits
    ("window 2048, one sequence", ([0, 1], [0, 100000], 1, 32, 2, 128, 2048, 1), 2 * 8 * 32 * 130 * 4),
    # 2 pairs, 20000 keys = 625 blocks: min(128, 78, 16) = 16 splits
    ("split count capped at 16", ([0, 1], [0, 20000], 1, 8, 2, 64, 0, 1), 2 * 16 * 32 * 66 * 4),
])
def test_workspace_bytes_rules(lib, what, args, want):
    assert mg.mgattn_attention_kv_workspace(*args) == want, what


@pytest.mark.parametrize("args,status", [
    (([0, 1], [0, 10], 1, 32, 3, 128, 0, 1), -4),
    (([0, 1], [0, 10], 1, 32, 2, 128, -1, 1), -15),
    (([0, 1], [0, 10], 1, 32, 2, 80, 0, 1), -3),
    (([0, 1], [0, 10], 1, 32, 2, 128, 0, 7), -2),
    (([0, 2], [0, 1], 1, 32, 2, 128, 0, 1), -5),   # fewer keys than queries
    (([1, 2], [0, 10], 1, 32, 2, 128, 0, 1), -5),
    (([0, 1], [0, 10], 0, 32, 2, 128, 0, 1), -6),
])
def test_workspace_bytes_refusals(lib, args, status):
    assert mg.mgattn_attention_kv_workspace(*args) == status


def test_workspace_bytes_null_seqlens(lib):
    vp = ctypes.c_void_p
    assert lib.mgattn_attention_kv_workspace(None, vp(0), 1, 32, 2, 128, 0, 1) == -1


WS = 0x800000


@pytest.mark.parametrize("ws,nbytes,kw,status", [
    (WS + 16, 4096, {}, -8),           # workspace not 256-byte aligned
    (None, 4096, {}, -1),              # NULL with a size
    (K, 4096, {}, -7),                 # workspace overlaps k
    (O - 256, 4096, {}, -7),           # ... and out
    (WS, 4096, dict(Hkv=3), -4),       # every mgattn_attention_kv check still applies
    (WS, 4096, dict(window=-1), -15),
    (WS, 4096, dict(o=K + 16), -7),
])
def test_attention_kv_ws_refusals(lib, ws, nbytes, kw, status):
    a = dict(cq=(0, 1, 2), ck=(0, 20, 50), Hq=32, Hkv=2, d=128, window=2048)
    a.update(kw)
    o = a.pop("o", O)
    cq, ck = a["cq"], a["ck"]
    Hq, Hkv, d = a["Hq"], a["Hkv"], a["d"]
    st = mg.mgattn_attention_kv_ws(Q, K, V, o, Hq * d, Hkv * d, Hkv * d, Hq * d, list(cq), list(ck), len(cq) - 1, Hq,
                                   Hkv, d, 0.1, a["window"], 1, ws, nbytes, None, check=False)
    assert st == status


def test_dense_rope2d_refusals(lib):
    """The fused RoPE path is bf16 at head_dim 96; the images must hold the call's
    tokens; checks run before anything is launched (no GPU here)."""
    base = 1 << 20
    q, k, v, o = base, base + (1 << 24), base + (2 << 24), base + (3 << 24)
    row = 16 * 96

    def call(d=96, dtype=1, grids=((8, 8),), cu=(0, 64), win=4, theta=10000.0, H=16):
        r = H * d
        return mg.mgattn_dense_rope2d(q, k, v, o, r, r, r, r, list(cu), len(cu) - 1, H, d, 0.1, 0, dtype,
                                      list(grids), win, theta, None, check=False)
    assert call(dtype=0) == -2
    assert call(d=64) == -3
    assert call(d=80) == -3
    assert call(cu=(0, 63)) == -14       # the images hold 64 tokens
    assert call(grids=((8, 8), (2, 3)), cu=(0, 64)) == -14
    assert call(win=-1) == -14
    assert call(theta=1.0) == -9
    assert call(cu=(0, 70, 64)) == -5
