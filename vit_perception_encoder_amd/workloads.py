"""Seeded synthetic inputs and workload shapes for the perception-encoder attention.

This module holds no attention arithmetic: it only draws inputs, rounds them to the
stored number type and lays out segment boundaries.  Both the HIP path (benchmark,
tests) and the f64 oracle (tests) consume its output, so it must stay free of any
step of the method itself.

Shapes come from the pages:
  * vllm.cpp issue #1545, "Why this one is bad": H=16 heads, head_dim=96, 50 layers,
    non-causal; its table pairs 1024 tokens (448x448 at patch 14) and 4096 tokens
    (896x896).
  * same issue, second comment, "Two of the three labelled uncertainties are now
    resolved": full attention at layers 3, 7, 11, ..., 47, 49 (13 layers) and window
    attention elsewhere (37 layers); a window is 32x32 = 1024 patches.
  * same comment, "The token count is still two readings": 16,384 patch tokens under
    the post-merge reading of max_image_tokens=4096.
The pages name no dataset: every tensor here is i.i.d. N(0,1) from a fixed seed.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HEADS = 16
HEAD_DIM = 96
N_LAYERS = 50
WINDOW = 32  # window side in patches
SCALE = 1.0 / math.sqrt(HEAD_DIM)

F32, BF16 = 0, 1  # dtype codes shared with the C ABI's enum values


# --------------------------------------------------------------------------- numbers

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bits (uint16) with round-to-nearest-even.

    NaN maps to the canonical quiet NaN 0x7FC0; infinities and overflow to inf follow
    from the integer rounding (a finite value that rounds past the largest bf16 gives
    the inf bit pattern, as IEEE round-to-nearest requires).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = r.copy()
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_f32(seed: int, shape) -> np.ndarray:
    """i.i.d. N(0,1) float32 from numpy's PCG64 with the given seed."""
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape, dtype=np.float32)


def normal_stored(seed: int, T: int, dtype: int, width: int = HEADS * HEAD_DIM) -> np.ndarray:
    """Seeded N(0,1) tensor [T, width] in its stored form: float32, or bf16 bits (uint16)."""
    x = normal_f32(seed, (T, width))
    return x if dtype == F32 else f32_to_bf16_bits(x)


def scale_rows_by_8(x: np.ndarray, seed: int, fraction: float = 0.05) -> np.ndarray:
    """Multiply ceil(fraction*T) distinct whole token rows (all heads) by 8.

    Rows are drawn without replacement from PCG64(seed).  Multiplying by 8 is exact in
    f32 and bf16 (it adds 3 to the exponent), so the stored bits stay exactly 8x.
    """
    T = x.shape[0]
    rows = np.random.Generator(np.random.PCG64(seed)).choice(T, size=math.ceil(fraction * T), replace=False)
    y = x.copy()
    if y.dtype == np.uint16:
        f = bf16_bits_to_f32(y[rows]) * np.float32(8.0)
        y[rows] = f32_to_bf16_bits(f)
    else:
        y[rows] = y[rows] * np.float32(8.0)
    return y


# ------------------------------------------------------------------------ segmentation

def cu_from_lengths(lengths) -> np.ndarray:
    """cu_seqlens (int32, n+1 entries, starting at 0) from segment lengths."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("token count does not fit int32")
    return cu.astype(np.int32)


def window_lengths(grid_h: int, grid_w: int, win: int = WINDOW) -> list[int]:
    """Token count of each window of a grid_h x grid_w patch grid, windows clipped at
    the bottom and right edges, in row-major window order."""
    out = []
    for r0 in range(0, grid_h, win):
        for c0 in range(0, grid_w, win):
            out.append(min(win, grid_h - r0) * min(win, grid_w - c0))
    return out


def tower_layer_kinds(n_layers: int = N_LAYERS) -> list[str]:
    """'full' at layers 3, 7, 11, ... and at the last layer; 'window' elsewhere."""
    return ["full" if (l % 4 == 3 or l == n_layers - 1) else "window" for l in range(n_layers)]


# ----------------------------------------------------------------------------- configs

@dataclass
class Case:
    """One call's inputs: stored Q/K/V [T, H*d] and the segment table."""
    name: str
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    cu_seqlens: np.ndarray
    dtype: int
    H: int = HEADS
    d: int = HEAD_DIM
    scale: float = SCALE
    causal: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_seg(self) -> int:
        return len(self.cu_seqlens) - 1

    def flops(self) -> float:
        """Algorithmic FLOP: 4 * S_q * S_k * d * H per segment (causal: half the square
        plus the diagonal)."""
        lens = np.diff(self.cu_seqlens.astype(np.int64))
        if self.causal:
            pairs = (lens * (lens + 1) // 2).sum()
        else:
            pairs = (lens * lens).sum()
        return 4.0 * float(pairs) * self.d * self.H


def _qkv(seeds, T, dtype):
    return tuple(normal_stored(s, T, dtype) for s in seeds)


def config_tiny() -> Case:
    """One 256-token segment, f32."""
    q, k, v = _qkv((101, 102, 103), 256, F32)
    return Case("tiny_f32_256", q, k, v, cu_from_lengths([256]), F32)


def config_full448() -> Case:
    """Full-attention layer at 448x448: one 1024-token segment, bf16."""
    q, k, v = _qkv((201, 202, 203), 1024, BF16)
    return Case("full_1024", q, k, v, cu_from_lengths([1024]), BF16)


def config_window896() -> Case:
    """Window layer at 896x896: a 64x64 grid as four 32x32 windows, bf16."""
    q, k, v = _qkv((301, 302, 303), 4096, BF16)
    return Case("window_4x1024", q, k, v, cu_from_lengths(window_lengths(64, 64)), BF16)


def tower_layer(layer: int, n_tokens_side: int = 64) -> Case:
    """Layer `layer` of the 50-layer schedule at a 64x64 grid (4096 tokens)."""
    T = n_tokens_side * n_tokens_side
    kind = tower_layer_kinds()[layer]
    q, k, v = _qkv((4000 + 3 * layer, 4001 + 3 * layer, 4002 + 3 * layer), T, BF16)
    lens = [T] if kind == "full" else window_lengths(n_tokens_side, n_tokens_side)
    return Case(f"tower_l{layer:02d}_{kind}", q, k, v, cu_from_lengths(lens), BF16,
                meta={"layer": layer, "kind": kind})


RAGGED_GRIDS = {
    # literal shapes: 128x96 + 64x64 + 32x32 = 17,408 tokens, whole windows only
    "5a": ((128, 96), (64, 64), (32, 32)),
    # literal 16,384 total with partial edge windows: 112x96 + 72x56 + 40x40
    "5b": ((112, 96), (72, 56), (40, 40)),
}
RAGGED_SEEDS = {"5a": (501, 502, 503, 504, 505), "5b": (511, 512, 513, 514, 515)}


def ragged_inputs(which: str):
    """Stored Q, K, V for a multi-image batch, with 5% of Q rows and (independently)
    5% of K rows scaled by 8.  V is left as drawn."""
    grids = RAGGED_GRIDS[which]
    sq, sk, sv, mq, mk = RAGGED_SEEDS[which]
    T = sum(h * w for h, w in grids)
    q, k, v = _qkv((sq, sk, sv), T, BF16)
    return scale_rows_by_8(q, mq), scale_rows_by_8(k, mk), v


def ragged_case(which: str, kind: str, qkv=None) -> Case:
    """Full layer: one segment per image.  Window layer: each image's clipped windows."""
    grids = RAGGED_GRIDS[which]
    q, k, v = qkv if qkv is not None else ragged_inputs(which)
    if kind == "full":
        lens = [h * w for h, w in grids]
    else:
        lens = [n for h, w in grids for n in window_lengths(h, w)]
    return Case(f"ragged{which}_{kind}", q, k, v, cu_from_lengths(lens), BF16,
                meta={"grids": grids, "kind": kind})


# --------------------------------------------------------------------- sampled checks

def sample_rows(cu_seqlens, H: int, n_random: int, seed: int, tile_edges=(32, 64, 128, 256)):
    """(token, head) pairs for checking a large output row by row: each segment's first
    and last tokens, tokens on both sides of every multiple of each tile edge up to a
    cap, plus n_random uniform draws.  Heads cycle so every head is covered."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    toks = []
    for g in range(len(cu) - 1):
        a, b = int(cu[g]), int(cu[g + 1])
        if b <= a:
            continue
        toks += [a, b - 1]
        for e in tile_edges:
            for m in range(e, min(b - a, 8 * e) + 1, e):
                for t in (a + m - 1, a + m):
                    if a <= t < b:
                        toks.append(t)
    rng = np.random.Generator(np.random.PCG64(seed))
    T = int(cu[-1])
    if n_random > 0 and T > 0:
        toks += rng.integers(0, T, size=n_random).tolist()
    toks = np.asarray(toks, dtype=np.int64)
    heads = (np.arange(len(toks)) * 7 + rng.integers(0, H)) % H
    return toks, heads.astype(np.int32)
