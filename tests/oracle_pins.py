"""Pins that tie the f64 oracle to facts it does not compute itself.

Each pin takes a loaded oracle library (so the mutation test can run the same pins
against deliberately broken copies of the oracle) and raises AssertionError on a
mismatch.  The facts used:

  * softmax weights are a probability vector (V = 1 gives O = 1; weights sum to 1);
  * identical keys give the mean of V (causal: the running mean);
  * a segment of one token returns its V row exactly;
  * the first query of a causal segment returns that segment's first V row exactly;
  * permuting (K, V) rows jointly inside a segment changes nothing; permuting queries
    permutes the output;
  * adding one vector to every key of a segment changes nothing (it adds a per-query
    constant to the logits);
  * scale = 0 gives the mean of V;
  * two keys give sigma(delta) v1 + (1 - sigma(delta)) v2 (also at logits near 1000,
    where exp overflows unless the maximum is taken out first);
  * brute force with exact rational dot products and 50-digit exp on tiny inputs;
  * window segmentation equals full attention under a dense block-diagonal -inf mask
    evaluated with numpy;
  * a multi-segment call equals one call per segment, bit for bit.

Attention semantics follow vllm.cpp issue #1545 ("Muse Glimmer's vision tower runs 50
layers on the naive attention kernel"), sections "Why this one is bad" and "The fix".
"""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np

from oracle import oracle as orc

TIGHT = 1e-12


def _rand(shape, seed, scale=1.0):
    return (np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale).astype(np.float32)


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _run(lib, q, k, v, cu, H, d, scale, causal=False):
    return orc.attention(q, k, v, cu, H, d, scale, causal=causal, n_threads=2, lib=lib)


# ----------------------------------------------------------------------------- pins

def pin_ones_value(lib):
    """V = 1 everywhere -> O = 1 (the weights sum to one), ragged and causal."""
    H, d = 3, 8
    lens = [5, 1, 17, 40]
    T = sum(lens)
    q, k = _rand((T, H, d), 1), _rand((T, H, d), 2)
    v = np.ones((T, H, d), np.float32)
    for causal in (False, True):
        o = _run(lib, q, k, v, _cu(lens), H, d, 0.7, causal)
        assert np.max(np.abs(o - 1.0)) <= TIGHT, "V=1 did not give O=1"


def pin_weights_sum(lib):
    H, d = 2, 6
    lens = [9, 23]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 3), _rand((T, H, d), 4), _rand((T, H, d), 5)
    cu = _cu(lens)
    for causal in (False, True):
        for t in (0, 8, 9, 20, 31):
            w, _ = orc.weights(q, k, v, cu, H, d, 0.9, t, t % H, causal=causal, lib=lib)
            seg_start = 0 if t < 9 else 9
            seg_end = 9 if t < 9 else 32
            assert len(w) == (t + 1 - seg_start if causal else seg_end - seg_start)
            assert np.all(w >= 0.0) and abs(w.sum() - 1.0) <= TIGHT


def pin_identical_keys(lib):
    """All keys of a segment equal -> O = mean of the segment's V (causal: running mean)."""
    H, d = 2, 8
    lens = [7, 12]
    T = sum(lens)
    q, v = _rand((T, H, d), 6), _rand((T, H, d), 7)
    k = np.empty((T, H, d), np.float32)
    cu = _cu(lens)
    for g in range(len(lens)):
        k[cu[g]:cu[g + 1]] = _rand((1, H, d), 100 + g)
    o = _run(lib, q, k, v, cu, H, d, 1.3)
    oc = _run(lib, q, k, v, cu, H, d, 1.3, causal=True)
    v64 = v.astype(np.float64)
    for g in range(len(lens)):
        a, b = cu[g], cu[g + 1]
        assert np.max(np.abs(o[a:b] - v64[a:b].mean(axis=0))) <= TIGHT
        run_mean = np.cumsum(v64[a:b], axis=0) / np.arange(1, b - a + 1)[:, None, None]
        assert np.max(np.abs(oc[a:b] - run_mean)) <= TIGHT


def pin_single_key_segment(lib):
    """A one-token segment returns its own V row exactly, whatever Q and K hold."""
    H, d = 4, 8
    lens = [1, 3, 1, 1]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 8, 5.0), _rand((T, H, d), 9, 5.0), _rand((T, H, d), 10)
    o = _run(lib, q, k, v, _cu(lens), H, d, 2.0)
    for t in (0, 4, 5):
        assert np.array_equal(o[t], v[t].astype(np.float64))


def pin_causal_first_query(lib):
    """Causal: the first query of each segment sees only its own key -> its V row."""
    H, d = 2, 8
    lens = [6, 10, 3]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 11), _rand((T, H, d), 12), _rand((T, H, d), 13)
    cu = _cu(lens)
    o = _run(lib, q, k, v, cu, H, d, 1.0, causal=True)
    for g in range(len(lens)):
        assert np.array_equal(o[cu[g]], v[cu[g]].astype(np.float64))
    # the last query of a causal segment sees the whole segment
    on = _run(lib, q, k, v, cu, H, d, 1.0)
    for g in range(len(lens)):
        assert np.max(np.abs(o[cu[g + 1] - 1] - on[cu[g + 1] - 1])) <= TIGHT


def pin_key_permutation(lib):
    """Permuting (K, V) rows jointly inside a segment leaves O unchanged."""
    H, d = 2, 8
    lens = [11, 19]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 14), _rand((T, H, d), 15), _rand((T, H, d), 16)
    cu = _cu(lens)
    perm = np.arange(T)
    rng = np.random.Generator(np.random.PCG64(17))
    for g in range(len(lens)):
        perm[cu[g]:cu[g + 1]] = cu[g] + rng.permutation(lens[g])
    o = _run(lib, q, k, v, cu, H, d, 0.8)
    o2 = _run(lib, q, k[perm], v[perm], cu, H, d, 0.8)
    assert np.max(np.abs(o - o2)) <= TIGHT
    # and the permutation really moved keys across the whole segment
    assert not np.array_equal(perm, np.arange(T))


def pin_query_permutation(lib):
    """Permuting queries inside a segment permutes the output rows, bit for bit."""
    H, d = 2, 8
    lens = [13, 8]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 18), _rand((T, H, d), 19), _rand((T, H, d), 20)
    cu = _cu(lens)
    perm = np.arange(T)
    rng = np.random.Generator(np.random.PCG64(21))
    for g in range(len(lens)):
        perm[cu[g]:cu[g + 1]] = cu[g] + rng.permutation(lens[g])
    o = _run(lib, q, k, v, cu, H, d, 0.8)
    o2 = _run(lib, q[perm], k, v, cu, H, d, 0.8)
    assert np.array_equal(o[perm], o2)


def pin_shift_invariance(lib):
    """K' = K + 1 u^T per segment (u per head) leaves O unchanged (f64 inputs)."""
    H, d = 2, 8
    lens = [10, 14]
    T = sum(lens)
    q = _rand((T, H, d), 22).astype(np.float64)
    k = _rand((T, H, d), 23).astype(np.float64)
    v = _rand((T, H, d), 24).astype(np.float64)
    cu = _cu(lens)
    k2 = k.copy()
    for g in range(len(lens)):
        k2[cu[g]:cu[g + 1]] += _rand((1, H, d), 200 + g, 3.0).astype(np.float64)
    o = _run(lib, q, k, v, cu, H, d, 0.5)
    o2 = _run(lib, q, k2, v, cu, H, d, 0.5)
    assert np.max(np.abs(o - o2)) <= 1e-10


def pin_scale_zero(lib):
    """scale = 0 -> uniform weights -> mean of V over the keys seen."""
    H, d = 2, 8
    lens = [5, 16]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 25, 10.0), _rand((T, H, d), 26, 10.0), _rand((T, H, d), 27)
    cu = _cu(lens)
    o = _run(lib, q, k, v, cu, H, d, 0.0)
    v64 = v.astype(np.float64)
    for g in range(len(lens)):
        a, b = cu[g], cu[g + 1]
        assert np.max(np.abs(o[a:b] - v64[a:b].mean(axis=0))) <= TIGHT


def pin_two_keys_closed_form(lib):
    """Two keys: O = sigma(D) v1 + (1 - sigma(D)) v2, D = s1 - s2; includes logits
    near 1000 (exp overflows there unless the maximum is subtracted)."""
    H, d = 1, 4
    v = np.array([[[1.5, -2.0, 0.25, 3.0]], [[-0.5, 4.0, 1.0, -1.0]]], np.float32)
    for qv, k1, k2, scale in [((1, 0, 0, 0), (2, 0, 0, 0), (1, 0, 0, 0), 1.0),
                              ((1, 1, 0, 0), (0.5, 0, 0, 0), (0, -2, 0, 0), 0.75),
                              ((16, 0, 0, 0), (62.5, 0, 0, 0), (62.4375, 0, 0, 0), 1.0),
                              ((0, 0, 1, 0), (0, 0, -3, 0), (0, 0, 5, 0), 2.0)]:
        q = np.array([[qv], [qv]], np.float32)
        k = np.array([[k1], [k2]], np.float32)
        sc = float(np.float32(scale))
        s1 = sc * float(np.dot(np.float64(qv), np.float64(k1)))
        s2 = sc * float(np.dot(np.float64(qv), np.float64(k2)))
        sig = 1.0 / (1.0 + np.exp(-(s1 - s2)))
        want = sig * v[0, 0].astype(np.float64) + (1 - sig) * v[1, 0].astype(np.float64)
        o = _run(lib, q, k, v, _cu([2]), H, d, scale)
        assert np.all(np.isfinite(o)), "non-finite output on large logits"
        assert np.max(np.abs(o[0, 0] - want)) <= 1e-12 * max(1.0, np.abs(want).max())


def _exact_attention(q, k, v, cu, H, d, scale, causal):
    """Brute force: exact rational logits, 50-digit decimal exp and sums."""
    ctx = decimal.Context(prec=50)
    sc = Fraction(float(np.float32(scale)))
    T = int(cu[-1])
    out = np.zeros((T, H, d))
    for g in range(len(cu) - 1):
        a, b = int(cu[g]), int(cu[g + 1])
        for h in range(H):
            for i in range(a, b):
                keys = range(a, i + 1) if causal else range(a, b)
                logits = []
                for j in keys:
                    dot = sum(Fraction(float(q[i, h, c])) * Fraction(float(k[j, h, c])) for c in range(d))
                    logits.append(sc * dot)
                mx = max(logits)
                ws = [ctx.exp(ctx.divide(decimal.Decimal((s - mx).numerator), decimal.Decimal((s - mx).denominator)))
                      for s in logits]
                z = sum(ws, decimal.Decimal(0))
                for c in range(d):
                    acc = decimal.Decimal(0)
                    for w, j in zip(ws, keys):
                        acc += w * decimal.Decimal(float(v[j, h, c]))
                    out[i, h, c] = float(ctx.divide(acc, z))
    return out


def pin_brute_force_tiny(lib):
    """Exact evaluation on tiny ragged inputs, causal and not, f32 and bf16 storage."""
    from vit_perception_encoder_amd.workloads import f32_to_bf16_bits

    for seed, lens, H, d, causal in [(30, [3, 5], 2, 4, False), (31, [1, 7], 2, 3, True),
                                     (32, [8], 1, 4, False), (33, [2, 2, 4], 2, 2, True)]:
        T = sum(lens)
        q, k, v = _rand((T, H, d), seed, 2.0), _rand((T, H, d), seed + 50, 2.0), _rand((T, H, d), seed + 99)
        cu = _cu(lens)
        want = _exact_attention(q, k, v, cu, H, d, 0.6, causal)
        got = _run(lib, q, k, v, cu, H, d, 0.6, causal)
        assert np.max(np.abs(got - want)) <= 1e-13, f"brute force mismatch (seed {seed})"
        # the same values stored as bf16 bits must give the same answer as their exact
        # f32 widening
        qb, kb, vb = (f32_to_bf16_bits(x) for x in (q, k, v))
        widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
        want_b = _exact_attention(widen(qb), widen(kb), widen(vb), cu, H, d, 0.6, causal)
        got_b = _run(lib, qb, kb, vb, cu, H, d, 0.6, causal)
        assert np.max(np.abs(got_b - want_b)) <= 1e-13, f"bf16 brute force mismatch (seed {seed})"


def _window_lengths(gh, gw, win):
    return [min(win, gh - r) * min(win, gw - c) for r in range(0, gh, win) for c in range(0, gw, win)]


def pin_dense_mask(lib):
    """Window segmentation of a 64x48 grid (32x32 windows, clipped) equals full
    attention with a dense block-diagonal mask, evaluated with numpy in f64."""
    H, d = 2, 8
    lens = _window_lengths(64, 48, 32)
    assert lens == [1024, 512, 1024, 512]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 40), _rand((T, H, d), 41), _rand((T, H, d), 42)
    cu = _cu(lens)
    scale = 0.35
    seg = np.repeat(np.arange(len(lens)), lens)
    allowed = seg[:, None] == seg[None, :]
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    want = np.empty((T, H, d))
    for h in range(H):
        s = float(np.float32(scale)) * (q64[:, h, :] @ k64[:, h, :].T)
        s = np.where(allowed, s, -np.inf)
        s -= s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        want[:, h, :] = w @ v64[:, h, :]
    got = _run(lib, q, k, v, cu, H, d, scale)
    assert np.max(np.abs(got - want)) <= 1e-12


def pin_segment_independence(lib):
    """A call over [0,L0,L0+L1,...] equals one call per segment, bit for bit."""
    H, d = 2, 8
    lens = [31, 64, 1, 40]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 43), _rand((T, H, d), 44), _rand((T, H, d), 45)
    cu = _cu(lens)
    for causal in (False, True):
        o = _run(lib, q, k, v, cu, H, d, 0.4, causal)
        for g in range(len(lens)):
            a, b = cu[g], cu[g + 1]
            og = _run(lib, q[a:b], k[a:b], v[a:b], _cu([b - a]), H, d, 0.4, causal)
            assert np.array_equal(o[a:b], og)


def pin_rows_match_full(lib):
    """The row-sampling entry point returns exactly the rows of the full output."""
    H, d = 3, 8
    lens = [20, 1, 33]
    T = sum(lens)
    q, k, v = _rand((T, H, d), 46), _rand((T, H, d), 47), _rand((T, H, d), 48)
    cu = _cu(lens)
    toks = np.array([0, 19, 20, 21, 53, 30], np.int64)
    heads = np.array([0, 2, 1, 0, 2, 1], np.int32)
    for causal in (False, True):
        full = _run(lib, q, k, v, cu, H, d, 0.3, causal)
        rows = orc.attention_rows(q, k, v, cu, H, d, 0.3, toks, heads, causal=causal, n_threads=2, lib=lib)
        assert np.array_equal(rows, full[toks, heads])


ALL_PINS = [pin_ones_value, pin_weights_sum, pin_identical_keys, pin_single_key_segment,
            pin_causal_first_query, pin_key_permutation, pin_query_permutation,
            pin_shift_invariance, pin_scale_zero, pin_two_keys_closed_form,
            pin_brute_force_tiny, pin_dense_mask, pin_segment_independence, pin_rows_match_full]
