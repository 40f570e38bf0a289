"""Plain numpy oracle of causal sliding-window attention with grouped key/value heads
over a key/value cache: the attention of the Muse Glimmer text decoder (mbext
next-steps page, "Architecture / Text decoder": 32 query heads, 2 key/value heads,
head size 128, a local attention window of 2048 tokens on sliding layers; prefill and
incremental decoding with a KV cache).

TEST INFRASTRUCTURE ONLY: imported by the test suite and the benchmark, never by the
product path.  It shares no code with the HIP library and never imports the
``vit_perception_encoder_amd`` package.

Readings where the page is silent: query head h reads key/value head h // (Hq / Hkv)
(consecutive query heads share a key/value head); the window of W tokens holds the
query's own key and the W-1 keys before it (W == 0: no window); the new queries of a
sequence are its last Lq positions, so query i sits at position Lk - Lq + i.
Everything is evaluated in f64 from the given values: a dense masked score matrix per
(sequence, head), max subtraction, exponentials, normalisation.
"""
from __future__ import annotations

import numpy as np


def allowed_keys(Lq, Lk, window):
    """Boolean [Lq, Lk]: key j is visible to query i."""
    pos = (Lk - Lq) + np.arange(Lq)[:, None]
    j = np.arange(Lk)[None, :]
    ok = j <= pos
    if window > 0:
        ok &= j > pos - window
    return ok


def attention_kv(q, k, v, cu_q, cu_k, Hq, Hkv, d, scale, window):
    """q: [Tq, >= Hq*d], k, v: [Tk, >= Hkv*d] (values widened to f64).  Returns the
    output [Tq, Hq, d] in f64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    group = Hq // Hkv
    out = np.zeros((int(cu_q[-1]), Hq, d))
    for s in range(len(cu_q) - 1):
        a, b = int(cu_q[s]), int(cu_q[s + 1])
        ka, kb = int(cu_k[s]), int(cu_k[s + 1])
        if b == a:
            continue
        ok = allowed_keys(b - a, kb - ka, window)
        for h in range(Hq):
            g = h // group
            Q = q[a:b, h * d:(h + 1) * d]
            K = k[ka:kb, g * d:(g + 1) * d]
            V = v[ka:kb, g * d:(g + 1) * d]
            S = np.where(ok, (Q @ K.T) * float(scale), -np.inf)
            m = S.max(axis=1, keepdims=True)
            P = np.exp(S - m)
            out[a:b, h] = (P / P.sum(axis=1, keepdims=True)) @ V
    return out
