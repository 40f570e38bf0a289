"""Pins of the text-decoder attention oracle (oracle/gqa_window.py) to facts fixed
independently of it: the special case that is the (separately pinned) dense causal
oracle, closed forms (window 1 returns the own value row; identical keys return the
mean of the values over exactly the window), the head grouping read off constant
value heads, and prefill/decode consistency.  Plus a mutation battery: each plausible
slip must fail a pin.

Page: mbext next-steps page, "Architecture / Text decoder" (32 query heads, 2 key/value
heads, head size 128, local window of 2048 tokens; prefill and incremental decoding
with a KV cache)."""
from __future__ import annotations

import types
from pathlib import Path

import numpy as np
import pytest

from oracle import gqa_window as G
from oracle import oracle as orc

pytestmark = pytest.mark.cpu
SRC = (Path(__file__).resolve().parent.parent / "oracle" / "gqa_window.py").read_text()


def _rand(seed, shape):
    return np.random.default_rng(seed).standard_normal(shape)


def pin_dense_causal_special_case(g, lib):
    """Hkv == Hq, keys = queries, no window: the dense causal oracle (C, f64; its scale
    argument is f32, so the scale here is exact in f32)."""
    H, d, lens = 3, 16, [5, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = (_rand(s, (T, H * d)) for s in (1, 2, 3))
    got = g.attention_kv(q, k, v, cu, cu, H, H, d, 0.375, 0)
    want = orc.attention(*(x.reshape(T, H, d) for x in (q, k, v)), cu, H, d, 0.375, causal=True, lib=lib)
    assert np.abs(got - want).max() < 1e-12


def pin_window_one_is_own_value(g, lib):
    T, Hq, Hkv, d = 9, 4, 2, 8
    q, k, v = _rand(4, (T, Hq * d)), _rand(5, (T, Hkv * d)), _rand(6, (T, Hkv * d))
    got = g.attention_kv(q, k, v, [0, T], [0, T], Hq, Hkv, d, 0.5, 1)
    for h in range(Hq):
        gh = h // (Hq // Hkv)
        assert np.array_equal(got[:, h], v[:, gh * d:(gh + 1) * d])


def pin_identical_keys_average_the_window(g, lib):
    """All keys equal: uniform weights over the visible keys, i.e. the mean of v over
    [max(0, p - W + 1), p] -- pins both window bounds and the cache offset."""
    Lk, Lq, Hq, Hkv, d = 23, 7, 2, 1, 4
    q = _rand(7, (Lq, Hq * d))
    k = np.tile(_rand(8, (1, Hkv * d)), (Lk, 1))
    v = _rand(9, (Lk, Hkv * d))
    for W in (0, 1, 3, 5, 16, 17, 40):
        got = g.attention_kv(q, k, v, [0, Lq], [0, Lk], Hq, Hkv, d, 0.7, W)
        for i in range(Lq):
            p = Lk - Lq + i
            lo = 0 if W == 0 else max(0, p - W + 1)
            want = v[lo:p + 1].mean(axis=0)
            for h in range(Hq):
                assert np.abs(got[i, h] - want).max() < 1e-12


def pin_head_groups(g, lib):
    """Value head j constant j+1: query head h must return h // (Hq/Hkv) + 1."""
    T, Hq, Hkv, d = 6, 8, 2, 4
    q, k = _rand(10, (T, Hq * d)), _rand(11, (T, Hkv * d))
    v = np.repeat(np.arange(1, Hkv + 1, dtype=np.float64), d)[None, :].repeat(T, axis=0)
    got = g.attention_kv(q, k, v, [0, T], [0, T], Hq, Hkv, d, 1.0, 0)
    for h in range(Hq):
        assert np.abs(got[:, h] - (h // (Hq // Hkv) + 1)).max() < 1e-13


def pin_prefill_equals_decode(g, lib):
    """Row i of a prefill over N tokens = a one-token decode with a cache of i+1 keys;
    the last Lq rows of a prefill = a call with Lq new queries over the same cache."""
    N, Hq, Hkv, d, W = 20, 4, 2, 8, 6
    q, k, v = _rand(12, (N, Hq * d)), _rand(13, (N, Hkv * d)), _rand(14, (N, Hkv * d))
    full = g.attention_kv(q, k, v, [0, N], [0, N], Hq, Hkv, d, 0.4, W)
    for i in (0, 3, 5, 6, 19):
        one = g.attention_kv(q[i:i + 1], k[:i + 1], v[:i + 1], [0, 1], [0, i + 1], Hq, Hkv, d, 0.4, W)
        assert np.abs(one[0] - full[i]).max() < 1e-12
    tail = g.attention_kv(q[12:], k, v, [0, 8], [0, N], Hq, Hkv, d, 0.4, W)
    assert np.abs(tail - full[12:]).max() < 1e-12


def pin_sequences_are_independent(g, lib):
    Hq, Hkv, d, W = 2, 1, 4, 3
    lq, lk = [3, 0, 5], [4, 2, 9]
    cq = np.concatenate([[0], np.cumsum(lq)])
    ck = np.concatenate([[0], np.cumsum(lk)])
    q, k, v = _rand(15, (cq[-1], Hq * d)), _rand(16, (ck[-1], Hkv * d)), _rand(17, (ck[-1], Hkv * d))
    got = g.attention_kv(q, k, v, cq, ck, Hq, Hkv, d, 0.9, W)
    for s in range(3):
        one = g.attention_kv(q[cq[s]:cq[s + 1]], k[ck[s]:ck[s + 1]], v[ck[s]:ck[s + 1]], [0, lq[s]], [0, lk[s]],
                             Hq, Hkv, d, 0.9, W)
        assert np.array_equal(one, got[cq[s]:cq[s + 1]])


PINS = [pin_dense_causal_special_case, pin_window_one_is_own_value, pin_identical_keys_average_the_window,
        pin_head_groups, pin_prefill_equals_decode, pin_sequences_are_independent]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(G, oracle_lib)


MUTANTS = [
    ("window off by one", "ok &= j > pos - window", "ok &= j >= pos - window"),
    ("heads interleaved", "g = h // group", "g = h % Hkv"),
    ("cache offset dropped", "pos = (Lk - Lq) + np.arange(Lq)[:, None]", "pos = np.arange(Lq)[:, None]"),
    ("not causal", "ok = j <= pos", "ok = j >= 0"),
    ("scale dropped", "(Q @ K.T) * float(scale)", "(Q @ K.T)"),
    ("key start ignored", "K = k[ka:kb, g * d:(g + 1) * d]", "K = k[:kb - ka, g * d:(g + 1) * d]"),
    ("no normalisation", "(P / P.sum(axis=1, keepdims=True)) @ V", "P @ V"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_fails_a_pin(name, old, new, oracle_lib):
    assert old in SRC, f"mutation target missing: {name}"
    mod = types.ModuleType(f"mutant_{name}")
    exec(compile(SRC.replace(old, new, 1), f"<mutant {name}>", "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            pin(mod, oracle_lib)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutant '{name}' passes every pin"
