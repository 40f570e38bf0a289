"""ctypes wrapper around the f64 CPU oracle (``mgattn_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code with the
HIP library and never imports the ``vit_perception_encoder_amd`` package.

The oracle is the plain definition of segmented softmax attention (vllm.cpp issue
#1545, sections "Why this one is bad" and "The fix": non-causal attention over
block-diagonal per-segment row slices, H=16, head_dim=96), evaluated in f64 from the
exact widening of the stored input bits.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SRC = HERE / "mgattn_oracle.c"
LIB = HERE / "liboracle.so"

F32, BF16, F64 = 0, 1, 2

_lib = None


def build(force: bool = False) -> Path:
    """Compile the oracle with gcc (plain -O2: no fast-math, sums stay in order)."""
    if force or not LIB.exists() or LIB.stat().st_mtime < SRC.stat().st_mtime:
        tmp = LIB.with_suffix(".so.tmp")
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", str(tmp), str(SRC), "-lm"],
            check=True,
        )
        os.replace(tmp, LIB)
    return LIB


def load(path: str | os.PathLike | None = None):
    """Load the oracle library (building it first if needed) and set ctypes signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    override = os.environ.get("MGATTN_ORACLE_LIB")  # e.g. a sanitizer build, for the host checks
    lib = ctypes.CDLL(str(path if path is not None else (override or build())))
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.mgattn_oracle_f64.restype = i32
    lib.mgattn_oracle_f64.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, i32, i32, i32]
    lib.mgattn_oracle_rows_f64.restype = i32
    lib.mgattn_oracle_rows_f64.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, i32, i32, i64, vp, vp, i32]
    lib.mgattn_oracle_weights_f64.restype = i64
    lib.mgattn_oracle_weights_f64.argtypes = [vp, vp, vp, vp, i32, i32, i32, f32, i32, i32, i64, i32, vp, vp]
    if path is None:
        _lib = lib
    return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.float32:
        return F32
    if x.dtype == np.uint16:
        return BF16
    if x.dtype == np.float64:
        return F64
    raise TypeError(f"oracle inputs must be float32, uint16 (bf16 bits) or float64, got {x.dtype}")


def _prep(q, k, v, cu_seqlens, H, d):
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T = int(cu[-1])
    for a in (q, k, v):
        if a.size != T * H * d:
            raise ValueError(f"expected {T}*{H}*{d} elements, got {a.size}")
    return q, k, v, cu, T


def attention(q, k, v, cu_seqlens, H: int, d: int, scale: float, causal: bool = False,
              n_threads: int | None = None, lib=None) -> np.ndarray:
    """Full output, f64, shape [T, H, d]."""
    q, k, v, cu, T = _prep(q, k, v, cu_seqlens, H, d)
    out = np.empty((T, H, d), dtype=np.float64)
    lib = lib or load()
    rc = lib.mgattn_oracle_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, out.ctypes.data,
                               cu.ctypes.data, len(cu) - 1, H, d, float(scale), int(bool(causal)),
                               _dtype_code(q), n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def attention_rows(q, k, v, cu_seqlens, H: int, d: int, scale: float, tokens, heads,
                   causal: bool = False, n_threads: int | None = None, lib=None) -> np.ndarray:
    """Selected rows O[tokens[r], heads[r], :], f64, shape [len(tokens), d]."""
    q, k, v, cu, T = _prep(q, k, v, cu_seqlens, H, d)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    hd = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
    if tok.shape != hd.shape or tok.ndim != 1:
        raise ValueError("tokens and heads must be 1-D and the same length")
    out = np.empty((len(tok), d), dtype=np.float64)
    lib = lib or load()
    rc = lib.mgattn_oracle_rows_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, out.ctypes.data,
                                    cu.ctypes.data, len(cu) - 1, H, d, float(scale), int(bool(causal)),
                                    _dtype_code(q), len(tok), tok.ctypes.data, hd.ctypes.data,
                                    n_threads or default_threads())
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out


def weights(q, k, v, cu_seqlens, H: int, d: int, scale: float, token: int, head: int,
            causal: bool = False, lib=None):
    """Softmax weights (over the keys the row sees, from the segment start) and the
    output row, both f64."""
    q, k, v, cu, T = _prep(q, k, v, cu_seqlens, H, d)
    w = np.empty(max(T, 1), dtype=np.float64)
    o = np.empty(d, dtype=np.float64)
    lib = lib or load()
    n = lib.mgattn_oracle_weights_f64(q.ctypes.data, k.ctypes.data, v.ctypes.data, cu.ctypes.data,
                                      len(cu) - 1, H, d, float(scale), int(bool(causal)),
                                      _dtype_code(q), int(token), int(head), w.ctypes.data,
                                      o.ctypes.data)
    if n < 0:
        raise ValueError("oracle rejected its arguments")
    return w[:n].copy(), o
