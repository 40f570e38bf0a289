"""Thin ctypes binding of the mgattn C ABI (include/mgattn.h), same names as the C side.

Argument marshalling only: every step of the attention runs in the HIP kernels of
``_lib/libmgattn.so``.  There is no fallback: if the library is missing or the call
is refused, these functions raise.  Tensors are torch tensors (device memory and
streams come from PyTorch); a raw integer device address is accepted as well.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path
from typing import Sequence

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "_lib" / "libmgattn.so"

MGATTN_F32 = 0
MGATTN_BF16 = 1

STATUS_NAMES = {
    0: "MGATTN_OK", -1: "MGATTN_ERR_NULL", -2: "MGATTN_ERR_DTYPE", -3: "MGATTN_ERR_HEAD_DIM",
    -4: "MGATTN_ERR_HEADS", -5: "MGATTN_ERR_SEQLENS", -6: "MGATTN_ERR_SEGMENTS",
    -7: "MGATTN_ERR_ALIAS", -8: "MGATTN_ERR_ALIGN", -9: "MGATTN_ERR_SCALE",
    -10: "MGATTN_ERR_LAUNCH", -11: "MGATTN_ERR_DEVICE", -12: "MGATTN_ERR_SIZE", -13: "MGATTN_ERR_STRIDE",
    -14: "MGATTN_ERR_GRID", -15: "MGATTN_ERR_WINDOW", -16: "MGATTN_ERR_SCRATCH",
}

EXPORTS = ["mgattn_dense", "mgattn_dense_strided", "mgattn_attention_kv", "mgattn_attention_kv_ws",
           "mgattn_attention_kv_noalloc", "mgattn_attention_kv_noalloc_scratch_bytes",
           "mgattn_attention_kv_workspace", "mgattn_strerror", "mgattn_dense_supported", "mgattn_dense_lds_bytes",
           "mgattn_dense_block_m", "mgattn_dense_plan_block_m", "mgattn_dense_plan", "mgattn_dense_tile", "mgattn_window_segments",
           "mgattn_window_permute", "mgattn_rope2d", "mgattn_dense_rope2d", "mgattn_version"]


class MgattnError(RuntimeError):
    def __init__(self, status: int, what: str = "mgattn_dense"):
        self.status = status
        super().__init__(f"{what} failed: {STATUS_NAMES.get(status, status)}: {mgattn_strerror(status)}")


_lib = None


def load_library(path: str | os.PathLike | None = None):
    """Load libmgattn.so (built by ``python -m vit_perception_encoder_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    # MGATTN_LIB names another build of the same library (e.g. host code under sanitizers)
    p = Path(path) if path is not None else Path(os.environ.get("MGATTN_LIB", LIB_PATH))
    if not p.exists():
        raise ImportError(f"mgattn HIP library not built: {p} is missing "
                          "(run `python -m vit_perception_encoder_amd.build`)")
    lib = ctypes.CDLL(str(p))
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    lib.mgattn_dense.restype = i32
    lib.mgattn_dense.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, f32, i32, i32, vp]
    lib.mgattn_dense_strided.restype = i32
    lib.mgattn_dense_strided.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, i32, i32, f32, i32, i32, vp]
    lib.mgattn_attention_kv.restype = i32
    lib.mgattn_attention_kv.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, i32, i32, i32, i32, f32, i32,
                                        i32, vp]
    lib.mgattn_attention_kv_ws.restype = i32
    lib.mgattn_attention_kv_ws.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, i32, i32, i32, i32, f32, i32,
                                           i32, vp, ctypes.c_size_t, vp]
    lib.mgattn_attention_kv_noalloc.restype = i32
    lib.mgattn_attention_kv_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, vp, i32, i32, i32, i32, f32,
                                                i32, i32, vp]
    lib.mgattn_attention_kv_noalloc_scratch_bytes.restype = ctypes.c_long
    lib.mgattn_attention_kv_noalloc_scratch_bytes.argtypes = []
    lib.mgattn_attention_kv_workspace.restype = ctypes.c_long
    lib.mgattn_attention_kv_workspace.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32]
    lib.mgattn_strerror.restype = ctypes.c_char_p
    lib.mgattn_strerror.argtypes = [i32]
    lib.mgattn_dense_supported.restype = i32
    lib.mgattn_dense_supported.argtypes = [i32, i32, i32]
    lib.mgattn_dense_lds_bytes.restype = ctypes.c_long
    lib.mgattn_dense_lds_bytes.argtypes = [i32, i32]
    lib.mgattn_dense_block_m.restype = i32
    lib.mgattn_dense_block_m.argtypes = [i32, i32]
    lib.mgattn_dense_plan_block_m.restype = i32
    lib.mgattn_dense_plan_block_m.argtypes = [vp, i32, i32, i32, i32, i32]
    lib.mgattn_dense_plan.restype = i32
    lib.mgattn_dense_plan.argtypes = [vp, i32, i32, i32, i32, i32, vp, i32]
    lib.mgattn_dense_tile.restype = i32
    lib.mgattn_dense_tile.argtypes = [vp, i32, i32, i32, i32, i32, i32, i64, vp]
    lib.mgattn_window_segments.restype = i32
    lib.mgattn_window_segments.argtypes = [vp, i32, i32, vp, i32]
    lib.mgattn_window_permute.restype = i32
    lib.mgattn_window_permute.argtypes = [vp, vp, i64, vp, i32, i32, i32, vp]
    lib.mgattn_rope2d.restype = i32
    lib.mgattn_rope2d.argtypes = [vp, i64, vp, i32, i32, i32, i32, f32, i32, vp]
    lib.mgattn_dense_rope2d.restype = i32
    lib.mgattn_dense_rope2d.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, vp, i32, i32, i32, f32, i32, i32, vp, i32,
                                        i32, f32, vp]
    lib.mgattn_version.restype = i32
    lib.mgattn_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        return 0
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


_ELEM_BYTES = {MGATTN_F32: 4, MGATTN_BF16: 2}


def _check_tensor(name: str, t, elem_bytes: int | None, need_bytes: int) -> None:
    """Refuse, before the C call, a torch tensor the kernels would read or write out
    of bounds: it must live on a GPU, have the element size of the call's dtype (None:
    any), and own at least ``need_bytes`` bytes of storage from its data pointer on.
    Raw integer addresses (and None) are passed through unchecked: the C side only
    sees pointers."""
    if t is None or isinstance(t, int):
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: expected a GPU tensor, got one on {getattr(t, 'device', type(t))}")
    if elem_bytes is not None and t.element_size() != elem_bytes:
        raise ValueError(f"{name}: element size {t.element_size()} B does not match the call's dtype "
                         f"({elem_bytes} B)")
    have = t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()
    if need_bytes > have:
        raise ValueError(f"{name}: the call spans {need_bytes} bytes from the data pointer, the tensor's storage "
                         f"holds {have}")


def _span(rows: int, ld: int, width: int, elem: int) -> int:
    """Bytes from the first element of row 0 to the end of row rows-1 (rows of
    `width` elements, `ld` elements apart)."""
    return 0 if rows <= 0 else ((rows - 1) * ld + width) * elem


def _cu_array(cu_seqlens):
    seq = [int(x) for x in cu_seqlens]
    return (ctypes.c_int32 * len(seq))(*seq), len(seq)


def mgattn_dense(q, k, v, out, cu_seqlens: Sequence[int], n_seg: int, H: int, d: int, scale: float,
                 causal: int, dtype: int, stream=None, check: bool = True) -> int:
    """Enqueue segmented attention (see mgattn_dense in include/mgattn.h).

    ``cu_seqlens`` is a host sequence of n_seg+1 ints.  Returns the status; with
    ``check`` (the default) a negative status raises MgattnError instead."""
    lib = load_library()
    cu, ncu = _cu_array(cu_seqlens)
    if ncu < n_seg + 1:
        raise ValueError(f"cu_seqlens has {ncu} entries, n_seg={n_seg} needs {n_seg + 1}")
    eb = _ELEM_BYTES.get(int(dtype))
    if eb is not None and n_seg >= 0:
        T = int(cu[n_seg])
        for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
            _check_tensor(name, t, eb, _span(T, H * d, H * d, eb))
    st = lib.mgattn_dense(_ptr(q), _ptr(k), _ptr(v), _ptr(out), ctypes.cast(cu, ctypes.c_void_p), int(n_seg),
                          int(H), int(d), float(scale), int(causal), int(dtype), _stream(stream))
    if check and st != 0:
        raise MgattnError(st)
    return st


def mgattn_dense_strided(q, k, v, out, ldq: int, ldk: int, ldv: int, ldo: int, cu_seqlens: Sequence[int],
                         n_seg: int, H: int, d: int, scale: float, causal: int, dtype: int, stream=None,
                         check: bool = True) -> int:
    """mgattn_dense on row-strided tensors (see mgattn_dense_strided in include/mgattn.h);
    ld* are leading dimensions in elements.  For torch views, pass e.g. ``t.stride(0)``."""
    lib = load_library()
    cu, ncu = _cu_array(cu_seqlens)
    if ncu < n_seg + 1:
        raise ValueError(f"cu_seqlens has {ncu} entries, n_seg={n_seg} needs {n_seg + 1}")
    eb = _ELEM_BYTES.get(int(dtype))
    if eb is not None and n_seg >= 0:
        T = int(cu[n_seg])
        for name, t, ld in (("q", q, ldq), ("k", k, ldk), ("v", v, ldv), ("out", out, ldo)):
            _check_tensor(name, t, eb, _span(T, int(ld), H * d, eb))
    st = lib.mgattn_dense_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), int(ldq), int(ldk), int(ldv), int(ldo),
                                  ctypes.cast(cu, ctypes.c_void_p), int(n_seg), int(H), int(d), float(scale),
                                  int(causal), int(dtype), _stream(stream))
    if check and st != 0:
        raise MgattnError(st, "mgattn_dense_strided")
    return st


def _check_kv(q, k, v, out, ldq, ldk, ldv, ldo, cq, ck, n_seq, Hq, Hkv, d, dtype) -> None:
    eb = _ELEM_BYTES.get(int(dtype))
    if eb is None or n_seq < 0:
        return
    Tq, Tk = int(cq[n_seq]), int(ck[n_seq])
    for name, t, rows, ld, width in (("q", q, Tq, ldq, Hq * d), ("k", k, Tk, ldk, Hkv * d),
                                     ("v", v, Tk, ldv, Hkv * d), ("out", out, Tq, ldo, Hq * d)):
        _check_tensor(name, t, eb, _span(rows, int(ld), width, eb))


def mgattn_attention_kv(q, k, v, out, ldq: int, ldk: int, ldv: int, ldo: int, cu_seqlens_q: Sequence[int],
                        cu_seqlens_k: Sequence[int], n_seq: int, Hq: int, Hkv: int, d: int, scale: float,
                        window: int, dtype: int, stream=None, check: bool = True) -> int:
    """Causal sliding-window GQA attention over a key/value cache (see
    mgattn_attention_kv in include/mgattn.h)."""
    lib = load_library()
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_k)
    if nq < n_seq + 1 or nk < n_seq + 1:
        raise ValueError(f"cu_seqlens_q/k need {n_seq + 1} entries")
    _check_kv(q, k, v, out, ldq, ldk, ldv, ldo, cq, ck, n_seq, Hq, Hkv, d, dtype)
    st = lib.mgattn_attention_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(out), int(ldq), int(ldk), int(ldv), int(ldo),
                                 ctypes.cast(cq, ctypes.c_void_p), ctypes.cast(ck, ctypes.c_void_p), int(n_seq),
                                 int(Hq), int(Hkv), int(d), float(scale), int(window), int(dtype), _stream(stream))
    if check and st != 0:
        raise MgattnError(st, "mgattn_attention_kv")
    return st


def mgattn_attention_kv_ws(q, k, v, out, ldq: int, ldk: int, ldv: int, ldo: int, cu_seqlens_q: Sequence[int],
                           cu_seqlens_k: Sequence[int], n_seq: int, Hq: int, Hkv: int, d: int, scale: float,
                           window: int, dtype: int, workspace, workspace_bytes: int, stream=None,
                           check: bool = True) -> int:
    """mgattn_attention_kv with a caller-provided device workspace, used to split
    one-token decoding over more workgroups (see mgattn_attention_kv_ws in
    include/mgattn.h)."""
    lib = load_library()
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_k)
    if nq < n_seq + 1 or nk < n_seq + 1:
        raise ValueError(f"cu_seqlens_q/k need {n_seq + 1} entries")
    _check_kv(q, k, v, out, ldq, ldk, ldv, ldo, cq, ck, n_seq, Hq, Hkv, d, dtype)
    _check_tensor("workspace", workspace, None, int(workspace_bytes))
    st = lib.mgattn_attention_kv_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(out), int(ldq), int(ldk), int(ldv), int(ldo),
                                    ctypes.cast(cq, ctypes.c_void_p), ctypes.cast(ck, ctypes.c_void_p), int(n_seq),
                                    int(Hq), int(Hkv), int(d), float(scale), int(window), int(dtype), _ptr(workspace),
                                    int(workspace_bytes), _stream(stream))
    if check and st != 0:
        raise MgattnError(st, "mgattn_attention_kv_ws")
    return st


def mgattn_attention_kv_noalloc(q, k, v, out, ldq: int, ldk: int, ldv: int, ldo: int, cu_seqlens_q: Sequence[int],
                                cu_seqlens_k: Sequence[int], n_seq: int, Hq: int, Hkv: int, d: int, scale: float,
                                window: int, dtype: int, stream=None, check: bool = True) -> int:
    """mgattn_attention_kv_ws without a workspace argument: the key-split partial
    results go to the library's per-device scratch (see mgattn_attention_kv_noalloc
    in include/mgattn.h); nothing is allocated."""
    lib = load_library()
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_k)
    if nq < n_seq + 1 or nk < n_seq + 1:
        raise ValueError(f"cu_seqlens_q/k need {n_seq + 1} entries")
    _check_kv(q, k, v, out, ldq, ldk, ldv, ldo, cq, ck, n_seq, Hq, Hkv, d, dtype)
    st = lib.mgattn_attention_kv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), int(ldq), int(ldk), int(ldv),
                                         int(ldo), ctypes.cast(cq, ctypes.c_void_p), ctypes.cast(ck, ctypes.c_void_p),
                                         int(n_seq), int(Hq), int(Hkv), int(d), float(scale), int(window), int(dtype),
                                         _stream(stream))
    if check and st != 0:
        raise MgattnError(st, "mgattn_attention_kv_noalloc")
    return st


def mgattn_attention_kv_noalloc_scratch_bytes() -> int:
    return int(load_library().mgattn_attention_kv_noalloc_scratch_bytes())


def mgattn_attention_kv_workspace(cu_seqlens_q: Sequence[int], cu_seqlens_k: Sequence[int], n_seq: int, Hq: int,
                                  Hkv: int, d: int, window: int, dtype: int) -> int:
    """Workspace bytes mgattn_attention_kv_ws would use (0: no split), or a negative
    status.  Host arithmetic only."""
    lib = load_library()
    cq, nq = _cu_array(cu_seqlens_q)
    ck, nk = _cu_array(cu_seqlens_k)
    if nq < n_seq + 1 or nk < n_seq + 1:
        raise ValueError(f"cu_seqlens_q/k need {n_seq + 1} entries")
    return int(lib.mgattn_attention_kv_workspace(ctypes.cast(cq, ctypes.c_void_p), ctypes.cast(ck, ctypes.c_void_p),
                                                 int(n_seq), int(Hq), int(Hkv), int(d), int(window), int(dtype)))


def mgattn_strerror(status: int) -> str:
    return load_library().mgattn_strerror(int(status)).decode()


def mgattn_dense_supported(H: int, d: int, dtype: int) -> int:
    return load_library().mgattn_dense_supported(int(H), int(d), int(dtype))


def mgattn_dense_lds_bytes(d: int, dtype: int) -> int:
    return load_library().mgattn_dense_lds_bytes(int(d), int(dtype))


def mgattn_dense_block_m(d: int, dtype: int) -> int:
    return load_library().mgattn_dense_block_m(int(d), int(dtype))


def mgattn_dense_plan_block_m(cu_seqlens, n_seg: int, H: int, d: int, dtype: int, causal: int = 0) -> int:
    """Queries per workgroup mgattn_dense uses for this segment table (raises on refusal)."""
    lib = load_library()
    cu, _ = _cu_array(cu_seqlens)
    r = lib.mgattn_dense_plan_block_m(ctypes.cast(cu, ctypes.c_void_p), int(n_seg), int(H), int(d), int(dtype),
                                      int(causal))
    if r < 0:
        raise MgattnError(r, "mgattn_dense_plan_block_m")
    return int(r)


def mgattn_dense_plan(cu_seqlens, n_seg: int, H: int, d: int, dtype: int, causal: int = 0) -> list[int]:
    """Workgroup count of each launch mgattn_dense would make (raises on refusal)."""
    lib = load_library()
    cu, _ = _cu_array(cu_seqlens)
    n = lib.mgattn_dense_plan(ctypes.cast(cu, ctypes.c_void_p), int(n_seg), int(H), int(d), int(dtype),
                              int(causal), None, 0)
    if n < 0:
        raise MgattnError(n, "mgattn_dense_plan")
    grids = (ctypes.c_int64 * max(n, 1))()
    lib.mgattn_dense_plan(ctypes.cast(cu, ctypes.c_void_p), int(n_seg), int(H), int(d), int(dtype),
                          int(causal), ctypes.cast(grids, ctypes.c_void_p), n)
    return [int(g) for g in grids[:n]]


def mgattn_dense_tile(cu_seqlens, n_seg: int, H: int, d: int, dtype: int, causal: int, launch: int, block: int):
    """(segment, head, q0) computed by one workgroup, or None for an idle one."""
    lib = load_library()
    cu, _ = _cu_array(cu_seqlens)
    out = (ctypes.c_int32 * 3)()
    r = lib.mgattn_dense_tile(ctypes.cast(cu, ctypes.c_void_p), int(n_seg), int(H), int(d), int(dtype),
                              int(causal), int(launch), int(block), ctypes.cast(out, ctypes.c_void_p))
    if r < 0:
        raise MgattnError(r, "mgattn_dense_tile")
    return (int(out[0]), int(out[1]), int(out[2])) if r == 1 else None


def _grid_array(grids):
    """[(gh, gw), ...] -> int32[2*n] (host)."""
    flat = [int(v) for g in grids for v in g]
    return (ctypes.c_int32 * max(len(flat), 1))(*flat), len(flat) // 2


def mgattn_window_segments(grids, win: int) -> list[int]:
    """cu_seqlens of the window layers for patch grids [(gh, gw), ...] (raises on refusal)."""
    lib = load_library()
    g, n_img = _grid_array(grids)
    gp = ctypes.cast(g, ctypes.c_void_p)
    n = lib.mgattn_window_segments(gp, n_img, int(win), None, 0)
    if n < 0:
        raise MgattnError(n, "mgattn_window_segments")
    cu = (ctypes.c_int32 * (n + 1))()
    r = lib.mgattn_window_segments(gp, n_img, int(win), ctypes.cast(cu, ctypes.c_void_p), n)
    if r < 0:
        raise MgattnError(r, "mgattn_window_segments")
    return [int(x) for x in cu]


def mgattn_window_permute(src, dst, row_bytes: int, grids, win: int, inverse: int, stream=None,
                          check: bool = True) -> int:
    """Gather rows into window order (inverse=0) or scatter them back (inverse=1)."""
    lib = load_library()
    g, n_img = _grid_array(grids)
    T = sum(int(gh) * int(gw) for gh, gw in grids)
    for name, t in (("src", src), ("dst", dst)):
        _check_tensor(name, t, None, T * int(row_bytes))
    st = lib.mgattn_window_permute(_ptr(src), _ptr(dst), int(row_bytes), ctypes.cast(g, ctypes.c_void_p), n_img,
                                   int(win), int(inverse), _stream(stream))
    if check and st != 0:
        raise MgattnError(st, "mgattn_window_permute")
    return st


def mgattn_rope2d(x, ldx: int, grids, win: int, H: int, d: int, theta: float, dtype: int, stream=None,
                  check: bool = True) -> int:
    """In-place 2D rotary embedding of x (token rows of leading dimension ldx)."""
    lib = load_library()
    g, n_img = _grid_array(grids)
    eb = _ELEM_BYTES.get(int(dtype))
    if eb is not None:
        T = sum(int(gh) * int(gw) for gh, gw in grids)
        _check_tensor("x", x, eb, _span(T, int(ldx), H * d, eb))
    st = lib.mgattn_rope2d(_ptr(x), int(ldx), ctypes.cast(g, ctypes.c_void_p), n_img, int(win), int(H), int(d),
                           float(theta), int(dtype), _stream(stream))
    if check and st != 0:
        raise MgattnError(st, "mgattn_rope2d")
    return st


def mgattn_dense_rope2d(q, k, v, out, ldq: int, ldk: int, ldv: int, ldo: int, cu_seqlens: Sequence[int], n_seg: int,
                        H: int, d: int, scale: float, causal: int, dtype: int, grids, win: int, theta: float,
                        stream=None, check: bool = True) -> int:
    """Attention over 2D-RoPE-rotated q and k, q rotated on load, k rotated in place
    (see mgattn_dense_rope2d in include/mgattn.h)."""
    lib = load_library()
    cu, ncu = _cu_array(cu_seqlens)
    if ncu < n_seg + 1:
        raise ValueError(f"cu_seqlens has {ncu} entries, n_seg={n_seg} needs {n_seg + 1}")
    eb = _ELEM_BYTES.get(int(dtype))
    if eb is not None and n_seg >= 0:
        T = int(cu[n_seg])
        for name, t, ld in (("q", q, ldq), ("k", k, ldk), ("v", v, ldv), ("out", out, ldo)):
            _check_tensor(name, t, eb, _span(T, int(ld), H * d, eb))
    g, n_img = _grid_array(grids)
    st = lib.mgattn_dense_rope2d(_ptr(q), _ptr(k), _ptr(v), _ptr(out), int(ldq), int(ldk), int(ldv), int(ldo),
                                 ctypes.cast(cu, ctypes.c_void_p), int(n_seg), int(H), int(d), float(scale), int(causal),
                                 int(dtype), ctypes.cast(g, ctypes.c_void_p), n_img, int(win), float(theta),
                                 _stream(stream))
    if check and st != 0:
        raise MgattnError(st, "mgattn_dense_rope2d")
    return st


def mgattn_version() -> int:
    return load_library().mgattn_version()
