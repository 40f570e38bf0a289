"""GPU parity of mgattn_dense_strided: the merged q|k|v projection output consumed
in place (one [T, 3*H*d] buffer, leading dimension 3*H*d), and a row-strided output
whose gap columns must stay untouched.  Compared with the f64 oracle on the separate
q, k, v arrays (same seeded values), to the tolerances of the dense tests."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import oracle as orc
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


def _inputs(lens, H, d, dtype, seed):
    T = int(sum(lens))
    q, k, v = (wl.normal_f32(seed + i, (T, H * d)) for i in range(3))
    if dtype == wl.BF16:
        q, k, v = (wl.f32_to_bf16_bits(x) for x in (q, k, v))
    return q, k, v, wl.cu_from_lengths(lens)


def _run_merged(torch, q, k, v, cu, H, d, dtype, scale, causal, pad_out=0):
    """Pack q|k|v into one [T, 3*H*d] device buffer, call the strided entry point on
    its three column views; out has leading dimension H*d + pad_out."""
    T, row = q.shape[0], H * d
    qkv = to_device(np.concatenate([q, k, v], axis=1), torch)
    assert qkv.shape == (T, 3 * row) and qkv.is_contiguous()
    tdt = torch.bfloat16 if dtype == wl.BF16 else torch.float32
    ldo = row + pad_out
    sentinel = -777.0
    out = torch.full((T, ldo), sentinel, dtype=tdt, device="cuda")
    mg.mgattn_dense_strided(qkv[:, :row], qkv[:, row:2 * row], qkv[:, 2 * row:], out,
                            qkv.stride(0), qkv.stride(0), qkv.stride(0), out.stride(0),
                            cu, len(cu) - 1, H, d, scale, causal, dtype, torch.cuda.current_stream())
    torch.cuda.synchronize()
    got = from_device(out[:, :row].contiguous(), torch).reshape(T, H, d)
    gaps_ok = bool((out[:, row:] == sentinel).all()) if pad_out else True
    return got, gaps_ok


@pytest.mark.parametrize("dtype,causal", [(wl.BF16, 0), (wl.BF16, 1), (wl.F32, 0)])
def test_merged_qkv_matches_oracle(torch, dtype, causal):
    H, d, lens = 16, 96, [300, 77, 513, 1]
    q, k, v, cu = _inputs(lens, H, d, dtype, seed=601)
    say(f"merged qkv dtype={dtype} causal={causal} lens={lens}")
    got, _ = _run_merged(torch, q, k, v, cu, H, d, dtype, 1 / np.sqrt(d), causal)
    want = orc.attention(*(x.reshape(-1, H, d) for x in (q, k, v)), cu, H, d, 1 / np.sqrt(d), causal=bool(causal))
    tol = BF16_TOL if dtype == wl.BF16 else F32_TOL
    assert np.abs(got - want).max() <= tol


@pytest.mark.parametrize("dtype,pad", [(wl.BF16, 64), (wl.F32, 4)])
def test_strided_out_leaves_gaps(torch, dtype, pad):
    H, d, lens = 4, 128, [257, 100]
    q, k, v, cu = _inputs(lens, H, d, dtype, seed=611)
    say(f"strided out dtype={dtype} pad={pad}")
    got, gaps_ok = _run_merged(torch, q, k, v, cu, H, d, dtype, 0.125, 0, pad_out=pad)
    want = orc.attention(*(x.reshape(-1, H, d) for x in (q, k, v)), cu, H, d, 0.125)
    assert gaps_ok, "a gap column of the strided out was written"
    assert np.abs(got - want).max() <= (BF16_TOL if dtype == wl.BF16 else F32_TOL)


def test_merged_qkv_equals_dense_bitwise(torch):
    """Same values through the strided and the contiguous entry points: identical
    results (the kernels only change addressing)."""
    H, d = 16, 96
    case = wl.tower_layer(3)  # 4096-token full layer, the benchmark's shape
    say("merged qkv vs dense, 4096-token full layer")
    got, _ = _run_merged(torch, case.q, case.k, case.v, case.cu_seqlens, H, d, wl.BF16, case.scale, 0)
    qd, kd, vd = (to_device(x, torch) for x in (case.q, case.k, case.v))
    out = torch.empty_like(qd)
    mg.mgattn_dense(qd, kd, vd, out, case.cu_seqlens, 1, H, d, case.scale, 0, wl.BF16, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(got, from_device(out, torch).reshape(case.T, H, d))
