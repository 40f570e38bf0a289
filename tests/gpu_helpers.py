"""Shared helpers of the GPU tests: move seeded inputs to the device, run the HIP path
through the C ABI, bring results back widened to f64."""
from __future__ import annotations

import sys

import numpy as np

from vit_perception_encoder_amd import mgattn as mg
from vit_perception_encoder_amd import workloads as wl

BF16_TOL = 2e-2   # max |GPU - oracle| for bf16 inputs, f32 accumulation
F32_TOL = 1e-4    # max |GPU - oracle| for f32 inputs


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failure names it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, torch):
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def from_device(t, torch) -> np.ndarray:
    """Device tensor -> f64 numpy (exact widening)."""
    if t.dtype == torch.bfloat16:
        return wl.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def run(torch, q, k, v, cu, H, d, scale, causal, dtype, guard_rows: int = 0):
    """Run mgattn_dense on host arrays; returns (out f64 [T,H,d], guard bands intact?)."""
    T = int(cu[-1])
    qd, kd, vd = (to_device(x, torch) for x in (q, k, v))
    tdt = torch.bfloat16 if dtype == wl.BF16 else torch.float32
    row = H * d
    sentinel = -12345.0
    buf = torch.full(((T + 2 * guard_rows) * row,), sentinel, dtype=tdt, device="cuda")
    out = buf[guard_rows * row:(guard_rows + T) * row]
    mg.mgattn_dense(qd, kd, vd, out, cu, len(cu) - 1, H, d, scale, causal, dtype,
                    torch.cuda.current_stream())
    torch.cuda.synchronize()
    ok = True
    if guard_rows:
        ok = bool((buf[:guard_rows * row] == sentinel).all()) and bool((buf[(guard_rows + T) * row:] == sentinel).all())
    return from_device(out, torch).reshape(T, H, d), ok


def case_arrays(case: wl.Case):
    return case.q, case.k, case.v, case.cu_seqlens
