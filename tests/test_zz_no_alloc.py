"""mgattn_attention_kv_noalloc (the entry point for callers that cannot allocate)
against mgattn_attention_kv_ws with a workspace of the size
mgattn_attention_kv_workspace gives: the same kernels and split, so the outputs agree
bit for bit.  Two calls in a row on one GPU, the second smaller (the scratch keeps the
first call's contents), and a host-only check that no call can need more scratch than
the library holds."""
import numpy as np
import pytest

from tests.gpu_helpers import say
from vit_perception_encoder_amd import mgattn as mg


def _decode_case(torch, B, Lk, Hq, Hkv, d, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    q = torch.randn(B, Hq * d, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(B * Lk, Hkv * d, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(B * Lk, Hkv * d, generator=g, device="cuda").to(torch.bfloat16)
    return q, k, v, list(range(B + 1)), [i * Lk for i in range(B + 1)]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice():
    import torch

    assert torch.cuda.is_available()
    mg.load_library()
    for B, Lk, Hq, Hkv, d, W, seed in ((32, 4096, 32, 2, 128, 2048, 1), (5, 700, 8, 2, 96, 0, 2)):
        say(f"noalloc decode B={B} Lk={Lk} Hq={Hq} Hkv={Hkv} d={d} window={W}")
        q, k, v, cq, ck = _decode_case(torch, B, Lk, Hq, Hkv, d, seed)
        need = mg.mgattn_attention_kv_workspace(cq, ck, B, Hq, Hkv, d, W, mg.MGATTN_BF16)
        assert 0 < need <= mg.mgattn_attention_kv_noalloc_scratch_bytes()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        want = torch.empty_like(q)
        got = torch.full_like(q, float("nan"))
        args = (Hq * d, Hkv * d, Hkv * d, Hq * d, cq, ck, B, Hq, Hkv, d, d ** -0.5, W, mg.MGATTN_BF16)
        mg.mgattn_attention_kv_ws(q, k, v, want, *args, ws, need, torch.cuda.current_stream())
        mg.mgattn_attention_kv_noalloc(q, k, v, got, *args, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), "noalloc differs from the workspace call"


def test_no_call_needs_more_scratch_than_held():
    mg.load_library()
    cap = mg.mgattn_attention_kv_noalloc_scratch_bytes()
    rng = np.random.Generator(np.random.PCG64(3))
    worst = 0
    for _ in range(300):
        B = int(rng.integers(1, 300))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8, 16, 32]))
        d = int(rng.choice([64, 96, 128]))
        lk = rng.integers(1, 20000, size=B)
        ck = np.concatenate([[0], np.cumsum(lk)]).tolist()
        need = mg.mgattn_attention_kv_workspace(list(range(B + 1)), ck, B, Hq, Hkv, d, int(rng.integers(0, 4096)),
                                                mg.MGATTN_BF16)
        assert 0 <= need <= cap
        worst = max(worst, need)
    assert worst > cap // 2  # the search reached large splits
