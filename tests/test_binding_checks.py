"""The Python binding refuses tensors the kernels would read or write out of bounds
(host only: the checks run before any C call, so no GPU is needed).

A tensor handed to the binding must be on a GPU, have the element size of the call's
dtype, and own storage covering the rows the call spans; raw integer addresses pass
through unchecked (the C side only sees pointers)."""
import pytest
import torch

from vit_perception_encoder_amd import mgattn as mg

pytestmark = pytest.mark.cpu


class FakeGpuTensor:
    """Stands in for a device tensor: the attributes the binding's checks read."""

    def __init__(self, n_elems, elem_bytes=2, offset=0):
        self.n, self.eb, self.off = n_elems, elem_bytes, offset

    is_cuda = True

    def element_size(self):
        return self.eb

    def storage_offset(self):
        return self.off

    def untyped_storage(self):
        n, eb = self.n, self.eb

        class S:
            def nbytes(self):
                return n * eb

        return S()

    def data_ptr(self):  # never reached: every case below is refused first
        raise AssertionError("the binding reached the C call")


T, H, D = 64, 16, 96
FULL = T * H * D


def test_cpu_tensor_is_refused():
    x = torch.zeros(FULL, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        mg.mgattn_dense(x, x, x, x, [0, T], 1, H, D, 0.1, 0, mg.MGATTN_BF16)


def test_dtype_size_mismatch_is_refused():
    ok = FakeGpuTensor(FULL, 2)
    f32 = FakeGpuTensor(FULL, 4)
    with pytest.raises(ValueError, match="element size"):
        mg.mgattn_dense(ok, ok, f32, FakeGpuTensor(FULL, 2), [0, T], 1, H, D, 0.1, 0, mg.MGATTN_BF16)
    with pytest.raises(ValueError, match="element size"):
        mg.mgattn_dense(ok, ok, ok, FakeGpuTensor(FULL, 2), [0, T], 1, H, D, 0.1, 0, mg.MGATTN_F32)


@pytest.mark.parametrize("which", ["q", "k", "v", "out"])
def test_short_tensor_is_refused(which):
    args = {n: FakeGpuTensor(FULL) for n in ("q", "k", "v", "out")}
    args[which] = FakeGpuTensor(FULL - 1)
    with pytest.raises(ValueError, match=which):
        mg.mgattn_dense(args["q"], args["k"], args["v"], args["out"], [0, T], 1, H, D, 0.1, 0, mg.MGATTN_BF16)


def test_storage_offset_counts():
    # a view whose data pointer starts 8 elements into a buffer of exactly FULL elements
    x = FakeGpuTensor(FULL, offset=8)
    with pytest.raises(ValueError, match="q"):
        mg.mgattn_dense(x, FakeGpuTensor(FULL), FakeGpuTensor(FULL), FakeGpuTensor(FULL), [0, T], 1, H, D, 0.1, 0,
                        mg.MGATTN_BF16)


def test_strided_span_uses_leading_dimension():
    ld = 3 * H * D
    # a merged qkv buffer of T rows: q at column 0 spans (T-1)*ld + H*D elements
    need = (T - 1) * ld + H * D
    with pytest.raises(ValueError, match="k"):
        mg.mgattn_dense_strided(FakeGpuTensor(need), FakeGpuTensor(need - 1), FakeGpuTensor(need),
                                FakeGpuTensor(FULL), ld, ld, ld, H * D, [0, T], 1, H, D, 0.1, 0, mg.MGATTN_BF16)


def test_attention_kv_spans():
    Hq, Hkv, d = 32, 2, 128
    cq, ck = [0, 1, 2], [0, 100, 300]
    q = FakeGpuTensor(2 * Hq * d)
    o = FakeGpuTensor(2 * Hq * d)
    k = FakeGpuTensor(300 * Hkv * d)
    v_short = FakeGpuTensor(299 * Hkv * d)
    with pytest.raises(ValueError, match="v"):
        mg.mgattn_attention_kv(q, k, v_short, o, Hq * d, Hkv * d, Hkv * d, Hq * d, cq, ck, 2, Hq, Hkv, d, 0.1, 0,
                               mg.MGATTN_BF16)
    with pytest.raises(ValueError, match="workspace"):
        mg.mgattn_attention_kv_ws(q, k, FakeGpuTensor(300 * Hkv * d), o, Hq * d, Hkv * d, Hkv * d, Hq * d, cq, ck, 2,
                                  Hq, Hkv, d, 0.1, 0, mg.MGATTN_BF16, FakeGpuTensor(100, 1), 4096)


def test_window_permute_and_rope_spans():
    grids = [(8, 8), (4, 6)]
    Tg = 64 + 24
    row = H * D * 2
    with pytest.raises(ValueError, match="dst"):
        mg.mgattn_window_permute(FakeGpuTensor(Tg * row, 1), FakeGpuTensor(Tg * row - 1, 1), row, grids, 32, 0)
    with pytest.raises(ValueError, match="x"):
        mg.mgattn_rope2d(FakeGpuTensor(Tg * H * D - 1), H * D, grids, 32, H, D, 10000.0, mg.MGATTN_BF16)
