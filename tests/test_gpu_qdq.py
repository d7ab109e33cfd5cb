"""GPU parity of the trainer-side weight fake quantization (QUADS section 3.2,
Eq. 12) against the oracle: the values c sb s_t bit-exact in fp32 and in bf16
(each one rounding of the exact value), in-call and supplied tensor scale."""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_from_f32, make_inputs
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def q4():
    import fp4_w4a4_quantized_nvfp4_amd as m
    return m


def _check(wb, ts=None):
    m = q4()
    say(f"qdq parity w={wb.shape} ts={ts}")
    w = dev(wb)
    tin = None if ts is None else torch.tensor([ts], dtype=torch.float32, device="cuda")
    y32, s32 = m.nvfp4_qdq(w, tensor_scale_in=tin, out_dtype=m.OUT_F32, want_scale=True)
    y16 = m.nvfp4_qdq(w, tensor_scale_in=tin, out_dtype=m.OUT_BF16)
    torch.cuda.synchronize()
    ref = oracle.nvfp4_qdq(wb, tensor_scale=ts)
    q = oracle.nvfp4_quantize(wb, tensor_scale=ts)
    assert np.float32(host(s32)[0]) == q.tensor_scale
    assert np.array_equal(host(y32).view(np.uint32), ref.astype(np.float32).view(np.uint32))
    assert np.array_equal(host(y16), oracle.f64_to_bf16_bits(ref))
    # the same codes the rollout quantizer produces
    A = m.nvfp4_quantize(w, tensor_scale_in=tin)
    assert np.array_equal(host(A["codes"]), q.codes)


def test_qdq_small_dense_weight():
    d = make_inputs("dense_64x512")
    _check(d["w"])
    _check(d["w"], ts=2.0 ** -14)


@pytest.mark.parametrize("rows,cols", [(1, 16), (300, 96), (257, 4096), (0, 64)])
def test_qdq_ragged(rows, cols):
    rng = np.random.default_rng(rows + cols)
    w = rng.standard_t(3, size=(rows, cols)).astype(np.float32) * 0.05
    if rows:
        w[:, rng.choice(cols, max(1, cols // 64), replace=False)] *= 30.0
    wb = bf16_bits_from_f32(w)
    if rows == 0:
        m = q4()
        y, s = m.nvfp4_qdq(dev(wb), want_scale=True)
        torch.cuda.synchronize()
        assert y.shape == (0, cols) and float(host(s)[0]) == 1.0
        return
    _check(wb)


def test_qdq_prefill_weight_rows():
    """The first 2048 rows of the 14336 x 4096 prefill weight."""
    d = make_inputs("dense_8192x14336x4096", rows=8)
    _check(np.ascontiguousarray(d["w"][:2048]))
