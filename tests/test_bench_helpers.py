"""CPU checks of the bench's measurement helpers (no GPU): the torch decode of an
NVFP4 weight that the selection-ratio sweep uses as its reference weight equals
the oracle's dequantized values up to one fp32 rounding."""
import numpy as np
import torch

import oracle
from workloads import bf16_bits_from_f32


def test_nvfp4_weight_values_match_oracle():
    import bench
    rng = np.random.default_rng(4)
    w = rng.standard_t(3, size=(48, 512)).astype(np.float32) * 0.05
    w[:, 7] *= 40.0
    wb = bf16_bits_from_f32(w)
    q = oracle.nvfp4_quantize(wb)
    W = {"codes": torch.from_numpy(q.codes), "scales": torch.from_numpy(q.scales),
         "tensor_scale": torch.tensor([float(q.tensor_scale)], dtype=torch.float32)}
    got = bench._nvfp4_weight_values(W).double().numpy()
    ref = oracle.dequantize(q)
    assert np.array_equal(got.astype(np.float32), ref.astype(np.float32))
