"""CPU oracle for the NVFP4 W4A4 + Residual Activation Compensation path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) imports, links or runs anything in this package; only the
tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code with the HIP kernels: it depends on
numpy alone, and its inputs come from the seeded generators in ``workloads``
(which contain no quantization, selection, GEMM or MoE arithmetic).

Every function is a plain, slow, obviously-correct restatement of the method
on the QUADS page (arXiv 2607.15810, "QUADS: Stabilizing NVFP4 Reinforcement
Learning for MoE via QUantization-error Alignment across Dual Sides"):

* NVFP4 format -- section 2.2, paragraph "FP4": E2M1 codes with magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}, one E4M3 block scale per sixteen consecutive
  elements, and a per-tensor FP32 scale on top; E4M3 maximum 448 from the
  paragraph "FP8".
* Activation quantization error -- section 3.3, Eq. 20.
* Per-channel residual score -- section 3.3, Eq. 23; top-k selection Eq. 24.
* Residual compensation -- section 3.3, Eq. 21-22 (applied with the bf16
  residual on the selected channels against the bf16 weight columns).
* MXFP4 variant -- the "open-standard MXFP4" of the Rollout-ResQ abstract
  (page thelatestinai.com/papers/2607.15810) with the OCP power-of-two scale.

Every rounding decision is taken by comparing exact fp64 products (all
operands have few significant bits), never by a rounded quotient.  Channel
scores are exact sums of squares rounded once to fp64, so no summation order
enters them.
"""
from .formats import (  # noqa: F401
    E2M1_MAGNITUDES,
    E4M3_MAX,
    E4M3_VALUES,
    bf16_bits_to_f64,
    e2m1_value,
    e4m3_value,
    f32_to_bf16_bits,
    f64_to_bf16_bits,
    f64_to_f32,
)
from .quant import (  # noqa: F401
    QuantResult,
    block_values,
    channel_scores,
    dequantize,
    mxfp4_quantize,
    nvfp4_qdq,
    nvfp4_quantize,
    nvfp4_tensor_scale,
    residual_gather,
    select_topk,
)
from .gemm import rac_gemm, w4a4_gemm, rac_gemm_eq21, eq21_residual_quant  # noqa: F401
from .moe import moe_route, moe_sort, moe_layer, swiglu_bf16  # noqa: F401
