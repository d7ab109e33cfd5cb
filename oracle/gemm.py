"""W4A4 GEMM and residual-compensated GEMM in fp64 (test oracle).

TEST INFRASTRUCTURE ONLY -- never used by the product path.

QUADS page (arXiv 2607.15810) section 3.3:
* Eq. 22's remark: the main product stays a native W4A4 GEMM on the NVFP4
  operands; with Y = A W^T, A [M x K] activations, W [N x K] weights:
      Y_w4a4[i, j] = s_A s_W sum_k (c sb)_A[i, k] (c sb)_W[j, k].
* Eq. 21, read as the residual correction that the compensation adds on the
  selected channel set S: the residual r = x - dequant(x) on S, rounded to
  bf16, multiplied by the bf16 weight columns W[:, S]:
      Y_rac = Y_w4a4 + sum_{t<k} R[i, t] W_hi[j, S_t].
* ``rac_gemm_eq21`` is the page-literal form: the residual tensor is itself
  quantized with the activation quantizer Q_A (its own tensor scale and blocks),
  masked to S after quantization, and the corrected activation
  X~ = Q_A(X) - M_S * Q_A(dX_q) multiplies the NVFP4 weight.

All sums use numpy's float64 matrix product (a library routine); the
operands are exact in fp64, so the only rounding is fp64 accumulation.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64
from .quant import QuantResult, block_values, nvfp4_quantize


def w4a4_gemm(A: QuantResult, W: QuantResult) -> np.ndarray:
    """fp64 Y [M, N] = s_A s_W (A_d @ W_d^T) for NVFP4 or MXFP4 operands."""
    if A.fmt != W.fmt:
        raise ValueError("A and W must share a format")
    ad = block_values(A.codes, A.scales, A.fmt)
    wd = block_values(W.codes, W.scales, W.fmt)
    y = ad @ wd.T
    return y * (float(A.tensor_scale) * float(W.tensor_scale))


def rac_gemm(A: QuantResult, W: QuantResult, R_bits: np.ndarray, w_hi_bits: np.ndarray,
             S: np.ndarray) -> np.ndarray:
    """fp64 Y_w4a4 + R @ W_hi[:, S]^T; R bf16 bits [M, k], w_hi bf16 bits [N, K]."""
    y = w4a4_gemm(A, W)
    S = np.asarray(S, dtype=np.int64)
    if S.size:
        r = bf16_bits_to_f64(R_bits)
        wh = bf16_bits_to_f64(w_hi_bits)[:, S]
        y = y + r @ wh.T
    return y


def eq21_residual_quant(A: QuantResult) -> QuantResult:
    """Q_A(dX_q), dX_q = Q_A(X) - X = -resid (fp32, rounded once), carried as
    bf16 like any activation entering Q_A: its own tensor scale and blocks."""
    from .formats import f32_to_bf16_bits
    return nvfp4_quantize(f32_to_bf16_bits(-A.resid))


def rac_gemm_eq21(x_bits: np.ndarray, A: QuantResult, W: QuantResult, S: np.ndarray,
                  rows=None, Q: QuantResult | None = None) -> np.ndarray:
    """Page-literal Eq. 21: X~ = Q_A(X) - M_S * Q_A(Q_A(X) - X), times the NVFP4 W.

    ``rows`` (optional index array) restricts the output to those rows; ``Q``
    may pass a precomputed ``eq21_residual_quant(A)``."""
    if Q is None:
        Q = eq21_residual_quant(A)
    sel = slice(None) if rows is None else np.asarray(rows, dtype=np.int64)
    qd = block_values(Q.codes[sel], Q.scales[sel], "nvfp4") * float(Q.tensor_scale)
    mask = np.zeros(A.resid.shape[1], dtype=bool)
    mask[np.asarray(S, dtype=np.int64)] = True
    xt = block_values(A.codes[sel], A.scales[sel], "nvfp4") * float(A.tensor_scale) - qd * mask[None, :]
    wd = block_values(W.codes, W.scales, "nvfp4") * float(W.tensor_scale)
    return xt @ wd.T
