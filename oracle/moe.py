"""Top-k MoE expert layer with W4A4 + residual compensation (test oracle).

TEST INFRASTRUCTURE ONLY -- never used by the product path.

The QUADS page (arXiv 2607.15810) applies the compensation at MoE projections
(section 3.3 "Online per-channel selection": the profiled W13 activation site;
Figure 4b: layer-wise MoE output).  It does not spell out the MoE block, so the
plain reading used here is the standard SwiGLU expert layer:

* routing: the top-k experts of each token by router logit (ties -> smaller
  expert index), weights p = softmax over the k selected logits;
* W13 projection (gate rows 0..F-1, up rows F..2F-1 of the logical [2F x H]
  weight) of the token's NVFP4 activation, with residual compensation on the
  channels selected over all tokens;
* h = bf16(silu(gate) * up), silu(g) = g / (1 + exp(-g));
* h of all routed rows, ordered by (expert, token, slot), is quantized as one
  activation tensor (one tensor scale, one channel selection);
* W2 projection with residual compensation, and y_t = sum over slots
  (slot 0 first) of p * out.
* With a bf16 layer output (``out_bf16``) the expert rows enter that sum as
  bf16 values (out rounded once, to nearest even), the form in which an
  expert-parallel layer hands them back for combining; with an fp32 output
  they enter unrounded.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64, f64_to_bf16_bits
from .gemm import rac_gemm
from .quant import (QuantResult, channel_scores, mxfp4_quantize, nvfp4_quantize, residual_gather,
                    select_topk)


def moe_route(logits: np.ndarray, topk: int):
    """idx int32 [T, topk] (highest logit first, ties -> lower expert), p fp64."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, topk), dtype=np.int32)
    p = np.empty((T, topk), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:topk]
        idx[t] = order
        sel = logits[t, order].astype(np.float64)
        w = np.exp(sel - sel.max())
        p[t] = w / w.sum()
    return idx, p


def moe_sort(idx: np.ndarray, E: int):
    """perm [T*topk] of flat (t*topk + s) sorted by (expert, t, s); offsets [E+1]."""
    T, k = idx.shape
    flat = [(int(idx[t, s]), t, s) for t in range(T) for s in range(k)]
    flat.sort()
    perm = np.array([t * k + s for (_, t, s) in flat], dtype=np.int32)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return perm, offsets


def swiglu_bf16(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """h = RN_bf16(silu(gate) * up), silu(g) = g / (1 + exp(-g)), computed in
    fp64 and rounded once (the SwiGLU expert block; the page does not spell
    the block out, this is its standard form)."""
    g = np.asarray(gate, dtype=np.float64)
    u = np.asarray(up, dtype=np.float64)
    with np.errstate(over="ignore"):          # exp(-g) = inf gives silu = -0
        return f64_to_bf16_bits(g / (1.0 + np.exp(-g)) * u)


def _rows(q: QuantResult, rows: np.ndarray) -> QuantResult:
    return QuantResult(q.fmt, q.codes[rows], q.scales[rows], q.tensor_scale, q.resid[rows],
                       q.mag[rows], q.sign[rows])


def moe_layer(x_bits, idx, p, w13_bits, w2_bits, rac_k: int, h_override=None,
              wq13=None, wq2=None, fmt: str = "nvfp4", Sx_override=None, Sh_override=None,
              h_tensor_scale=None, out_bf16: bool = False):
    """Whole expert layer; returns a dict of every intermediate (fp64 unless noted).

    x_bits [T, H] bf16 bits; idx/p from ``moe_route``; w13_bits [E, 2F, H] and
    w2_bits [E, H, F] bf16 bits (logical layout).  ``h_override`` replaces the
    oracle's own h (bf16 bits [T*topk, F], sorted order) before the second
    quantization, for stage-wise comparison.  ``wq13``/``wq2`` are optional
    pre-quantized expert weights (lists of QuantResult).  ``fmt`` selects the
    activation and weight format ("nvfp4" or "mxfp4").  ``Sx_override`` /
    ``Sh_override`` replace the selected channel sets of the two sites (a set
    already validated against this oracle's scores, where several sets are
    correct at a near-tie).  ``h_tensor_scale`` (NVFP4) quantizes h under that
    supplied tensor scale instead of RN32(amax(h) / 2688) (delayed scaling).
    ``out_bf16`` rounds each W2 row to bf16 before the combine ("out" stays
    the exact product, "out_used" is what the combine sums).
    """
    quant = nvfp4_quantize if fmt == "nvfp4" else mxfp4_quantize
    T, H = x_bits.shape
    E, F2, _ = w13_bits.shape
    F = F2 // 2
    k = idx.shape[1]
    perm, offsets = moe_sort(idx, E)
    tok = perm // k
    qx = quant(x_bits)
    sx = channel_scores(qx.resid)
    Sx = select_topk(sx, rac_k) if Sx_override is None else np.asarray(Sx_override)
    Rx = residual_gather(qx.resid, Sx)
    if wq13 is None:
        wq13 = [quant(w13_bits[e]) for e in range(E)]
    if wq2 is None:
        wq2 = [quant(w2_bits[e]) for e in range(E)]
    y13 = np.zeros((T * k, F2), dtype=np.float64)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        rows = tok[r0:r1]
        y13[r0:r1] = rac_gemm(_rows(qx, rows), wq13[e], Rx[rows], w13_bits[e], Sx)
    h = swiglu_bf16(y13[:, :F], y13[:, F:])
    h_used = h if h_override is None else np.asarray(h_override, dtype=np.uint16)
    if h_tensor_scale is not None and fmt == "nvfp4":
        qh = quant(h_used, tensor_scale=float(h_tensor_scale))
    else:
        qh = quant(h_used)
    sh = channel_scores(qh.resid)
    Sh = select_topk(sh, rac_k) if Sh_override is None else np.asarray(Sh_override)
    Rh = residual_gather(qh.resid, Sh)
    out = np.zeros((T * k, H), dtype=np.float64)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 == r0:
            continue
        rows = np.arange(r0, r1)
        out[r0:r1] = rac_gemm(_rows(qh, rows), wq2[e], Rh[rows], w2_bits[e], Sh)
    out_used = bf16_bits_to_f64(f64_to_bf16_bits(out)) if out_bf16 else out
    pos = np.empty(T * k, dtype=np.int64)
    pos[perm] = np.arange(T * k)
    y = np.zeros((T, H), dtype=np.float64)
    for s in range(k):
        y += p[:, s:s + 1] * out_used[pos[np.arange(T) * k + s]]
    return dict(perm=perm, offsets=offsets, qx=qx, scores_x=sx, Sx=Sx, Rx=Rx, y13=y13, h=h,
                qh=qh, scores_h=sh, Sh=Sh, Rh=Rh, out=out, out_used=out_used, y=y, wq13=wq13,
                wq2=wq2)


def dense_swiglu_reference(x_bits, w13_bits, w2_bits):
    """Unquantized fp64 SwiGLU MLP (E = 1, top-1 reduction target)."""
    x = bf16_bits_to_f64(x_bits)
    w13 = bf16_bits_to_f64(w13_bits)
    F = w13.shape[0] // 2
    y13 = x @ w13.T
    g, u = y13[:, :F], y13[:, F:]
    h = g / (1.0 + np.exp(-g)) * u
    return h @ bf16_bits_to_f64(w2_bits).T
