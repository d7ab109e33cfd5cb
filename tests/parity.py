"""Parity criteria shared by the GPU tests (numpy only, so the criteria
themselves are unit-tested on the CPU).

Channel scores (QUADS section 3.3, Eq. 23 squared): the oracle's score is the
fp64 value nearest to the exact sum of squared residuals.  The GPU sums the
same exact fp64 squares in a fixed order of its own; any fp64 summation of n
non-negative terms is within gamma_(n-1) = (n-1) u / (1 - (n-1) u), u = 2^-53,
of the exact sum, relative, and the oracle is within u of it, so the two differ
by at most (rows + 1) 2^-53 (plus a hair for the denominator) relative.

Selection (Eq. 24): a selection decided on scores that carry that relative
error eps can differ from the exact top-k only among channels whose exact
score lies within the factor (1 + eps) / (1 - eps) of the k-th largest; every
channel above that band must be selected and none below it.  Where the GPU's
set equals the oracle's top-k it is compared exactly; otherwise the rest is
checked for validity and the near-tie is reported.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle


def score_rel_bound(rows: int) -> float:
    n = max(int(rows), 1)
    return (n + 1) * 2.0 ** -53 * (1.0 + 1e-6)


def check_scores(gpu: np.ndarray, ref: np.ndarray, rows: int) -> float:
    """GPU fp64 channel scores within the summation bound of the oracle's.
    Returns the largest relative difference found."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    eps = score_rel_bound(rows)
    diff = np.abs(gpu - ref)
    bad = diff > eps * ref
    assert not bad.any(), (f"scores outside the (rows + 1) 2^-53 bound at "
                           f"{np.argwhere(bad).ravel()[:5].tolist()}: gpu "
                           f"{gpu[bad][:3].tolist()} oracle {ref[bad][:3].tolist()}")
    nz = ref > 0
    return float(np.max(diff[nz] / ref[nz])) if nz.any() else 0.0


def check_selection(S_gpu, ref: np.ndarray, k: int, rows: int, gpu_scores=None) -> np.ndarray:
    """Validate a GPU channel set against the oracle's exact scores ``ref``.

    * it is k ascending, unique channels in range;
    * if the GPU's own scores are given, it is exactly the top-k of them
      (ties to the smaller channel): the selection kernel's decision is exact;
    * it equals the oracle's top-k, or differs only inside the near-tie band.
    Returns the set (int64) for use as the oracle's S downstream."""
    S = np.asarray(S_gpu).astype(np.int64).ravel()
    ref = np.asarray(ref, dtype=np.float64)
    K = ref.shape[0]
    assert S.shape == (k,), (S.shape, k)
    if k == 0:
        return S
    assert np.all(np.diff(S) > 0), "channel set not ascending and unique"
    assert S[0] >= 0 and S[-1] < K, "channel out of range"
    if gpu_scores is not None:
        assert np.array_equal(S, oracle.select_topk(np.asarray(gpu_scores, np.float64), k)), \
            "channel set is not the top-k of the GPU's own scores"
    So = oracle.select_topk(ref, k).astype(np.int64)
    if np.array_equal(S, So):
        return S
    eps = score_rel_bound(rows)
    t = float(ref[So].min())
    hi = t * (1 + eps) / (1 - eps) * (1 + 1e-12)
    lo = t * (1 - eps) / (1 + eps) * (1 - 1e-12)
    inS = np.zeros(K, dtype=bool)
    inS[S] = True
    must = ref > hi
    never = ref < lo
    assert not (must & ~inS).any(), f"channels {np.argwhere(must & ~inS).ravel()[:5].tolist()} missing"
    assert not (never & inS).any(), f"channels {np.argwhere(never & inS).ravel()[:5].tolist()} wrongly selected"
    extra = sorted(set(S.tolist()) - set(So.tolist()))
    miss = sorted(set(So.tolist()) - set(S.tolist()))
    print(f"selection differs from the exact top-{k} inside the near-tie band "
          f"(k-th score {t!r}): gpu takes {extra}, oracle {miss}", flush=True)
    sys.stdout.flush()
    return S


# fp16 rounding of the NVFP4 compensation operands (unit roundoff 2^-11; the
# fp32 product with the reciprocal of s_W f_A before it adds 2^-23 at most)
RAC_FP16_REL = 2.0 ** -11 * (1.0 + 2.0 ** -10)


def rac_fp16_bound(R: np.ndarray, Wsel: np.ndarray, s_a: float, s_w: float) -> np.ndarray:
    """Elementwise bound, in output units, of what the NVFP4 GEMM's fp16
    compensation operands add to its error.  The selected weight columns enter
    as fp16(w / (s_W f_A)) (s_A = f_A 2^e_A, f_A in [0.5, 1)): relative error
    RAC_FP16_REL, or 2^-25 absolute in those units below fp16's normal range;
    the residual enters as bf16(r) 2^-e_A, exact down to 2^-17 and within
    2^-25 absolute below.  With R [rows][k] and Wsel [cols][k] the residual
    and weight values on the selected channels:
        RAC_FP16_REL |R| |Wsel|^T + 2^-25 (s_W |R| 1 + s_A 1 |Wsel|^T)."""
    R = np.abs(np.asarray(R, dtype=np.float64))
    W = np.abs(np.asarray(Wsel, dtype=np.float64))
    if R.shape[1] == 0:
        return np.zeros((R.shape[0], W.shape[0]))
    b = RAC_FP16_REL * (R @ W.T)
    b += 2.0 ** -25 * (s_w * R.sum(axis=1)[:, None] + s_a * W.sum(axis=1)[None, :])
    return b


def check_close(y: np.ndarray, ref: np.ndarray, tol: float, extra=None, bf16_ulp=False) -> float:
    """|y - ref| <= tol max(|ref|, rms(ref)) (+ extra, elementwise) (+ one bf16
    ulp of ref when y was rounded to bf16).  Returns the largest relative
    error against the tol term alone."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 1.0
    den = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    lim = tol * den
    if extra is not None:
        lim = lim + extra
    if bf16_ulp:
        lim = lim + np.abs(ref) * 2.0 ** -8
    bad = np.abs(y - ref) > lim
    assert not bad.any(), f"outside the bound at {np.argwhere(bad)[:5].tolist()}"
    return float(np.max(np.abs(y - ref) / den)) if ref.size else 0.0

