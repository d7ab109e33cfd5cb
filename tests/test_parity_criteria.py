"""CPU checks of the score and selection criteria used by the GPU tests: the
bound accepts any fp64 summation order and rejects a selection that is wrong
outside the near-tie band."""
import numpy as np
import pytest

import oracle
from tests.parity import check_scores, check_selection, score_rel_bound


def _resid(rows=700, cols=96, seed=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_t(3, size=(rows, cols)) * 0.1).astype(np.float32)


def test_any_summation_order_within_bound():
    r = _resid()
    ref = oracle.channel_scores(r)
    sq = r.astype(np.float64) ** 2
    fwd = np.zeros(r.shape[1])
    for i in range(r.shape[0]):
        fwd += sq[i]
    rev = np.zeros(r.shape[1])
    for i in range(r.shape[0] - 1, -1, -1):
        rev += sq[i]
    pair = sq.copy()
    while pair.shape[0] > 1:
        if pair.shape[0] % 2:
            pair = np.vstack([pair, np.zeros((1, pair.shape[1]))])
        pair = pair[0::2] + pair[1::2]
    for s in (fwd, rev, pair[0]):
        check_scores(s, ref, r.shape[0])
        check_selection(oracle.select_topk(s, 10), ref, 10, r.shape[0], gpu_scores=s)


def test_score_outside_bound_rejected():
    r = _resid()
    ref = oracle.channel_scores(r)
    bad = ref.copy()
    bad[7] *= 1 + 4 * score_rel_bound(r.shape[0])
    with pytest.raises(AssertionError):
        check_scores(bad, ref, r.shape[0])


def test_selection_near_tie_accepted_clear_error_rejected():
    ref = np.array([5.0, 3.0, 3.0 * (1 + 2.0 ** -50), 1.0, 0.5, 3.0 * (1 - 2.0 ** -51)])
    # exact top-2 is {0, 2}; {0, 1} and {0, 5} differ only inside the band
    assert check_selection([0, 2], ref, 2, rows=4096).tolist() == [0, 2]
    check_selection([0, 1], ref, 2, rows=4096)
    check_selection([0, 5], ref, 2, rows=4096)
    with pytest.raises(AssertionError):
        check_selection([0, 3], ref, 2, rows=4096)         # 1.0 is far below the band
    with pytest.raises(AssertionError):
        check_selection([1, 2], ref, 2, rows=4096)         # drops the clear winner
    with pytest.raises(AssertionError):
        check_selection([2, 0], ref, 2, rows=4096)         # not ascending
    with pytest.raises(AssertionError):
        check_selection([0, 0], ref, 2, rows=4096)         # duplicate
    with pytest.raises(AssertionError):                    # not the top-k of its own scores
        check_selection([0, 1], ref, 2, rows=4096, gpu_scores=ref)


def test_rac_fp16_bound_covers_fp16_operands():
    """The compensation bound holds for the product formed the GPU's way (the
    weight divided by s_W f_A and rounded to fp16, the residual times 2^-e_A,
    then scaled back by s_A s_W), including saturated-block magnitudes and
    fp16-subnormal weights, and a coarser (bf16) rounding of the weight
    breaks it."""
    from tests.parity import RAC_FP16_REL, rac_fp16_bound
    rng = np.random.default_rng(3)
    R = (rng.standard_normal((64, 32)) * 50.0).astype(np.float32)
    R = R.astype(np.float64)
    W = rng.standard_normal((48, 32)) * 0.02
    W[:, :4] *= 1e-6                                      # fp16 subnormals in the sum's units
    W = W.astype(np.float32).astype(np.float64)
    s_a, s_w = 0.0371, 0.00123
    f_a, e_a = np.frexp(s_a)
    exact = R @ W.T
    Rg = R * 2.0 ** -e_a                                  # exact scaling by a power of two
    rinv = np.float32(1.0) / np.float32(np.float32(s_w) * np.float32(f_a))
    Wg = (W.astype(np.float32) * rinv).astype(np.float32).astype(np.float16).astype(np.float64)
    got = (Rg @ Wg.T) * (s_a * s_w)
    b = rac_fp16_bound(R, W, s_a, s_w)
    assert (np.abs(got - exact) <= b * (1 + 1e-9) + 1e-300).all()
    # a bf16 weight (unit roundoff 2^-9) exceeds it somewhere
    import torch
    Wb = torch.from_numpy(W / (s_w * f_a)).to(torch.bfloat16).to(torch.float64).numpy()
    worse = (Rg @ Wb.T) * (s_a * s_w)
    assert (np.abs(worse - exact) > b).any()
    assert RAC_FP16_REL > 2.0 ** -11
