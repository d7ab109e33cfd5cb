"""Device-side input contracts: channel sets (ascending, unique, in range) and
expert indices (in [0, E)) that break them are reported in the status word and
take the documented safe path; NaN router logits still give valid experts.
Every case here is in bounds by construction (the kernels clamp before any
access), so nothing can fault."""
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


def _status():
    return torch.full((1,), -7, dtype=torch.int32, device="cuda")


BAD_SETS = {"duplicate": [3, 40, 40, 100], "unsorted": [40, 3, 100, 200],
            "negative": [-1, 3, 40, 100], "past_end": [3, 40, 100, 512]}


@pytest.mark.parametrize("case", sorted(BAD_SETS))
def test_rac_gemm_invalid_channel_set(case):
    m = q4()
    say(f"invalid channel set {case}")
    d = make_inputs("dense_64x512")
    x, w = dev(d["x"]), dev(d["w"])
    A = m.nvfp4_quantize(x)
    W = m.prepare_weight(w)
    S = torch.tensor(BAD_SETS[case], dtype=torch.int32, device="cuda")
    st = _status()
    Y = m.rac_gemm(x, A, W, W["w_hi_t"], S, status=st)
    Y0 = m.w4a4_gemm(A, W)
    st21 = _status()
    Y21 = m.rac_gemm_eq21(x, A, W, S, status=st21)
    stg = _status()
    R = m.q4_residual_gather(x, A, S, ld_r=8, status=stg)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 1 and int(host(st21)[0]) == 1 and int(host(stg)[0]) == 1
    assert torch.equal(Y, Y0), "an invalid set must add no compensation"
    # the Eq. 21 form carries its W4A4 sum at another scale (s_A / s_R), so a
    # zero compensation leaves it equal to w4a4_gemm up to fp32 rounding
    y21, y0 = host(Y21).astype(np.float64), host(Y0).astype(np.float64)
    assert np.max(np.abs(y21 - y0)) <= 1e-6 * np.max(np.abs(y0))
    assert not host(R).any()


def test_valid_set_reports_ok_and_k0():
    m = q4()
    d = make_inputs("dense_64x512")
    x, w = dev(d["x"]), dev(d["w"])
    A = m.nvfp4_quantize(x, topk=16)
    W = m.prepare_weight(w)
    for S in (A["chan_idx"], None):
        st, st21 = _status(), _status()
        m.rac_gemm(x, A, W, W["w_hi_t"], S, status=st)
        m.rac_gemm_eq21(x, A, W, S, status=st21)
        torch.cuda.synchronize()
        assert int(host(st)[0]) == 0 and int(host(st21)[0]) == 0
    # an empty product still validates its set
    xe = torch.empty((0, 512), dtype=torch.int16, device="cuda")
    Ae = m.nvfp4_quantize(xe)
    st = _status()
    m.rac_gemm(xe, Ae, W, W["w_hi_t"], torch.tensor([5, 5], dtype=torch.int32, device="cuda"),
               status=st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 1


def test_route_nan_logits():
    m = q4()
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((40, 128)).astype(np.float32)
    logits[0, :] = np.nan                       # no finite logit
    logits[1, 5:] = np.nan                      # only five finite logits, topk 8
    logits[2, 7] = np.nan
    idx, p = m.q4_moe_route(dev(logits), 8)
    idx, p = host(idx), host(p)
    assert idx.min() >= 0 and idx.max() < 128
    for t in range(40):
        assert len(set(idx[t].tolist())) == 8
    assert idx[0].tolist() == list(range(8))            # NaN ranks last, ties -> lower expert
    np.testing.assert_allclose(p[0], np.full(8, 1 / 8), rtol=1e-6)
    assert sorted(idx[1, :5].tolist()) == [0, 1, 2, 3, 4] and idx[1, 5:].tolist() == [5, 6, 7]
    assert np.all(p[1, 5:] == 0)
    clean = logits.copy()
    clean[2, 7] = -np.inf
    oi, _ = oracle.moe_route(clean[2:], 8)
    assert np.array_equal(idx[2:], oi)


def test_sort_and_layer_with_invalid_expert_index():
    m = q4()
    rng = np.random.default_rng(4)
    T, H, E, F, topk, k = 64, 256, 8, 128, 2, 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, p = m.q4_moe_route(dev(logits), topk)
    bad = idx.clone()
    bad[3, 1] = -1
    bad[10, 0] = E
    st = _status()
    perm, off = m.q4_moe_sort(bad, E, status=st)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 1
    fixed = host(bad).copy()
    fixed[(fixed < 0) | (fixed >= E)] = 0                # sorted as expert 0
    pe, oe = oracle.moe_sort(fixed, E)
    assert np.array_equal(host(perm), pe) and np.array_equal(host(off), oe)
    # the layer: an invalid slot is computed as expert 0 and weighted zero, so
    # the result equals the layer with index 0 and weight 0 in those slots
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, 7] *= 30
    xd = dev(bf16_bits_from_f32(x))
    w13 = dev(bf16_bits_from_f32((rng.standard_normal((E, 2 * F, H)) * 0.05).astype(np.float32)))
    w2 = dev(bf16_bits_from_f32((rng.standard_normal((E, H, F)) * 0.05).astype(np.float32)))
    experts = m.prepare_moe_weights(w13, w2)
    st = _status()
    Y1, _ = m.moe_w4a4_grouped_gemm(xd, bad, p, experts, k, status=st)
    idx0 = torch.from_numpy(fixed).cuda()
    p0 = p.clone()
    p0[3, 1] = 0.0
    p0[10, 0] = 0.0
    st0 = _status()
    Y0, _ = m.moe_w4a4_grouped_gemm(xd, idx0, p0, experts, k, status=st0)
    torch.cuda.synchronize()
    assert int(host(st)[0]) == 1 and int(host(st0)[0]) == 0
    assert torch.equal(Y1, Y0)
