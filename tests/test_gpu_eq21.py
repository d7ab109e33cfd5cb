"""GPU parity of the page-literal compensation (QUADS section 3.3, Eq. 20-21:
the quantization error re-quantized to NVFP4, masked to the selected channels,
times the NVFP4 weight) against the fp64 CPU oracle: the residual's tensor
scale and its masked code x scale values bit-exact, the GEMM within the
relative tolerance."""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_from_f32, make_inputs
from tests.gpu_util import GEMM_TOL, cached, check_bf16_output, dev, gemm_rel_err, host, say
from tests.parity import check_selection

pytestmark = pytest.mark.gpu


def q4():
    import fp4_w4a4_quantized_nvfp4_amd as m
    return m


def _bits(a):
    return bf16_bits_from_f32(np.asarray(a, dtype=np.float32))


def _run(xb, wb, k, out_dtypes, rows=None, key=None):
    """GPU quantize x and W, select k channels, rac_gemm_eq21 in each output
    type; compare with one oracle computation (on `rows` of the output when
    given)."""
    m = q4()
    M, K = xb.shape
    N = wb.shape[0]
    say(f"eq21 parity x={xb.shape} w={wb.shape} k={k} out={out_dtypes}")
    x, w = dev(xb), dev(wb)
    qa = m.nvfp4_quantize(x, topk=k)
    W = m.nvfp4_quantize(w)
    kp = (k + 31) // 32 * 32
    wsb = m.lib().rac_gemm_eq21_workspace_size(M, N, K, k)
    ws = torch.zeros((max(wsb, 1),), dtype=torch.uint8, device="cuda")
    sr = torch.full((1,), -1.0, dtype=torch.float32, device="cuda")
    S = qa["chan_idx"] if k else None
    Ys = [host(m.rac_gemm_eq21(x, qa, W, S, out_dtype=o, workspace=ws, resid_tensor_scale=sr))
          for o in out_dtypes]
    torch.cuda.synchronize()
    Rp = host(ws[: M * kp * 2].view(torch.int16).view(M, kp)) if k else None
    if key:
        Ao = cached(key + "_Ao", lambda: oracle.nvfp4_quantize(xb))
        Wo = cached(key + "_Wo", lambda: oracle.nvfp4_quantize(wb))
    else:
        Ao = oracle.nvfp4_quantize(xb)
        Wo = oracle.nvfp4_quantize(wb)
    So = check_selection(host(S) if k else np.zeros(0), oracle.channel_scores(Ao.resid), k, M,
                         gpu_scores=host(qa["chan_score"]))
    Q = oracle.eq21_residual_quant(Ao)
    if k:
        # s_R and R' = (c sb) of Q(dX) on S, bit-exact
        assert np.float32(host(sr)[0]) == Q.tensor_scale, (host(sr)[0], Q.tensor_scale)
        rv = Rp.view(np.float16).astype(np.float64)          # R' is exact in fp16
        ref_r = oracle.block_values(Q.codes, Q.scales, "nvfp4")[:, So]
        assert np.array_equal(rv[:, :k], ref_r)
        assert not rv[:, k:].any()
    ref = oracle.rac_gemm_eq21(xb, Ao, Wo, So, rows=rows, Q=Q)
    for o, Y in zip(out_dtypes, Ys):
        y = Y if rows is None else Y[rows]
        if o == m.OUT_F32:
            err = gemm_rel_err(y, ref)
            say(f"  max rel err {err:.3e}")
            assert err <= GEMM_TOL
        else:
            check_bf16_output(y, ref)


def test_small_dense_workload_eq21():
    """64 x 512 x 512, 4 outlier channels, k = 16 (256 x 128 tile kernel)."""
    d = make_inputs("dense_64x512")
    _run(d["x"], d["w"], 16, (0, 1))


def test_eq21_k0_equals_w4a4():
    m = q4()
    d = make_inputs("dense_64x512")
    x, w = dev(d["x"]), dev(d["w"])
    A = m.nvfp4_quantize(x)
    W = m.nvfp4_quantize(w)
    Y0 = m.w4a4_gemm(A, W)
    Y1 = m.rac_gemm_eq21(x, A, W, None)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)


@pytest.mark.parametrize("M,N,K,k", [(300, 200, 96, 20), (1, 1, 32, 1), (257, 129, 160, 32),
                                     (513, 384, 1024, 100), (1000, 1300, 512, 64),
                                     (512, 512, 4096, 128), (777, 640, 384, 512)])
def test_eq21_ragged_shapes(M, N, K, k):
    """Ragged M and N, K a multiple of 32 but not 128, k not a multiple of 32,
    k = K; the 512-and-up shapes with K % 128 == 0 run the 256 x 256 kernel."""
    k = min(k, K)
    rng = np.random.default_rng(7 * M + N + K)
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 40.0
    xb = _bits(x)
    wb = _bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    _run(xb, wb, k, (0, 1))


def test_eq21_dense_prefill_workload_full():
    """8192 x 14336 x 4096, k = 128: s_R and R' bit-exact on every row, and
    every output element against the oracle, fp32 and bf16 output."""
    d = cached("dense_inputs", lambda: make_inputs("dense_8192x14336x4096"))
    _run(d["x"], d["w"], 128, (0, 1), key="dense")


def test_eq21_golden_mask_after_quantize():
    """The hand-worked Eq. 21 example (tests/golden/eq21_mask_after_quantize.txt):
    the selected channel 2 shares its block with a larger unselected residual,
    so its quantized correction is zero; the GPU reproduces the exact values."""
    m = q4()
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :3] = [5.25, 1.9140625, 0.87890625]
    w = np.zeros((2, 32), dtype=np.float32)
    w[0, 2] = 5.25
    w[1, :3] = 5.25
    xd, wd = dev(_bits(x)), dev(_bits(w))
    A = m.nvfp4_quantize(xd)
    W = m.nvfp4_quantize(wd)
    for S, y in (([2], [4.59375, 41.34375]), ([1, 2], [4.59375, 42.205078125])):
        Y = m.rac_gemm_eq21(xd, A, W, torch.tensor(S, dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert host(Y).tolist() == [y], (S, host(Y).tolist())


def test_eq21_zero_residual():
    """x exactly representable (E2M1 values times power-of-two block scales
    with the amax element at code 6): dX is all zero, s_R = 1, R' = 0 and the
    result equals w4a4_gemm bit for bit."""
    m = q4()
    rng = np.random.default_rng(21)
    M, N, K = 96, 160, 256
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    mag = rng.integers(0, 8, size=(M, K))
    mag[:, ::16] = 7
    xv = grid[mag] * np.where(rng.random((M, K)) < 0.5, -1, 1) * 2.0 ** rng.integers(-3, 3, size=(M, K // 16)).repeat(16, 1)
    # with a supplied s_t = 1 every block scale is its power of two and every
    # element a grid point
    xb = _bits(xv.astype(np.float32))
    wb = _bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    x, w = dev(xb), dev(wb)
    one = torch.ones((1,), dtype=torch.float32, device="cuda")
    A = m.nvfp4_quantize(x, tensor_scale_in=one)
    W = m.nvfp4_quantize(w)
    S = torch.arange(0, K, 4, dtype=torch.int32, device="cuda")
    sr = torch.zeros((1,), dtype=torch.float32, device="cuda")
    Y1 = m.rac_gemm_eq21(x, A, W, S, resid_tensor_scale=sr)
    Y0 = m.w4a4_gemm(A, W)
    torch.cuda.synchronize()
    assert float(host(sr)[0]) == 1.0
    assert torch.equal(Y0, Y1)
