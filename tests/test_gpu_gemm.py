"""GPU parity of the W4A4 GEMM and the residual-compensated GEMM against the
fp64 CPU oracle on the same quantized operands."""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_from_f32, make_inputs
from tests.gpu_util import GEMM_TOL, cached, check_bf16_output, dev, gemm_rel_err, host, say
from tests.parity import check_scores, check_selection

pytestmark = pytest.mark.gpu


def q4():
    import fp4_w4a4_quantized_nvfp4_amd as m
    return m


def _bits(a):
    return bf16_bits_from_f32(np.asarray(a, dtype=np.float32))


PAGE_GRID = [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _exact_operand(rng, rows, cols, scales=(0.5, 1.0, 2.0)):
    sb = rng.choice(scales, size=(rows, cols // 16))
    mag = rng.integers(0, 8, size=(rows, cols))
    mag[:, ::16] = 7
    sign = rng.random((rows, cols)) < 0.5
    val = np.array(PAGE_GRID)[mag] * np.repeat(sb, 16, axis=1) * np.where(sign, -1, 1)
    return _bits(val.astype(np.float32))


def _quant_pair(m, xb, wb, fmt="nv", ts=None):
    x, w = dev(xb), dev(wb)
    if fmt == "mx":
        return x, m.mxfp4_quantize(x), m.mxfp4_quantize(w), oracle.mxfp4_quantize(xb), oracle.mxfp4_quantize(wb)
    tin = None if ts is None else torch.tensor([ts], dtype=torch.float32, device="cuda")
    A = m.nvfp4_quantize(x, tensor_scale_in=tin)
    W = m.nvfp4_quantize(w, tensor_scale_in=tin)
    return x, A, W, oracle.nvfp4_quantize(xb, tensor_scale=ts), oracle.nvfp4_quantize(wb, tensor_scale=ts)


# E4M3 subnormal block scales m * 2^-9, m = 1..7
SUBNORMAL_SCALES = tuple(m * 2.0 ** -9 for m in range(1, 8))


@pytest.mark.parametrize("M,N,K,scales", [(300, 200, 512, (0.5, 1.0, 2.0)),
                                          (512, 768, 512, (0.5, 1.0, 2.0)),
                                          (512, 768, 512, SUBNORMAL_SCALES),
                                          (300, 200, 512, SUBNORMAL_SCALES)],
                         ids=["small", "large_tile", "large_tile_subnormal", "small_subnormal"])
def test_exact_special_case_bit_identical(M, N, K, scales):
    """E2M1 values times exact E4M3 scales with a supplied tensor scale of 1:
    every product and partial sum is exact in fp32, so any correct GEMM gives
    the oracle's result bit for bit (the subnormal case checks that E4M3
    subnormal block scales are widened exactly)."""
    say(f"gemm exact special case {M}x{N}x{K}")
    m = q4()
    rng = np.random.default_rng(11 + M + len(scales))
    xb = _exact_operand(rng, M, K, scales)
    wb = _exact_operand(rng, N, K, scales)
    x, A, W, Ao, Wo = _quant_pair(m, xb, wb, ts=1.0)
    assert np.array_equal(host(A["scales"]), Ao.scales)
    if scales is SUBNORMAL_SCALES:
        assert Ao.scales.max() < 8          # exponent field 0: subnormal E4M3
    Y = host(m.w4a4_gemm(A, W))
    ref = oracle.w4a4_gemm(Ao, Wo)
    assert np.array_equal(Y.astype(np.float64), ref)


def _gpu_selection(m, x, Ao, k, fmt="nv"):
    """GPU channel selection on x, validated against the oracle's exact scores;
    returns (device S, host S) -- the host copy is the oracle's S downstream."""
    if not k:
        return None, np.zeros(0, dtype=np.int64)
    qs = m.mxfp4_quantize(x, topk=k) if fmt == "mx" else m.nvfp4_quantize(x, topk=k)
    ref = oracle.channel_scores(Ao.resid)
    gsc = host(qs["chan_score"])
    check_scores(gsc, ref, Ao.resid.shape[0])
    So = check_selection(host(qs["chan_idx"]), ref, k, Ao.resid.shape[0], gpu_scores=gsc)
    return qs["chan_idx"], So


def _check_rac(xb, wb, k, out_dtype, fmt="nv"):
    say(f"rac parity x={xb.shape} w={wb.shape} k={k} out={out_dtype} fmt={fmt}")
    m = q4()
    x, A, W, Ao, Wo = _quant_pair(m, xb, wb, fmt)
    w_hi_t = m.q4_transpose_bf16(dev(wb))
    S, So = _gpu_selection(m, x, Ao, k, fmt)
    Y = m.rac_gemm(x, A, W, w_hi_t, S, out_dtype=out_dtype)
    Ro = oracle.residual_gather(Ao.resid, So)
    ref = oracle.rac_gemm(Ao, Wo, Ro, wb, So)
    if out_dtype == m.OUT_F32:
        err = gemm_rel_err(host(Y), ref)
        say(f"  max rel err {err:.3e}")
        assert err <= GEMM_TOL
    else:
        check_bf16_output(host(Y), ref)
    return Y


def test_small_dense_workload_rac():
    d = make_inputs("dense_64x512")
    _check_rac(d["x"], d["w"], 16, 0)


def test_k0_equals_w4a4():
    m = q4()
    d = make_inputs("dense_64x512")
    x, A, W, _, _ = _quant_pair(m, d["x"], d["w"])
    Y0 = m.w4a4_gemm(A, W)
    Y1 = m.rac_gemm(x, A, W, None, None)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)


@pytest.mark.parametrize("M,N,K,k", [(300, 200, 96, 20), (1, 1, 32, 1), (257, 129, 160, 32),
                                     (513, 384, 1024, 100), (600, 520, 160, 24),
                                     (1000, 1300, 512, 64), (512, 512, 4096, 128),
                                     (512, 768, 1024, 80), (520, 512, 512, 17),
                                     (640, 520, 1024, 200)])
def test_ragged_shapes(M, N, K, k):
    rng = np.random.default_rng(M + N + K)
    xb = _bits(rng.standard_t(3, size=(M, K)).astype(np.float32))
    wb = _bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    _check_rac(xb, wb, k, 0)
    _check_rac(xb, wb, k, 1)


@pytest.mark.parametrize("M,N,K,xs,ws", [(300, 200, 512, 1e-30, 1e-5), (600, 520, 512, 1e-30, 1e-5),
                                         (300, 200, 512, 1e30, 1e3), (600, 520, 512, 1e30, 1e3),
                                         (520, 512, 1024, 1e-25, 1e-12)],
                         ids=["tiny_small", "tiny_large", "huge_small", "huge_large", "tinier_large"])
def test_extreme_tensor_scales(M, N, K, xs, ws):
    """Tensor scales whose product s_A s_W is subnormal in fp32 (or large):
    the outputs are normal numbers and must stay within the tolerance (the
    product is applied as mantissa and exponent, so it cannot underflow)."""
    rng = np.random.default_rng(int(M + K))
    x = rng.standard_t(3, size=(M, K)) * xs
    x[:, rng.choice(K, 4, replace=False)] *= 30
    xb = _bits(x.astype(np.float32))
    wb = _bits((rng.standard_normal((N, K)) * 0.05 * ws).astype(np.float32))
    Ao = oracle.nvfp4_quantize(xb)
    Wo = oracle.nvfp4_quantize(wb)
    alpha = float(np.float32(Ao.tensor_scale)) * float(np.float32(Wo.tensor_scale))
    say(f"extreme scales: s_A {float(Ao.tensor_scale):.3g} s_W {float(Wo.tensor_scale):.3g} "
        f"s_A s_W {alpha:.3g}")
    _check_rac(xb, wb, 16, 0)
    _check_rac(xb, wb, 0, 0)


def test_dense_prefill_workload_full():
    """8192 x 14336 x 4096, k = 128: x quantization bit-exact, scores within the
    summation bound and the selection validated, W codes and scales bit-exact
    on every row, and EVERY output element of rac_gemm against the fp64
    oracle, in bf16 (the workload's output type) and in fp32."""
    m = q4()
    d = cached("dense_inputs", lambda: make_inputs("dense_8192x14336x4096"))
    xb, wb = d["x"], d["w"]
    say("prefill workload: GPU quantize + rac_gemm (bf16 and fp32 output)")
    x, w = dev(xb), dev(wb)
    A = m.nvfp4_quantize(x, topk=128)
    W = m.prepare_weight(w)
    Yb = host(m.rac_gemm(x, A, W, W["w_hi_t"], A["chan_idx"], out_dtype=m.OUT_BF16))
    Yf = host(m.rac_gemm(x, A, W, W["w_hi_t"], A["chan_idx"], out_dtype=m.OUT_F32))
    torch.cuda.synchronize()
    say("prefill workload: oracle quantization of x and W")
    Ao = cached("dense_Ao", lambda: oracle.nvfp4_quantize(xb))
    assert np.array_equal(host(A["codes"]), Ao.codes)
    assert np.array_equal(host(A["scales"]), Ao.scales)
    ref_sc = oracle.channel_scores(Ao.resid)
    gsc = host(A["chan_score"])
    check_scores(gsc, ref_sc, 8192)
    So = check_selection(host(A["chan_idx"]), ref_sc, 128, 8192, gpu_scores=gsc)
    Wo = cached("dense_Wo", lambda: oracle.nvfp4_quantize(wb))
    assert np.float32(Wo.tensor_scale) == host(W["tensor_scale"])[0]
    assert np.array_equal(host(W["codes"]), Wo.codes)
    assert np.array_equal(host(W["scales"]), Wo.scales)
    del W
    say("prefill workload: oracle fp64 GEMM (every row)")
    ref = oracle.rac_gemm(Ao, Wo, oracle.residual_gather(Ao.resid, So), wb, So)
    err = gemm_rel_err(Yf, ref)
    say(f"  fp32 output max rel err {err:.3e}")
    assert err <= GEMM_TOL
    check_bf16_output(Yb, ref)
    say("prefill workload full parity ok")


@pytest.mark.parametrize("k", [128, 256, 512, 768])
def test_selection_ratio_sweep_parity(k):
    """The selection-ratio sweep's projection, 8192 x 4096 x 1024, at k = 12.5,
    25, 50 and 75 % of the channels (4 to 24 compensation chunks per tile):
    rac_gemm and rac_gemm_eq21 against the oracle on every output element."""
    m = q4()
    d = make_inputs("sweep_8192x4096x1024")
    xb, wb = d["x"], d["w"]
    say(f"sweep parity k={k}")
    x, w = dev(xb), dev(wb)
    A = m.nvfp4_quantize(x, topk=k)
    W = m.prepare_weight(w)
    Y = host(m.rac_gemm(x, A, W, W["w_hi_t"], A["chan_idx"], out_dtype=m.OUT_F32))
    Y21 = host(m.rac_gemm_eq21(x, A, W, A["chan_idx"], out_dtype=m.OUT_F32))
    torch.cuda.synchronize()
    Ao = oracle.nvfp4_quantize(xb)
    Wo = oracle.nvfp4_quantize(wb)
    assert np.array_equal(host(A["codes"]), Ao.codes)
    assert np.array_equal(host(W["codes"]), Wo.codes)
    ref_sc = oracle.channel_scores(Ao.resid)
    So = check_selection(host(A["chan_idx"]), ref_sc, k, xb.shape[0],
                         gpu_scores=host(A["chan_score"]))
    ref = oracle.rac_gemm(Ao, Wo, oracle.residual_gather(Ao.resid, So), wb, So)
    err = gemm_rel_err(Y, ref)
    say(f"  rac_gemm max rel err {err:.3e}")
    assert err <= GEMM_TOL
    ref21 = oracle.rac_gemm_eq21(xb, Ao, Wo, So)
    err21 = gemm_rel_err(Y21, ref21)
    say(f"  rac_gemm_eq21 max rel err {err21:.3e}")
    assert err21 <= GEMM_TOL


@pytest.mark.parametrize("M,N,K,k", [(64, 512, 512, 16), (300, 200, 96, 20), (513, 640, 1024, 64),
                                     (1000, 1300, 512, 64), (512, 520, 640, 32),
                                     (700, 512, 384, 100)])
def test_mxfp4_rac_gemm(M, N, K, k):
    """MXFP4 operands on the scaled FP4 matrix instruction, RAC on bf16."""
    rng = np.random.default_rng(M * 7 + K)
    x = rng.standard_t(3, size=(M, K)).astype(np.float32)
    x[:, rng.choice(K, 3, replace=False)] *= 50
    xb = _bits(x)
    wb = _bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    _check_rac(xb, wb, k, 0, fmt="mx")
    _check_rac(xb, wb, k, 1, fmt="mx")


@pytest.mark.parametrize("M,N,K", [(96, 160, 256), (512, 768, 512), (600, 520, 1024),
                                   (512, 512, 384), (520, 600, 640)],
                         ids=["small_tile", "large_tile", "large_tile_ragged", "large_tile_3_chunks",
                              "large_tile_5_chunks"])
def test_mxfp4_exact_special_case(M, N, K):
    """Power-of-two scales and E2M1 values: every partial sum is exact, so the
    scaled-MFMA product must equal the integer result bit for bit (both the
    256 x 128 and the 256 x 256 kernels)."""
    m = q4()
    say(f"mxfp4 exact special case {M}x{N}x{K}")
    rng = np.random.default_rng(17 + M)
    def operand(rows):
        e = rng.integers(-2, 3, size=(rows, K // 32))
        mag = rng.integers(0, 8, size=(rows, K))
        mag[:, ::32] = 7
        val = np.array(PAGE_GRID)[mag] * np.repeat(2.0 ** e, 32, axis=1) * 0.25
        val *= np.where(rng.random((rows, K)) < 0.5, -1, 1)
        return _bits(val.astype(np.float32))
    xb, wb = operand(M), operand(N)
    x, A, W, Ao, Wo = _quant_pair(m, xb, wb, "mx")
    Y = host(m.w4a4_gemm(A, W))
    assert np.array_equal(Y.astype(np.float64), oracle.w4a4_gemm(Ao, Wo))


@pytest.mark.parametrize("M,N,K,sub", [(512, 768, 512, False), (512, 768, 512, True),
                                       (1000, 1300, 1024, False), (777, 640, 384, True)])
def test_tiled_scale_records_match_in_place_scales(M, N, K, sub):
    """rac_gemm with k = 0 (workspace given: the large-tile kernel reads the
    re-laid-out fp16 scale records) equals w4a4_gemm (no workspace: it reads
    the E4M3 scales in place) bit for bit, subnormal E4M3 scales included."""
    m = q4()
    rng = np.random.default_rng(M + N + K)
    if sub:
        xb = _exact_operand(rng, M, K, SUBNORMAL_SCALES)
        wb = _exact_operand(rng, N, K, SUBNORMAL_SCALES)
        ts = 1.0
    else:
        xb = _bits(rng.standard_t(3, size=(M, K)).astype(np.float32))
        wb = _bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
        ts = None
    x, A, W, _, _ = _quant_pair(m, xb, wb, ts=ts)
    for out in (m.OUT_F32, m.OUT_BF16):
        Y0 = m.w4a4_gemm(A, W, out_dtype=out)
        Y1 = m.rac_gemm(x, A, W, None, None, out_dtype=out)
        torch.cuda.synchronize()
        assert torch.equal(Y0, Y1), (M, N, K, sub, out)
