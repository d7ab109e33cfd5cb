"""GPU parity of the top-k MoE expert layer (route, token sort, grouped W4A4+RAC
GEMMs with the SwiGLU epilogue, second activation site, combine) against the
oracle, stage by stage.

The silu in the W13 epilogue uses the device exp, so h cannot be bit-matched
to the fp64 oracle; h is compared within the GEMM tolerance and every later
stage is checked on the GPU's own h (the oracle quantizes it bit-exactly and
recomputes the W2 GEMM and the combine from it)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.quant import QuantResult
from workloads import WORKLOADS, bf16_bits_from_f32, make_activations, make_logits, make_moe_weights
from tests.gpu_util import GEMM_TOL, bf16_to_f64, cached, check_bf16_output, dev, gemm_rel_err, host, say
from tests.parity import check_close, check_scores, check_selection, rac_fp16_bound

pytestmark = pytest.mark.gpu


def q4():
    import fp4_w4a4_quantized_nvfp4_amd as m
    return m


def _bits(a):
    return bf16_bits_from_f32(np.asarray(a, dtype=np.float32))


def _rows(q, rows):
    return QuantResult(q.fmt, q.codes[rows], q.scales[rows], q.tensor_scale, q.resid[rows],
                       q.mag[rows], q.sign[rows])


def _swiglu64(y13, F):
    g, u = y13[:, :F], y13[:, F:]
    return g / (1.0 + np.exp(-g)) * u


def _ws_field(ws, offs, i, nbytes, dtype):
    return host(ws[offs[i]:offs[i] + nbytes].view(dtype))


# routed rows 2400 and 8192 (the one-workgroup sort, up to 8 blocks of 1024
# rows) and 8800 (the block-histogram sort, a ragged last block)
@pytest.mark.parametrize("T,E", [(300, 128), (1024, 128), (1100, 128), (300, 40)])
def test_route_and_sort(T, E):
    m = q4()
    rng = np.random.default_rng(5 + T + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[7, 10] = logits[7, 39] = logits[7].max() + 1.0           # tie at the top
    idx, w = m.q4_moe_route(dev(logits), 8)
    idx, w = host(idx), host(w)
    oi, op = oracle.moe_route(logits, 8)
    assert np.array_equal(idx, oi)
    np.testing.assert_allclose(w, op, rtol=2e-6, atol=1e-7)
    perm, off = m.q4_moe_sort(dev(idx), E)
    pe, oe = oracle.moe_sort(idx, E)
    assert np.array_equal(host(perm), pe) and np.array_equal(host(off), oe)


def _run_layer(m, xb, logits, w13, w2, topk, rac_k, fmt=0, out_dtype=1, h_ts=None,
               experts=None, fuse_h=False):
    T, H = xb.shape
    E, F2, _ = w13.shape
    F = F2 // 2
    x = dev(xb)
    idx, p = m.q4_moe_route(dev(logits), topk)
    if experts is None:
        experts = m.prepare_moe_weights(dev(w13), dev(w2), fmt=fmt)
    hts = None if h_ts is None else dev(np.array([h_ts], dtype=np.float32))
    Y, ws = m.moe_w4a4_grouped_gemm(x, idx, p, experts, rac_k, out_dtype=out_dtype,
                                    h_tensor_scale=hts, fuse_h=fuse_h)
    torch.cuda.synchronize()
    offs, _ = m.moe_workspace_layout(fmt, T, E, H, F, topk, rac_k)
    R = T * topk
    sdiv = 16 if fmt == 0 else 32
    got = {
        "idx": host(idx), "p": host(p), "Y": host(Y),
        "perm": _ws_field(ws, offs, 0, R * 4, torch.int32),
        "offsets": _ws_field(ws, offs, 1, (E + 1) * 4, torch.int32),
        "x_codes": _ws_field(ws, offs, 2, T * H // 2, torch.uint8),
        "x_scales": _ws_field(ws, offs, 3, T * H // sdiv, torch.uint8),
        "x_ts": _ws_field(ws, offs, 4, 4, torch.float32),
        "x_S": _ws_field(ws, offs, 5, rac_k * 4, torch.int32),
        "h": _ws_field(ws, offs, 7, R * F * 2, torch.int16).reshape(R, F),
        "h_codes": _ws_field(ws, offs, 8, R * F // 2, torch.uint8),
        "h_scales": _ws_field(ws, offs, 9, R * F // sdiv, torch.uint8),
        "h_ts": _ws_field(ws, offs, 10, 4, torch.float32),
        "h_S": _ws_field(ws, offs, 11, rac_k * 4, torch.int32),
        # W2 rows: bf16 with a bf16 layer output, else fp32
        "out": (bf16_to_f64(_ws_field(ws, offs, 13, R * H * 2, torch.int16).reshape(R, H))
                if out_dtype == 1 else
                _ws_field(ws, offs, 13, R * H * 4, torch.float32).reshape(R, H)),
        "x_scores": _ws_field(ws, offs, 14, H * 8, torch.float64),
        "h_scores": _ws_field(ws, offs, 15, F * 8, torch.float64),
    }
    return got, experts


def _slot_rounding_bound(got, ref, T, topk):
    """Elementwise bound on what rounding the W2 rows to bf16 adds to the
    layer output: each slot's rounded GPU row and rounded oracle row differ by
    their product error plus at most 2^-8 (|a| + |b|) (one round to nearest
    each), weighted by the slot's p."""
    pos = np.empty(T * topk, dtype=np.int64)
    pos[ref["perm"]] = np.arange(T * topk)
    yb = np.zeros((T, got["out"].shape[1]))
    for sl in range(topk):
        r = pos[np.arange(T) * topk + sl]
        yb += np.abs(got["p"][:, sl:sl + 1].astype(np.float64)) * 2.0 ** -8 * (
            np.abs(got["out"][r]) + np.abs(ref["out"][r]))
    return yb


def _check_site(fmt, xb, got, prefix, rac_k, ts=None):
    """One activation site: codes, scales and tensor scale bit-exact, scores
    within the summation bound, the channel set validated; returns the oracle
    quantization and the (validated) GPU channel set.  ``ts``: the supplied
    tensor scale the site was quantized with (NVFP4)."""
    if fmt == 0:
        q = oracle.nvfp4_quantize(xb, tensor_scale=ts)
    else:
        q = oracle.mxfp4_quantize(xb)
    assert np.array_equal(got[prefix + "_codes"].reshape(q.codes.shape), q.codes)
    assert np.array_equal(got[prefix + "_scales"].reshape(q.scales.shape), q.scales)
    if fmt == 0:
        assert got[prefix + "_ts"][0] == np.float32(q.tensor_scale)
    ref = oracle.channel_scores(q.resid)
    check_scores(got[prefix + "_scores"], ref, xb.shape[0])
    S = check_selection(got[prefix + "_S"], ref, rac_k, xb.shape[0],
                        gpu_scores=got[prefix + "_scores"])
    return q, S


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("T,H,E,F,topk,k", [(64, 256, 8, 128, 2, 16), (37, 512, 16, 64, 4, 32),
                                            (300, 256, 4, 96, 1, 8),
                                            # grouped tiles (256 x 256 for W13 when
                                            # K >= 1024): partial M tiles, gathered rows
                                            (300, 256, 2, 128, 2, 16),
                                            (520, 1024, 4, 256, 2, 32),
                                            # NVFP4: both grouped GEMMs on 128 x 512
                                            # tiles reading the tiled scale records
                                            # (K = 512 at both sites, ragged 128-row
                                            # tiles)
                                            (600, 512, 4, 512, 2, 32),
                                            # records with N not a multiple of 512:
                                            # W13 (N = 768) on 256 x 256 tiles; W2
                                            # (N = 768, K = 512) on 256 x 256 tiles
                                            (600, 512, 4, 384, 2, 32),
                                            (600, 768, 4, 512, 2, 32),
                                            # decode-shaped (streaming kernel) with the
                                            # compensation columns read from W_hi^T:
                                            # kp = 128 in two passes with padding
                                            # channels, kp = 96 as 64 + 32, column
                                            # counts not a multiple of 256; W2 with
                                            # K % 64 != 0 (NVFP4) or K % 128 != 0
                                            # (MXFP4) falls back to the gathered W_S
                                            (48, 512, 8, 160, 2, 100),
                                            (40, 256, 8, 192, 2, 70),
                                            # degenerate routing: one expert (every
                                            # token's single slot) on the streaming
                                            # and on the 128 x 512 kernels; every
                                            # expert in every token's top-k
                                            (37, 256, 1, 128, 1, 16),
                                            (600, 512, 1, 512, 1, 32),
                                            (50, 256, 4, 128, 4, 16)])
def test_small_layer_stagewise(fmt, T, H, E, F, topk, k):
    say(f"moe small fmt={fmt} T={T} H={H} E={E} F={F} topk={topk} k={k}")
    m = q4()
    rng = np.random.default_rng(T + H + E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, rng.choice(H, 3, replace=False)] *= 40
    xb = _bits(x)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w13 = _bits((rng.standard_normal((E, 2 * F, H)) * 0.05).astype(np.float32))
    w2 = _bits((rng.standard_normal((E, H, F)) * 0.05).astype(np.float32))
    got, _ = _run_layer(m, xb, logits, w13, w2, topk, k, fmt)
    oi, op = oracle.moe_route(logits, topk)
    assert np.array_equal(got["idx"], oi)
    _, Sx = _check_site(fmt, xb, got, "x", k)
    # second site on the GPU's h, bit-exact
    _, Sh = _check_site(fmt, got["h"], got, "h", k)
    ref = oracle.moe_layer(xb, got["idx"], got["p"].astype(np.float64), w13, w2, k,
                           h_override=got["h"], fmt="nvfp4" if fmt == 0 else "mxfp4",
                           Sx_override=Sx, Sh_override=Sh, out_bf16=True)
    assert np.array_equal(got["perm"], ref["perm"]) and np.array_equal(got["offsets"], ref["offsets"])
    # h (bf16) against the unrounded SwiGLU of the oracle's fp64 W13 product:
    # the GEMM tolerance plus one bf16 ulp
    check_bf16_output(got["h"], _swiglu64(ref["y13"], F), tol=2 * GEMM_TOL)
    # W2 rows (bf16): the GEMM tolerance plus their rounding
    err_o = check_close(got["out"], ref["out"], GEMM_TOL, bf16_ulp=True)
    say(f"  W2 out rel err {err_o:.2e}")
    check_close(bf16_to_f64(got["Y"]), ref["y"], 2 * GEMM_TOL,
                extra=_slot_rounding_bound(got, ref, T, topk), bf16_ulp=True)


@pytest.mark.parametrize("fmt", [0, 1], ids=["nvfp4", "mxfp4"])
@pytest.mark.parametrize("T,H,E,F,topk,k", [(600, 512, 4, 512, 2, 32),   # 128 x 512 tiles (NVFP4)
                                            (40, 256, 8, 192, 2, 70)])   # streaming kernel
def test_small_layer_f32_output(fmt, T, H, E, F, topk, k):
    """An fp32 layer output keeps the W2 rows in fp32: they are within the
    GEMM tolerance of the oracle's exact rows with no rounding allowance, and
    the output is the oracle's unrounded combine within twice that."""
    say(f"moe f32 out fmt={fmt} T={T} H={H} E={E} F={F} topk={topk} k={k}")
    m = q4()
    rng = np.random.default_rng(3 * T + H + E)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, rng.choice(H, 3, replace=False)] *= 40
    xb = _bits(x)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w13 = _bits((rng.standard_normal((E, 2 * F, H)) * 0.05).astype(np.float32))
    w2 = _bits((rng.standard_normal((E, H, F)) * 0.05).astype(np.float32))
    got, _ = _run_layer(m, xb, logits, w13, w2, topk, k, fmt, out_dtype=0)
    assert got["out"].dtype == np.float32 and got["Y"].dtype == np.float32
    _, Sx = _check_site(fmt, xb, got, "x", k)
    _, Sh = _check_site(fmt, got["h"], got, "h", k)
    ref = oracle.moe_layer(xb, got["idx"], got["p"].astype(np.float64), w13, w2, k,
                           h_override=got["h"], fmt="nvfp4" if fmt == 0 else "mxfp4",
                           Sx_override=Sx, Sh_override=Sh)
    err_o = gemm_rel_err(got["out"], ref["out"])
    say(f"  W2 out rel err {err_o:.2e}")
    assert err_o <= GEMM_TOL
    check_close(got["Y"], ref["y"], 2 * GEMM_TOL)


@pytest.mark.parametrize("fmt", [0, 1], ids=["nvfp4", "mxfp4"])
def test_empty_token_batch(fmt):
    """T = 0: the layer runs, writes nothing and reports no error."""
    m = q4()
    E, H, F, topk, k = 4, 256, 128, 2, 16
    rng = np.random.default_rng(9)
    w13 = _bits((rng.standard_normal((E, 2 * F, H)) * 0.05).astype(np.float32))
    w2 = _bits((rng.standard_normal((E, H, F)) * 0.05).astype(np.float32))
    experts = m.prepare_moe_weights(dev(w13), dev(w2), fmt=fmt)
    x = torch.empty((0, H), dtype=torch.int16, device="cuda")
    idx = torch.empty((0, topk), dtype=torch.int32, device="cuda")
    p = torch.empty((0, topk), dtype=torch.float32, device="cuda")
    st = torch.zeros((1,), dtype=torch.int32, device="cuda")
    Y, _ = m.moe_w4a4_grouped_gemm(x, idx, p, experts, k, out_dtype=m.OUT_BF16, status=st)
    torch.cuda.synchronize()
    assert tuple(Y.shape) == (0, H) and int(host(st)[0]) == 0


@pytest.mark.parametrize("fuse", [True, False], ids=["fused", "separate"])
@pytest.mark.parametrize("T,H,E,F,topk,k", [(600, 512, 4, 512, 2, 32),      # records at both sites
                                            (520, 1024, 4, 256, 2, 32),     # W2 on 256 x 128 tiles
                                            (700, 1024, 3, 128, 2, 0)])     # no compensation
def test_fused_h_quantization(T, H, E, F, topk, k, fuse):
    """A supplied h tensor scale on a prefill-shaped layer, h quantized in
    the W13 epilogue (fused, on 256 x 256 tiles) or by the quantizer without
    an amax pass (separate).  With s_h equal to the in-call one, below it
    (saturated blocks) and above it: h agrees with the in-call layer's (whose
    tiles may order the sums of experts' last rows differently) within the
    GEMM tolerance, codes and scales are bit-exact against the oracle's
    quantization of the GPU's h under that s_h, scores within the bound, the
    selection valid, and the W2 product and the layer output agree with the
    oracle."""
    say(f"moe supplied s_h ({'fused' if fuse else 'separate'}) T={T} H={H} E={E} F={F} "
        f"topk={topk} k={k}")
    m = q4()
    rng = np.random.default_rng(T + 7 * H + F)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, rng.choice(H, 3, replace=False)] *= 40
    xb = _bits(x)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    w13 = _bits((rng.standard_normal((E, 2 * F, H)) * 0.05).astype(np.float32))
    w2 = _bits((rng.standard_normal((E, H, F)) * 0.05).astype(np.float32))
    experts = m.prepare_moe_weights(dev(w13), dev(w2))
    base, _ = _run_layer(m, xb, logits, w13, w2, topk, k, experts=experts)
    s_h = float(base["h_ts"][0])
    for mult in (1.0, 0.37, 3.0):
        ts = float(np.float32(s_h * mult))
        got, _ = _run_layer(m, xb, logits, w13, w2, topk, k, h_ts=ts, experts=experts,
                            fuse_h=fuse)
        assert np.array_equal(got["x_S"], base["x_S"])
        assert got["h_ts"][0] == np.float32(ts)
        check_bf16_output(got["h"], bf16_to_f64(base["h"]), tol=2 * GEMM_TOL)
        _, Sh = _check_site(0, got["h"], got, "h", k, ts=ts)
        _, Sx = _check_site(0, xb, got, "x", k)
        ref = oracle.moe_layer(xb, got["idx"], got["p"].astype(np.float64), w13, w2, k,
                               h_override=got["h"], Sx_override=Sx, Sh_override=Sh,
                               h_tensor_scale=ts, out_bf16=True)
        # a scale below h's amax / 2688 saturates blocks, whose large residuals
        # make the compensation a large part of the output: its fp16 operands'
        # rounding (rac_fp16_bound) is then allowed on top of the tolerance
        bound = np.zeros_like(ref["out"])
        off = ref["offsets"]
        for e in range(E):
            r0, r1 = off[e], off[e + 1]
            if r1 > r0 and k:
                Wsel = bf16_to_f64(w2[e])[:, Sh]
                bound[r0:r1] = rac_fp16_bound(bf16_to_f64(ref["Rh"][r0:r1]), Wsel, ts,
                                              float(experts["w2"]["tensor_scale"][e]))
        err_o = check_close(got["out"], ref["out"], GEMM_TOL, extra=bound, bf16_ulp=True)
        say(f"  s_h x {mult}: W2 out rel err {err_o:.2e} "
            f"(compensation rounding bound up to {float((bound / np.maximum(np.abs(ref['out']), 1e-30)).max()):.1e})")
        pos = np.empty(T * topk, dtype=np.int64)
        pos[ref["perm"]] = np.arange(T * topk)
        yb = _slot_rounding_bound(got, ref, T, topk)
        for sl in range(topk):
            yb += got["p"][:, sl:sl + 1].astype(np.float64) * bound[pos[np.arange(T) * topk + sl]]
        check_close(bf16_to_f64(got["Y"]), ref["y"], 2 * GEMM_TOL, extra=yb, bf16_ulp=True)


def test_scale_records_layout():
    """q4_scale_records against the documented layout.  First part: record
    (c, r) of operand b holds the E4M3 scales of row r, columns 128 c ..
    128 c + 127, as fp16, dword d stored at d ^ ((r / 8) % 4); the expected
    fp16 values are the oracle's E4M3 decoding (exact in fp16).  Second part:
    the same scales' raw bytes, 8 per record, in block order.  Rows past
    `rows` are zero in both."""
    m = q4()
    rng = np.random.default_rng(11)
    b, rows, K = 3, 300, 384
    sc = rng.integers(0, 127, size=(b, rows, K // 16), dtype=np.uint8)   # every finite E4M3 code
    flat = host(m.q4_scale_records(dev(sc), K))
    pad = 512
    n16 = b * (K // 128) * pad * 16
    assert flat.size == n16 + b * (K // 128) * pad * 8
    raw = flat[n16:].reshape(b, K // 128, pad, 8)
    assert np.array_equal(raw[:, :, :rows], sc.reshape(b, rows, K // 128, 8).transpose(0, 2, 1, 3))
    assert not raw[:, :, rows:].any()
    rec = flat[:n16].reshape(b, K // 128, pad, 4, 4)
    assert rec.shape[2] == pad
    vals = rec.view(np.uint16).view(np.float16).astype(np.float64)    # [b][c][row][dword][2 halves]
    vals = vals.reshape(b, K // 128, pad, 4, 2)
    for r in range(pad):
        q = (r // 8) % 4
        d_store = np.arange(4) ^ q                                     # logical dword d is stored at d ^ q
        logical = vals[:, :, r, d_store, :].reshape(b, K // 128, 8)    # scale 2 d + half
        if r < rows:
            want = oracle.formats.E4M3_VALUES[sc[:, r, :].astype(np.int64)].reshape(b, K // 128, 8)
            assert np.array_equal(logical, want), r
        else:
            assert not logical.any(), r


def test_transpose_interleaved_layout():
    """q4_transpose_bf16 of stacked matrices: out[c][b][r] = in[b][r][c]
    (channel-major, matrices interleaved); one matrix: the plain transpose."""
    m = q4()
    rng = np.random.default_rng(14)
    x = rng.integers(0, 1 << 16, size=(3, 70, 130), dtype=np.uint16)
    got = host(m.q4_transpose_bf16(dev(x)))
    assert got.shape == (130, 3, 70) and np.array_equal(got, x.transpose(2, 0, 1))
    got1 = host(m.q4_transpose_bf16(dev(x[1])))
    assert np.array_equal(got1, x[1].T)


def test_mx_scale_records_layout():
    """MXFP4 records: record (c, r) of operand b is the four E8M0 bytes of row
    r, blocks 4 c .. 4 c + 3, in order; rows past `rows` are zero."""
    m = q4()
    rng = np.random.default_rng(13)
    b, rows, K = 2, 300, 512
    sc = rng.integers(0, 256, size=(b, rows, K // 32), dtype=np.uint8)
    rec = host(m.q4_scale_records(dev(sc), K, fmt=m.MXFP4)).reshape(b, K // 128, 512, 4)
    want = sc.reshape(b, rows, K // 128, 4).transpose(0, 2, 1, 3)
    assert np.array_equal(rec[:, :, :rows], want)
    assert not rec[:, :, rows:].any()


@pytest.mark.parametrize("T,H,E,F,topk,k", [(600, 1024, 4, 1024, 2, 32),   # NVFP4: 128 x 512
                                            # tiles with the records, 256 x 256
                                            # without; MXFP4: 256 x 256 both
                                            # decode-shaped: the streaming kernel with
                                            # the raw E4M3 records (NVFP4) against
                                            # the raw scales
                                            (64, 1024, 16, 512, 4, 32),
                                            (48, 768, 8, 384, 8, 0)])
@pytest.mark.parametrize("fmt", [0, 1])
def test_scale_records_same_result(T, H, E, F, topk, k, fmt):
    """The grouped layer with the weights' scale records equals the layer
    without them bit for bit: the records change where the scales come from,
    not the arithmetic.  At K >= 1024 the prefill-shaped NVFP4 layer runs
    128 x 512 tiles with the records and 256 x 256 tiles without, and each
    output element still sums the same products in the same order; the
    decode-shaped layer runs the streaming kernel either way."""
    m = q4()
    rng = np.random.default_rng(12 + T)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, rng.choice(H, 3, replace=False)] *= 40
    logits = dev(rng.standard_normal((T, E)).astype(np.float32))
    w13 = dev(_bits((rng.standard_normal((E, 2 * F, H)) * 0.05).astype(np.float32)))
    w2 = dev(_bits((rng.standard_normal((E, H, F)) * 0.05).astype(np.float32)))
    xd = dev(_bits(x))
    idx, p = m.q4_moe_route(logits, topk)
    with_rec = m.prepare_moe_weights(w13, w2, fmt=fmt)
    without = m.prepare_moe_weights(w13, w2, fmt=fmt, scale_records=False)
    assert "scale_records" in with_rec["w13"] and "scale_records" not in without["w13"]
    Y1, ws1 = m.moe_w4a4_grouped_gemm(xd, idx, p, with_rec, k, out_dtype=m.OUT_F32)
    Y0, ws0 = m.moe_w4a4_grouped_gemm(xd, idx, p, without, k, out_dtype=m.OUT_F32)
    torch.cuda.synchronize()
    offs, _ = m.moe_workspace_layout(fmt, T, E, H, F, topk, k)
    R = T * topk
    h1 = _ws_field(ws1, offs, 7, R * F * 2, torch.int16)
    h0 = _ws_field(ws0, offs, 7, R * F * 2, torch.int16)
    assert np.array_equal(h1, h0)
    assert np.array_equal(host(Y1).view(np.uint32), host(Y0).view(np.uint32))


def _quant(fmt):
    return oracle.nvfp4_quantize if fmt == 0 else oracle.mxfp4_quantize


def _w13_packed_order(F):
    """Logical W13 row of each packed row: groups of 32 gate rows then the
    matching 32 up rows (the documented q4_moe_pack_w13 layout)."""
    p = np.arange(2 * F)
    g, i = p // 64, p % 64
    return np.where(i < 32, 32 * g + i, F + 32 * g + (i - 32))


def _gpu_weights(experts, key, fmt, e, order=None):
    """The GPU's quantization of expert e as an oracle QuantResult (codes and
    scales in logical row order)."""
    q = experts[key]
    codes = host(q["codes"][e])
    scales = host(q["scales"][e])
    if order is not None:
        inv = np.empty_like(order)
        inv[order] = np.arange(order.size)
        codes, scales = codes[inv], scales[inv]
    ts = np.float32(host(q["tensor_scale"][e:e + 1])[0]) if fmt == 0 else np.float32(1.0)
    return QuantResult("nvfp4" if fmt == 0 else "mxfp4", codes, scales, ts, None, None, None)


def _check_weight_sample(fmt, wl_bits, Wq, rng, n=8):
    """The GPU's expert weight quantization: tensor scale = RN32(amax / 2688)
    (NVFP4) and n random rows bit-exact against the oracle."""
    if fmt == 0:
        amax = float(np.abs(bf16_to_f64(wl_bits)).max())
        st = np.float32(amax / 2688.0) if amax else np.float32(1.0)
        assert Wq.tensor_scale == st
    rows = np.sort(rng.choice(wl_bits.shape[0], n, replace=False))
    o = _quant(fmt)(wl_bits[rows], tensor_scale=float(Wq.tensor_scale)) if fmt == 0 else \
        _quant(fmt)(wl_bits[rows])
    assert np.array_equal(Wq.codes[rows], o.codes) and np.array_equal(Wq.scales[rows], o.scales)


def _full_layer(name, fmt=0):
    """The whole workload layer against the oracle: routing of every token,
    the sort, both activation sites, the W13 product (through h) and the W2
    product of EVERY expert, and the combine; the expert weight codes are the
    GPU's, each expert's tensor scale and a row sample checked bit-exact."""
    m = q4()
    wl = WORKLOADS[name]
    T, H, E, F, topk, k = wl.rows, wl.cols, wl.experts, wl.ffn, wl.route_topk, wl.topk_channels
    say(f"moe {name} fmt={fmt}: generating inputs")
    xb = cached(name + "_x", lambda: make_activations(wl))
    logits = cached(name + "_logits", lambda: make_logits(wl))
    w13, w2 = cached(name + "_w", lambda: make_moe_weights(wl))
    say(f"moe {name}: GPU layer")
    got, experts = _run_layer(m, xb, logits, w13, w2, topk, k, fmt)
    say(f"moe {name}: routing of all {T} tokens")
    oi, op = cached(name + "_route", lambda: oracle.moe_route(logits, topk))
    assert np.array_equal(got["idx"], oi)
    np.testing.assert_allclose(got["p"], op, rtol=2e-6, atol=1e-7)
    perm, offsets = oracle.moe_sort(got["idx"], E)
    assert np.array_equal(got["perm"], perm) and np.array_equal(got["offsets"], offsets)
    say(f"moe {name}: site 1")
    qx, Sx = _check_site(fmt, xb, got, "x", k)
    Rx = oracle.residual_gather(qx.resid, Sx)
    say(f"moe {name}: site 2")
    qh, Sh = _check_site(fmt, got["h"], got, "h", k)
    Rh = oracle.residual_gather(qh.resid, Sh)
    order = _w13_packed_order(F)
    tok = perm // topk
    rng = np.random.default_rng(1)
    worst13 = worst2 = 0.0
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        wq13 = _gpu_weights(experts, "w13", fmt, e, order)
        wq2 = _gpu_weights(experts, "w2", fmt, e)
        _check_weight_sample(fmt, w13[e], wq13, rng)
        _check_weight_sample(fmt, w2[e], wq2, rng)
        if r1 == r0:
            continue
        y13 = oracle.rac_gemm(_rows(qx, tok[r0:r1]), wq13, Rx[tok[r0:r1]], w13[e], Sx)
        hr = _swiglu64(y13, F)
        check_bf16_output(got["h"][r0:r1], hr, tol=2 * GEMM_TOL)
        rows = np.arange(r0, r1)
        out_ref = oracle.rac_gemm(_rows(qh, rows), wq2, Rh[rows], w2[e], Sh)
        # bf16 W2 rows: the GEMM tolerance plus their rounding
        err = check_close(got["out"][r0:r1], out_ref, GEMM_TOL, bf16_ulp=True)
        worst2 = max(worst2, err)
        worst13 = max(worst13, gemm_rel_err(bf16_to_f64(got["h"][r0:r1]), hr))
    say(f"moe {name}: all {E} experts; h max rel err {worst13:.2e} (bf16 output), "
        f"W2 out max rel err {worst2:.2e}")
    # combine on the GPU's out and routing weights
    pos = np.empty(T * topk, dtype=np.int64)
    pos[perm] = np.arange(T * topk)
    y = np.zeros((T, H))
    for s in range(topk):
        y += got["p"][:, s:s + 1].astype(np.float64) * got["out"][pos[np.arange(T) * topk + s]]
    check_bf16_output(got["Y"], y)


@pytest.mark.parametrize("fmt", [0, 1], ids=["nvfp4", "mxfp4"])
def test_moe_decode_workload_full(fmt):
    """256 tokens, 128 experts of 4096 -> 2 x 1536 -> 4096, top-8: run as NVFP4
    and again as MXFP4 (E8M0 per 32, native scaled FP4 MFMA); every expert."""
    _full_layer("moe_decode_256", fmt=fmt)


@pytest.mark.parametrize("fmt", [0, 1], ids=["nvfp4", "mxfp4"])
def test_moe_prefill_workload_full(fmt):
    """8192 tokens, 128 experts of 2048 -> 2 x 768 -> 2048, top-8, as NVFP4 and as
    MXFP4; every expert, every token."""
    _full_layer("moe_prefill_8192", fmt=fmt)
