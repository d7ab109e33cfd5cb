"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test ties the oracle to something other than itself: the E2M1 grid and
E4M3 maximum printed on the QUADS page (section 2.2), hand-worked fixtures in
tests/golden/, brute force over every candidate with exact rational
arithmetic, closed forms, invariants and library routines.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_from_f32, f32_from_bf16_bits, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGE_GRID = [0, 0.5, 1, 1.5, 2, 3, 4, 6]           # QUADS section 2.2 "FP4"


def _bits(vals):
    return bf16_bits_from_f32(np.asarray(vals, dtype=np.float32))


def _frac_e4m3():
    return [Fraction(oracle.e4m3_value(c)) for c in range(127)]


def _nearest_even(value: Fraction, table):
    """Brute force: index of the nearest table entry, ties -> even index, saturating."""
    best, bd = None, None
    for i, t in enumerate(table):
        d = abs(value - t)
        if bd is None or d < bd or (d == bd and i % 2 == 0):
            best, bd = i, d
    return best


# ---------------------------------------------------------------- formats
def test_e2m1_grid_matches_page():
    vals = [oracle.e2m1_value(n) for n in range(16)]
    assert vals[:8] == PAGE_GRID
    assert vals[8:] == [-v for v in PAGE_GRID]


def test_e4m3_table_against_torch_decode():
    assert len(oracle.E4M3_VALUES) == 127
    assert oracle.E4M3_MAX == 448.0                     # section 2.2 "FP8"
    assert np.all(np.diff(oracle.E4M3_VALUES) > 0)
    codes = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn)
    ref = codes.to(torch.float64).numpy()
    np.testing.assert_array_equal(ref, oracle.E4M3_VALUES)


def test_bf16_rounding_against_torch():
    rng = np.random.default_rng(1)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16_bits(f), ref)
    np.testing.assert_array_equal(oracle.f64_to_bf16_bits(f.astype(np.float64)), ref)
    # single rounding from fp64: 1 + 2^-8 + 2^-30 is above the bf16 midpoint
    # 1 + 2^-8, so it rounds up; rounding through fp32 first would tie to 1.0
    v = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.f64_to_bf16_bits(np.array([v]))[0] == 0x3F81


# ---------------------------------------------------------------- golden
def _load(name):
    rows = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    return rows


def test_golden_block_ties():
    rows = _load("nvfp4_block_ties.txt")
    x = np.array([[float(r[0]) for r in rows]], dtype=np.float32)
    q = oracle.nvfp4_quantize(_bits(x), tensor_scale=1.0)
    assert q.scales[0, 0] == 0x38
    nib = np.empty(16, dtype=np.uint8)
    nib[0::2], nib[1::2] = q.codes[0] & 0xF, q.codes[0] >> 4
    assert nib.tolist() == [int(r[1]) for r in rows]
    deq = oracle.dequantize(q)[0]
    exp = np.array([float(r[2]) for r in rows])
    np.testing.assert_array_equal(deq, exp)
    np.testing.assert_array_equal(np.signbit(deq), np.signbit(exp))


def test_golden_tensor_scale():
    for amax, bits in _load("nvfp4_tensor_scale.txt"):
        amax = float(amax)
        x = np.zeros((1, 32), dtype=np.float32)
        x[0, 17] = amax
        q = oracle.nvfp4_quantize(_bits(x))
        assert int(np.float32(q.tensor_scale).view(np.uint32)) == int(bits, 16)
        if amax:
            assert q.scales[0, 1] == 0x7E                # block holding amax -> 448
            assert q.mag[0, 17] == 7                     # amax -> code 6


# ---------------------------------------------------------------- brute force
def _random_bf16_blocks(rng, rows, cols, spread=8.0):
    x = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-spread, spread, (rows, 1)))
    x[rng.random((rows, cols)) < 0.05] = 0.0
    x[rng.random((rows, cols)) < 0.02] *= -0.0
    return _bits(x.astype(np.float32))


@pytest.mark.parametrize("seed,supplied", [(0, None), (1, None), (2, 0.37), (3, 3.0e-3)])
def test_nvfp4_brute_force_exact(seed, supplied):
    rng = np.random.default_rng(seed)
    xb = _random_bf16_blocks(rng, 6, 64)
    q = oracle.nvfp4_quantize(xb, tensor_scale=supplied)
    x = f32_from_bf16_bits(xb).astype(np.float64)
    st = Fraction(float(q.tensor_scale))
    if supplied is None:
        amax = Fraction(float(np.abs(x).max()))
        cands = [np.float32(float(amax / 2688))]
        cands += [np.nextafter(cands[0], np.float32(0)), np.nextafter(cands[0], np.float32(1e30))]
        best = min(cands, key=lambda c: abs(Fraction(float(c)) - amax / 2688))
        assert np.float32(q.tensor_scale) == best
    e4 = _frac_e4m3()
    grid = [Fraction(v) for v in PAGE_GRID]
    for i in range(x.shape[0]):
        for b in range(x.shape[1] // 16):
            blk = [Fraction(float(v)) for v in x[i, 16 * b:16 * b + 16]]
            ab = max(abs(v) for v in blk)
            sbc = _nearest_even(ab / (6 * st), e4)
            assert q.scales[i, b] == sbc, (i, b)
            sb = e4[sbc]
            for j, v in enumerate(blk):
                col = 16 * b + j
                mag = 0 if sb == 0 else _nearest_even(abs(v) / (sb * st), grid)
                assert q.mag[i, col] == mag, (i, col)
                assert q.sign[i, col] == np.signbit(x[i, col])
                deq = (-1 if np.signbit(x[i, col]) else 1) * grid[mag] * sb * st
                exact = v - deq
                r = np.float32(float(exact))
                # r must be the fp32 nearest to the exact residual
                for nb in (np.nextafter(r, np.float32(np.inf)), np.nextafter(r, np.float32(-np.inf))):
                    assert abs(Fraction(float(r)) - exact) <= abs(Fraction(float(nb)) - exact)
                assert q.resid[i, col] == r


def test_e2m1_every_bf16_value_unit_scale():
    # every bf16 in [-6, 6] with a block scale of exactly 1 (a 6.0 in each block)
    vals = f32_from_bf16_bits(np.arange(0, 0x40C1, dtype=np.uint16))
    vals = np.concatenate([vals, -vals])
    n = (len(vals) + 14) // 15
    blocks = np.full((n, 16), 6.0, dtype=np.float32)
    flat = blocks[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(n, 15)
    xb = _bits(blocks.reshape(1, -1))
    q = oracle.nvfp4_quantize(xb, tensor_scale=1.0)
    assert np.all(q.scales == 0x38)
    grid = [Fraction(v) for v in PAGE_GRID]
    x = f32_from_bf16_bits(xb)[0]
    for col in range(x.shape[0]):
        assert q.mag[0, col] == _nearest_even(abs(Fraction(float(x[col]))), grid)


def test_e4m3_scale_ties_go_to_even_code():
    e4 = oracle.E4M3_VALUES
    for c in range(60, 126):
        mid = (e4[c] + e4[c + 1]) / 2
        amax = 6.0 * mid                      # u = mid exactly with s_t = 1
        if np.float32(amax) != amax or f32_from_bf16_bits(_bits([amax]))[0] != amax:
            continue                          # needs more bits than bf16 holds
        x = np.zeros((1, 16), dtype=np.float32)
        x[0, 3] = amax
        q = oracle.nvfp4_quantize(_bits(x), tensor_scale=1.0)
        assert q.scales[0, 0] == (c if c % 2 == 0 else c + 1)


# ---------------------------------------------------------------- invariants
@pytest.fixture(scope="module")
def c1():
    d = make_inputs("dense_64x512")
    return d, oracle.nvfp4_quantize(d["x"])


def _t3_bits(seed=7, rows=256, cols=512):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    x[:, rng.choice(cols, 5, replace=False)] *= 80
    return _bits(x)


@pytest.mark.parametrize("which", ["c1", "t3"])
def test_block_invariants(c1, which):
    xb = c1[0]["x"] if which == "c1" else _t3_bits()
    q = oracle.nvfp4_quantize(xb)
    x = f32_from_bf16_bits(xb).astype(np.float64)
    M, K = x.shape
    sb = oracle.E4M3_VALUES[q.scales.astype(int)]
    st = float(q.tensor_scale)
    ax = np.abs(x).reshape(M, K // 16, 16)
    arg = ax.argmax(axis=2)
    mags = q.mag.reshape(M, K // 16, 16)
    top = np.take_along_axis(mags, arg[..., None], axis=2)[..., 0]
    normal = sb >= 2.0 ** -6
    assert np.all(top[normal] == 7)                      # block amax -> code 6
    # half a grid step (0.25 / 0.5 / 1 on [0,2] / [2,4] / [4,6]) times the scale
    S = np.repeat(sb, 16, axis=1) * st
    v = np.abs(x) / np.where(S == 0, 1, S)
    gap = np.where(v <= 2, 0.5, np.where(v <= 4, 1.0, 2.0))
    err = np.abs(x - oracle.dequantize(q))
    sat = v > 6
    assert np.all(err[~sat] <= gap[~sat] / 2 * S[~sat])
    assert np.all(err[sat & normal.repeat(16, 1)] <= 0.4 * S[sat & normal.repeat(16, 1)])
    # sign symmetry (bitwise) and zero preservation
    qn = oracle.nvfp4_quantize(xb ^ np.uint16(0x8000))
    np.testing.assert_array_equal(qn.codes, q.codes ^ np.uint8(0x88))
    np.testing.assert_array_equal(qn.scales, q.scales)
    np.testing.assert_array_equal(qn.resid, -q.resid)
    zero = x == 0
    assert np.all(q.mag[zero] == 0)
    # the tensor's amax lands on scale 448 and code 6
    i, j = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q.scales[i, j // 16] == 0x7E and q.mag[i, j] == 7


def test_all_zero_tensor():
    q = oracle.nvfp4_quantize(np.zeros((3, 32), dtype=np.uint16))
    assert q.tensor_scale == 1.0 and np.all(q.scales == 0) and np.all(q.codes == 0)
    assert np.all(q.resid == 0)


def test_round_trip_unit_tensor_scale(c1):
    q = oracle.nvfp4_quantize(c1[0]["x"], tensor_scale=1.0)
    deq = oracle.dequantize(q)
    q2 = oracle.nvfp4_quantize(_bits(deq.astype(np.float32)), tensor_scale=1.0)
    has6 = (q.mag.reshape(q.mag.shape[0], -1, 16) == 7).any(axis=2)
    np.testing.assert_array_equal(q2.scales[has6], q.scales[has6])
    c = q.mag.reshape(q.mag.shape[0], -1, 16)
    c2 = q2.mag.reshape(q.mag.shape[0], -1, 16)
    np.testing.assert_array_equal(c2[has6], c[has6])


# ---------------------------------------------------------------- scores / top-k
def test_scores_exact_and_topk_brute_force():
    """Eq. 23 squared: each channel's score is the fp64 value nearest to the
    exact sum of squared residuals (float() of a Fraction rounds correctly),
    so the oracle must equal it bit for bit; Eq. 24: top-k by brute force."""
    xb = _t3_bits(rows=130, cols=64)
    q = oracle.nvfp4_quantize(xb)
    s = oracle.channel_scores(q.resid)
    ex = [sum(Fraction(float(v)) ** 2 for v in q.resid[:, j]) for j in range(64)]
    assert [float(e) for e in ex] == s.tolist()
    for k in (0, 1, 5, 17, 64):
        brute = sorted(sorted(range(64), key=lambda j: (-ex[j], j))[:k])
        assert oracle.select_topk(s, k).tolist() == brute
    # ties -> smaller index
    assert oracle.select_topk(np.array([1.0, 2.0, 2.0, 0.0, 2.0]), 2).tolist() == [1, 2]


def test_scores_extreme_exponents_exact():
    """Residuals spanning the whole fp32 range (subnormals to 1e38) in one
    channel: still the correctly rounded exact sum."""
    rng = np.random.default_rng(8)
    r = (rng.standard_normal((300, 24)) * np.exp(rng.uniform(-85, 85, (300, 24)))).astype(np.float32)
    r[0, 0], r[1, 0], r[2, 0] = 3.0e38, 1.0e-45, -2.0e-40
    r[:, 5] = 0.0
    s = oracle.channel_scores(r)
    for j in range(24):
        assert s[j] == float(sum(Fraction(float(v)) ** 2 for v in r[:, j])), j
    assert s[5] == 0.0


def test_scores_order_free_closed_form():
    """The score has no summation order: 1 + three squares of 2^-27 is
    1 + 1.5 * 2^-53 exactly, whose nearest fp64 is 1 + 2^-52, wherever the
    four rows sit; a row permutation leaves every score bit-identical."""
    e = np.float32(2.0 ** -27)
    for rows in ([1, 2, 3], [32, 64, 96], [256, 288, 511], [5, 300, 700]):
        r = np.zeros((1024, 1), dtype=np.float32)
        r[0, 0] = 1.0
        r[rows, 0] = e
        assert oracle.channel_scores(r)[0] == 1.0 + 2.0 ** -52
        r2 = r[::-1].copy()
        assert oracle.channel_scores(r2)[0] == 1.0 + 2.0 ** -52
    # one square of 2^-27 is a quarter of an ulp of 1 (rounds down); two make
    # exactly half an ulp, a tie that goes to the even neighbour 1.0
    for n in (1, 2):
        r = np.zeros((4, 1), dtype=np.float32)
        r[0, 0] = 1.0
        r[1:1 + n, 0] = e
        assert oracle.channel_scores(r)[0] == 1.0
    q = oracle.nvfp4_quantize(_t3_bits(seed=3, rows=300, cols=96))
    perm = np.random.default_rng(1).permutation(300)
    np.testing.assert_array_equal(oracle.channel_scores(q.resid[perm]).view(np.uint64),
                                  oracle.channel_scores(q.resid).view(np.uint64))


def test_selection_lands_in_outlier_blocks(c1):
    # Figure 4a: residual concentrates in persistent channel bands
    d, q = c1
    S = oracle.select_topk(oracle.channel_scores(q.resid), 16)
    x = f32_from_bf16_bits(d["x"])
    outl = set(np.where(np.abs(x).mean(axis=0) > 10)[0] // 16)
    assert len(outl) == 4
    assert set((S // 16).tolist()) <= outl


# ---------------------------------------------------------------- GEMM
def _exact_operand(rng, rows, cols, scales=(0.5, 1.0, 2.0)):
    """bf16 tensor whose NVFP4 form (s_t = 1) has known block scales and codes."""
    sb = rng.choice(scales, size=(rows, cols // 16))
    mag = rng.integers(0, 8, size=(rows, cols))
    mag[:, ::16] = 7                                     # one 6 per block pins sb
    sign = rng.random((rows, cols)) < 0.5
    val = np.array(PAGE_GRID)[mag] * np.repeat(sb, 16, axis=1) * np.where(sign, -1, 1)
    return _bits(val.astype(np.float32)), val


def test_w4a4_gemm_exact_special_case():
    rng = np.random.default_rng(11)
    xb, xv = _exact_operand(rng, 48, 256)
    wb, wv = _exact_operand(rng, 40, 256)
    A = oracle.nvfp4_quantize(xb, tensor_scale=1.0)
    W = oracle.nvfp4_quantize(wb, tensor_scale=1.0)
    np.testing.assert_array_equal(oracle.dequantize(A), xv)
    y = oracle.w4a4_gemm(A, W)
    ia, iw = (xv * 4).astype(np.int64), (wv * 4).astype(np.int64)   # integers
    exact = (ia @ iw.T).astype(np.float64) / 16.0
    np.testing.assert_array_equal(y, exact)


def test_rac_closed_forms(c1):
    d, A = c1
    W = oracle.nvfp4_quantize(d["w"])
    S0 = np.zeros(0, dtype=np.int32)
    R0 = oracle.residual_gather(A.resid, S0)
    np.testing.assert_array_equal(oracle.rac_gemm(A, W, R0, d["w"], S0), oracle.w4a4_gemm(A, W))
    # full channel set against the dequantized weight as "bf16 weight":
    # Y = (deq_A + bf16(r)) @ W_d^T, which is x @ W_d^T up to the bf16 rounding of r
    K = A.resid.shape[1]
    S = np.arange(K, dtype=np.int32)
    W = oracle.nvfp4_quantize(d["w"], tensor_scale=2.0 ** -8)   # dequant exact in bf16
    wd = oracle.dequantize(W)
    wd_bits = _bits(wd.astype(np.float32))
    assert np.array_equal(f32_from_bf16_bits(wd_bits).astype(np.float64), wd)
    R = oracle.residual_gather(A.resid, S)
    y = oracle.rac_gemm(A, W, R, wd_bits, S)
    x = f32_from_bf16_bits(d["x"]).astype(np.float64)
    ref = x @ wd.T
    rerr = f32_from_bf16_bits(R).astype(np.float64) - A.resid.astype(np.float64)
    bound = np.abs(rerr) @ np.abs(wd.T) + 1e-9 * np.abs(ref).max()
    assert np.all(np.abs(y - ref) <= bound)
    # Eq. 22: compensation on S moves the activation closer to X
    S16 = oracle.select_topk(oracle.channel_scores(A.resid), 16)
    deq = oracle.dequantize(A)
    xt = deq.copy()
    xt[:, S16] += f32_from_bf16_bits(oracle.residual_gather(A.resid, S16))
    assert np.linalg.norm(xt - x) < np.linalg.norm(deq - x)


def test_eq21_literal_reduces_error(c1):
    d, A = c1
    W = oracle.nvfp4_quantize(d["w"])
    S = oracle.select_topk(oracle.channel_scores(A.resid), 64)
    x = f32_from_bf16_bits(d["x"]).astype(np.float64)
    wd = oracle.dequantize(W)
    ref = x @ wd.T
    y0 = oracle.w4a4_gemm(A, W)
    y1 = oracle.rac_gemm_eq21(d["x"], A, W, S)
    assert np.linalg.norm(y1 - ref) < np.linalg.norm(y0 - ref)


def test_golden_eq21_mask_after_quantize():
    """Eq. 21's order (mask applied to the quantized residual), worked by hand
    in tests/golden/eq21_mask_after_quantize.txt: a selected channel whose
    16-block holds a larger unselected residual is quantized at that block's
    scale (here to zero), which masking before quantizing would not do."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :3] = [5.25, 1.9140625, 0.87890625]
    w = np.zeros((2, 32), dtype=np.float32)
    w[0, 2] = 5.25
    w[1, :3] = 5.25
    xb, wb = _bits(x), _bits(w)
    A = oracle.nvfp4_quantize(xb)
    W = oracle.nvfp4_quantize(wb)
    assert float(A.tensor_scale) == 2.0 ** -9 and float(W.tensor_scale) == 2.0 ** -9
    Q = oracle.eq21_residual_quant(A)
    assert float(Q.tensor_scale) == 2.0 ** -14 and Q.scales[0, 0] == 0x7E
    assert Q.mag[0, 1] == 7 and Q.mag[0, 2] == 0
    for S, y0, y1, before in _load("eq21_mask_after_quantize.txt"):
        S = np.array([int(s) for s in S.split(",")], dtype=np.int64)
        y = oracle.rac_gemm_eq21(xb, A, W, S)
        assert y.tolist() == [[float(y0), float(y1)]]
        if float(before) != float(y0):
            assert abs(y[0, 0] - float(before)) > 0.01


def test_swiglu_against_torch_silu():
    """The SwiGLU product h = bf16(silu(gate) * up): silu against torch's
    own silu in fp64 (a library routine), silu on the gate half only, and
    one rounding to the nearest bf16."""
    from oracle.moe import swiglu_bf16
    rng = np.random.default_rng(17)
    g = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-4, 3, (64, 96)))
    u = rng.standard_normal((64, 96)) * np.exp(rng.uniform(-4, 3, (64, 96)))
    g[0, :6] = [0.0, -0.0, 40.0, -40.0, 1e-30, -750.0]
    ref = (torch.nn.functional.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    h = f32_from_bf16_bits(swiglu_bf16(g, u)).astype(np.float64)
    # h is a neighbour of the library value and the nearer one (up to fp64
    # rounding of the two computations): |h - ref| <= half a bf16 ulp of ref
    ulp = np.where(ref == 0, 0.0, 2.0 ** (np.floor(np.log2(np.abs(np.where(ref == 0, 1, ref)))) - 7))
    assert np.all(np.abs(h - ref) <= ulp / 2 * (1 + 1e-9) + 1e-300)
    # swapping the halves changes the result (silu is applied to the gate)
    h_sw = f32_from_bf16_bits(swiglu_bf16(u, g)).astype(np.float64)
    assert np.mean(h_sw != h) > 0.9
    # large positive gate: silu(g) -> g, so h -> bf16(g * u); large negative -> 0
    assert h[0, 2] == f32_from_bf16_bits(_bits([40.0 * u[0, 2]]))[0] or \
        abs(h[0, 2] - 40.0 * u[0, 2]) <= abs(40.0 * u[0, 2]) * 2.0 ** -8
    assert h[0, 5] == 0.0


def test_eq21_all_channels_error_bound(c1):
    """Eq. 21 with S = every channel: X~ - x = dX - dequant(Q(dX)) up to the bf16
    carrying of dX, so each element is within half an E2M1 grid step of dX's own
    block scale (at most 1 * sb * s_R) plus 2^-8 |dX|, and the whole residual
    shrinks well below the plain quantization error (a dropped or sign-flipped
    correction leaves it at 1x or 2x)."""
    d, A = c1
    x = f32_from_bf16_bits(d["x"]).astype(np.float64)
    deq = oracle.dequantize(A)
    Q = oracle.eq21_residual_quant(A)
    qd = oracle.dequantize(Q)
    xt = deq - qd
    dx = deq - x
    sbq = np.repeat(oracle.E4M3_VALUES[Q.scales.astype(np.int64)], 16, axis=1) * float(Q.tensor_scale)
    assert np.all(np.abs(xt - x) <= np.abs(dx) * 2.0 ** -8 + sbq)
    assert np.linalg.norm(xt - x) <= 0.2 * np.linalg.norm(dx)
    # and the GEMM form agrees with the corrected activation times dequant(W)
    W = oracle.nvfp4_quantize(d["w"])
    y = oracle.rac_gemm_eq21(d["x"], A, W, np.arange(x.shape[1]))
    ref = xt @ oracle.dequantize(W).T
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_qdq_identity_and_idempotence():
    """Weight QDQ (Eq. 12): (a) a tensor that is already E2M1 values times
    power-of-two block scales, each block holding a +-6, comes back unchanged at
    s_t = 1; (b) with a supplied power-of-two s_t and every block scale an E4M3
    normal, QDQ of the (bf16-exact) QDQ output is the QDQ output."""
    rng = np.random.default_rng(12)
    grid = np.array(PAGE_GRID)
    mag = rng.integers(0, 8, size=(24, 256))
    mag[:, ::16] = 7
    sign = np.where(rng.random((24, 256)) < 0.5, -1.0, 1.0)
    sc = 2.0 ** rng.integers(-4, 4, size=(24, 16)).repeat(16, axis=1)
    xv = grid[mag] * sign * sc
    xb = bf16_bits_from_f32(xv.astype(np.float32))
    assert np.array_equal(oracle.nvfp4_qdq(xb, tensor_scale=1.0), xv)
    w = rng.standard_normal((32, 512)) * 3.0
    wb = bf16_bits_from_f32(w.astype(np.float32))
    st = 2.0 ** -6
    q1 = oracle.nvfp4_qdq(wb, tensor_scale=st)
    assert np.all(oracle.nvfp4_quantize(wb, tensor_scale=st).scales >= 8)   # normal E4M3 scales
    q1b = bf16_bits_from_f32(q1.astype(np.float32))
    assert np.array_equal(f32_from_bf16_bits(q1b).astype(np.float64), q1)   # exact in bf16
    assert np.array_equal(oracle.nvfp4_qdq(q1b, tensor_scale=st), q1)
    # and it is the dequantized rollout quantization, element for element
    assert np.array_equal(q1, oracle.dequantize(oracle.nvfp4_quantize(wb, tensor_scale=st)))


# ---------------------------------------------------------------- MXFP4
def test_mxfp4_brute_force():
    rng = np.random.default_rng(5)
    xb = _random_bf16_blocks(rng, 4, 128, spread=20)
    q = oracle.mxfp4_quantize(xb)
    x = f32_from_bf16_bits(xb).astype(np.float64)
    grid = [Fraction(v) for v in PAGE_GRID]
    for i in range(4):
        for b in range(4):
            blk = x[i, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            if amax == 0:
                assert q.scales[i, b] == 0
                continue
            e = int(np.floor(np.log2(amax))) - 2
            assert Fraction(2) ** (e + 2) <= Fraction(float(amax)) < Fraction(2) ** (e + 3)
            assert q.scales[i, b] == e + 127
            sc = Fraction(2) ** e
            for j in range(32):
                mag = _nearest_even(abs(Fraction(float(blk[j]))) / sc, grid)
                assert q.mag[i, 32 * b + j] == mag
            assert q.mag[i, 32 * b + np.argmax(np.abs(blk))] in (6, 7)


# ---------------------------------------------------------------- MoE
def test_moe_route_and_sort_brute_force():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((40, 16)).astype(np.float32)
    logits[5, 3] = logits[5, 9]                           # a tie -> lower expert first
    idx, p = oracle.moe_route(logits, 4)
    for t in range(40):
        order = np.lexsort((np.arange(16), -logits[t].astype(np.float64)))[:4]
        assert idx[t].tolist() == order.tolist()
        sel = logits[t, order].astype(np.float64)
        np.testing.assert_allclose(p[t], np.exp(sel) / np.exp(logits[t].astype(np.float64)[order]).sum(),
                                   rtol=1e-14)
    assert abs(p.sum(axis=1) - 1).max() < 1e-14
    perm, off = oracle.moe_sort(idx, 16)
    assert sorted(perm.tolist()) == list(range(160))
    ex = idx.reshape(-1)[perm]
    assert np.all(np.diff(ex) >= 0)
    for e in range(16):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(idx.reshape(-1)[seg] == e) and np.all(np.diff(seg) > 0)


def test_moe_bf16_expert_rows():
    # one slot of weight 1: the layer output is the expert row itself, so with
    # bf16 expert rows it is out rounded once to nearest bf16 (ties to even);
    # everything before the combine is unchanged
    rng = np.random.default_rng(10)
    T, H, F = 16, 64, 32
    x = _bits(rng.standard_normal((T, H)).astype(np.float32))
    w13 = _bits((rng.standard_normal((1, 2 * F, H)) * 0.1).astype(np.float32))
    w2 = _bits((rng.standard_normal((1, H, F)) * 0.1).astype(np.float32))
    idx = np.zeros((T, 1), dtype=np.int32)
    ex = oracle.moe_layer(x, idx, np.ones((T, 1)), w13, w2, rac_k=8)
    rb = oracle.moe_layer(x, idx, np.ones((T, 1)), w13, w2, rac_k=8, out_bf16=True)
    np.testing.assert_array_equal(rb["out"], ex["out"])
    np.testing.assert_array_equal(ex["y"], ex["out"])
    # every value is a bf16 value, the nearest one to the exact row
    u = rb["y"].astype(np.float32).view(np.uint32)
    assert np.all(u & 0xFFFF == 0) and np.all(rb["y"].astype(np.float32) == rb["y"])
    up = (u + (1 << 16)).view(np.float32).astype(np.float64)
    dn = (u - (1 << 16)).view(np.float32).astype(np.float64)
    d = np.abs(rb["y"] - ex["out"])
    assert np.all(d <= np.abs(up - ex["out"])) and np.all(d <= np.abs(dn - ex["out"]))
    assert np.any(d > 0)


def test_moe_identical_experts_collapse_to_one():
    # with every expert identical, sum_s p_s out_s == out (weights sum to 1)
    rng = np.random.default_rng(9)
    T, H, F, E = 24, 64, 32, 6
    x = _bits(rng.standard_normal((T, H)).astype(np.float32))
    w13 = _bits((rng.standard_normal((2 * F, H)) * 0.1).astype(np.float32))
    w2 = _bits((rng.standard_normal((H, F)) * 0.1).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    idx, p = oracle.moe_route(logits, 3)
    many = oracle.moe_layer(x, idx, p, np.stack([w13] * E), np.stack([w2] * E), rac_k=8)
    one_idx = np.zeros((T, 1), dtype=np.int32)
    one = oracle.moe_layer(x, one_idx, np.ones((T, 1)), w13[None], w2[None], rac_k=8)
    # h of the many-expert run holds each token three times, so the second
    # quantization sees the same amax; its scores are three times as large
    # (same selection); the outputs agree to fp64 rounding
    np.testing.assert_allclose(many["y"], one["y"], rtol=1e-9, atol=1e-9 * np.abs(one["y"]).max())
    # and the quantized chain tracks the unquantized SwiGLU MLP
    from oracle.moe import dense_swiglu_reference
    ref = dense_swiglu_reference(x, w13, w2)
    assert np.linalg.norm(one["y"] - ref) / np.linalg.norm(ref) < 0.25
