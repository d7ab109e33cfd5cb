"""GPU parity of the NVFP4 / MXFP4 quantizer, channel scores, selection and
residual gather against the CPU oracle (bit-exact)."""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits_from_f32, make_inputs
from tests.gpu_util import dev, host, say
from tests.parity import check_scores, check_selection

pytestmark = pytest.mark.gpu


def q4():
    import fp4_w4a4_quantized_nvfp4_amd as m
    return m


def _bits(a):
    return bf16_bits_from_f32(np.asarray(a, dtype=np.float32))


def _t3(rows, cols, seed, n_out=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    x[:, rng.choice(cols, n_out, replace=False)] *= rng.uniform(20, 100, n_out).astype(np.float32)
    return _bits(x)


def _compare_nvfp4(xb, topk, ts=None, mx=False):
    say(f"quantize parity {'mx' if mx else 'nv'} shape={xb.shape} topk={topk} ts={ts}")
    m = q4()
    x = dev(xb)
    if mx:
        g = m.mxfp4_quantize(x, topk=topk)
        o = oracle.mxfp4_quantize(xb)
    else:
        tin = None if ts is None else torch.tensor([ts], dtype=torch.float32, device="cuda")
        g = m.nvfp4_quantize(x, tensor_scale_in=tin, topk=topk)
        o = oracle.nvfp4_quantize(xb, tensor_scale=ts)
    torch.cuda.synchronize()
    if not mx:
        assert host(g["tensor_scale"])[0].view(np.uint32) == np.float32(o.tensor_scale).view(np.uint32)
    gc, gs = host(g["codes"]), host(g["scales"])
    bad = np.argwhere(gc != o.codes)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()}: gpu {gc[tuple(bad[0])]:#x} oracle {o.codes[tuple(bad[0])]:#x}"
    bad = np.argwhere(gs != o.scales)
    assert bad.size == 0, f"scales differ at {bad[:5].tolist()}"
    # scores: the oracle's exact sums, within the fp64 summation bound; the
    # selection: exact top-k of the GPU's own scores, equal to the oracle's
    # exact top-k outside a near-tie band
    sc = oracle.channel_scores(o.resid)
    gsc = host(g["chan_score"])
    rel = check_scores(gsc, sc, xb.shape[0])
    say(f"  scores: max rel diff {rel:.2e}")
    if topk:
        S = check_selection(host(g["chan_idx"]), sc, topk, xb.shape[0], gpu_scores=gsc)
        R = host(m.q4_residual_gather(x, g, g["chan_idx"], ld_r=topk + 5))
        Ro = oracle.residual_gather(o.resid, S)
        assert np.array_equal(R[:, :topk], Ro)
        assert np.all(R[:, topk:] == 0)
    return g, o


def test_small_dense_workload():
    d = make_inputs("dense_64x512")
    _compare_nvfp4(d["x"], 16)
    _compare_nvfp4(d["w"], 0)


@pytest.mark.parametrize("rows,cols,seed", [(333, 592, 1), (1, 16, 2), (64, 512, 3), (130, 2048, 4),
                                            (65, 1040, 5)])
def test_ragged_t3(rows, cols, seed):
    _compare_nvfp4(_t3(rows, cols, seed, n_out=min(5, cols // 16)), min(40, cols))


def test_supplied_tensor_scale():
    xb = _t3(200, 512, 9)
    _compare_nvfp4(xb, 32, ts=0.37)
    _compare_nvfp4(xb, 8, ts=1.0e-3)      # heavy block-scale saturation


def test_exact_ties_and_signed_zeros():
    # every bf16 in [-6, 6] against a unit block scale: hits every E2M1 midpoint
    vals = (np.arange(0, 0x40C1, dtype=np.uint32) << 16).view(np.float32)
    vals = np.concatenate([vals, -vals])
    n = (len(vals) + 14) // 15
    blocks = np.full((n, 16), 6.0, dtype=np.float32)
    flat = blocks[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(n, 15)
    cols = 512
    total = blocks.size
    rows = (total + cols - 1) // cols
    x = np.zeros(rows * cols, dtype=np.float32)
    x[:total] = blocks.reshape(-1)
    xb = _bits(x.reshape(rows, cols))
    _compare_nvfp4(xb, 16, ts=1.0)
    # E4M3 midpoints: amax = 6 * midpoint with s_t = 1
    e4 = oracle.E4M3_VALUES
    mids = (e4[:-1] + e4[1:]) / 2 * 6
    y = np.zeros((1, 16 * len(mids)), dtype=np.float32)
    y[0, ::16] = mids.astype(np.float32)
    _compare_nvfp4(_bits(y), 4, ts=1.0)


def _tie_direction_amax():
    """bf16 amax mantissas whose s_t = RN32(a / 2688) is rounded down, up and
    exact (the three in-call tie rules of the kernel)."""
    from fractions import Fraction
    from tests.test_tie_rule import _rn32
    picks = {}
    for am in range(128):
        a = 1 + Fraction(am, 128)
        st = _rn32(a / 2688)
        d = "up" if st < a / 2688 else ("down" if st > a / 2688 else "even")
        picks.setdefault(d, am)
    return picks


@pytest.mark.parametrize("direction", ["up", "down", "even"])
def test_in_call_tie_directions(direction):
    # Student-t data whose amax is a chosen bf16 value, so that s_t = RN32(amax
    # / 2688) is rounded down, rounded up or exact; structural ties occur at
    # every such amax
    am = _tie_direction_amax()[direction]
    target = np.float32((1 + am / 128) * 64.0)
    rng = np.random.default_rng(40 + am)
    x = rng.standard_t(3, size=(256, 1024)).astype(np.float32)
    x *= 0.9 * target / np.abs(x).max()
    x[7, 100] = -target
    xb = _bits(x)
    assert np.float32(oracle.nvfp4_quantize(xb).tensor_scale) == np.float32(float(target) / 2688.0)
    _compare_nvfp4(xb, 32)


@pytest.mark.parametrize("direction", ["up", "down", "even"])
def test_supplied_derived_scale_tie_directions(direction):
    # a supplied s_t = RN32(a / 2688) for a bf16 a other than this tensor's
    # amax (a scale kept from an earlier step): the same tie structure
    am = _tie_direction_amax()[direction]
    a2 = np.float32((1 + am / 128) * 128.0)
    st = float(np.float32(float(a2) / 2688.0))
    rng = np.random.default_rng(60 + am)
    x = rng.standard_t(3, size=(256, 1024)).astype(np.float32)
    x *= 100.0 / np.abs(x).max()
    _compare_nvfp4(_bits(x), 32, ts=st)


def test_zero_tiny_and_huge():
    z = np.zeros((70, 64), dtype=np.uint16)
    z[3, 5] = 0x8000                     # -0.0
    _compare_nvfp4(z, 3)
    rng = np.random.default_rng(4)
    tiny = _bits((rng.standard_normal((80, 256)) * 1e-36).astype(np.float32))
    _compare_nvfp4(tiny, 7)
    mixed = rng.standard_normal((90, 256)).astype(np.float32)
    mixed[::3] *= 1e-30
    mixed[1::7] *= 1e30
    _compare_nvfp4(_bits(mixed), 9)
    huge = _bits((rng.standard_normal((10, 128)) * 1e37).astype(np.float32))
    _compare_nvfp4(huge, 2)


def test_empty_rows():
    m = q4()
    x = torch.empty((0, 64), dtype=torch.int16, device="cuda")
    g = m.nvfp4_quantize(x, topk=5)
    torch.cuda.synchronize()
    assert host(g["tensor_scale"])[0] == 1.0
    assert np.all(host(g["chan_score"]) == 0)
    assert host(g["chan_idx"]).tolist() == [0, 1, 2, 3, 4]


@pytest.mark.parametrize("rows,cols,seed", [(64, 512, 11), (301, 736, 12), (5, 32, 13)])
def test_mxfp4(rows, cols, seed):
    _compare_nvfp4(_t3(rows, cols, seed, n_out=3), min(24, cols), mx=True)


def test_mxfp4_extremes():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((40, 256)).astype(np.float32)
    x[::4] *= 1e-38
    x[2::4] *= 1e36
    x[5] = 0
    _compare_nvfp4(_bits(x), 10, mx=True)


def test_mxfp4_zero_blocks_wide_layout():
    """MXFP4 on the 16-channels-per-lane layout with a ragged last strip (768
    columns: a quarter of the lanes hold no channel) and all-zero 32-blocks,
    signed zeros and bf16 subnormals in the data: an all-zero block takes the
    smallest E8M0 scale and signed-zero codes, bit-exact."""
    rng = np.random.default_rng(22)
    rows, cols = 65536, 768
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    blk = x.reshape(rows, cols // 32, 32)
    blk[rng.random((rows, cols // 32)) < 0.05] = 0.0
    blk[rng.random((rows, cols // 32)) < 0.01] = -0.0
    tiny = rng.random((rows, cols // 32)) < 0.01
    blk[tiny] = rng.standard_normal((int(tiny.sum()), 32)).astype(np.float32) * 1e-39
    _compare_nvfp4(_bits(x), 64, mx=True)


def test_deterministic():
    m = q4()
    x = dev(_t3(500, 1024, 31))
    a = m.nvfp4_quantize(x, topk=50)
    b = m.nvfp4_quantize(x, topk=50)
    torch.cuda.synchronize()
    for key in ("codes", "scales", "tensor_scale", "chan_score", "chan_idx"):
        assert torch.equal(a[key], b[key])


def test_quantizer_workload_full_size():
    """16384 x 7168 Student-t(3) activations with 1% outlier channels: every
    code, scale and score bit-exact, the top-64 selection identical."""
    d = make_inputs("quant_16384x7168")
    g, o = _compare_nvfp4(d["x"], 64)
    say("full-size quantizer parity ok; s_t", float(o.tensor_scale))


@pytest.mark.parametrize("cols", [1, 100, 1024, 1500, 4096, 7168, 8192, 10000, 16384, 20000])
def test_select_channels_ties(cols):
    """Top-k over crafted fp64 scores: long runs of equal values, zeros, values
    that share their top bytes, k at the edges and inside a tie run; every
    register-resident size class and the general kernel."""
    m = q4()
    rng = np.random.default_rng(cols)
    base = rng.choice([0.0, 1.0, 2.5, 1e-300, 3.0e5], size=cols)
    base = base * (1.0 + rng.integers(0, 3, size=cols) * 2.0 ** -50)   # ties in the low bits only
    base[rng.random(cols) < 0.3] = 7.0                                   # a long run of ties
    for k in sorted({1, min(cols, 2), min(cols, 64), min(cols, 1000), min(cols // 2 or 1, 1024),
                     min(cols, 1024)}):
        got = m.q4_select_channels(dev(base), k)
        ref = oracle.select_topk(base, k)
        assert np.array_equal(host(got), ref), (cols, k)
