"""NVFP4 / MXFP4 quantization, residual, channel scores and top-k (test oracle).

TEST INFRASTRUCTURE ONLY -- never used by the product path.

Definitions (QUADS page, arXiv 2607.15810):

* Section 2.2 "FP4": an NVFP4 tensor is E2M1 codes, one E4M3 block scale per
  sixteen consecutive elements and a per-tensor FP32 scale.  The page gives no
  formula for either scale; the plain reading used here is

  - tensor scale  s_t = RN32(amax / (6 * 448)), the smallest scale that keeps
    the largest block scale inside E4M3's maximum (section 2.2 "FP8" gives
    448, the E2M1 grid's top is 6); s_t = 1 for an all-zero tensor;
  - block scale   sb  = E4M3 nearest to amax_b / (6 * s_t), ties to the even
    code, saturating at 448 (the sixteen elements run along the channel axis,
    the GEMM reduction axis, so the scale factors out of a dot product);
  - code          the E2M1 magnitude nearest to |x| / (sb * s_t), ties to the
    even code, saturating at 6; the sign bit is the sign bit of x (so -0 and
    tiny negatives give the code 0x8); sb == 0 gives zero magnitudes.

  Every "nearest" is decided on exact reals by comparing x (or amax_b) with the
  exact product (midpoint * scale), which fp64 holds exactly because every
  factor has few significant bits (bf16: 8, E4M3: 4, fp32 scale: 24,
  midpoints: at most 5 -> at most 31 bits).
* Section 3.3, Eq. 20: the quantization error.  This oracle keeps the
  residual r = x - dequant(quant(x)) = -(Eq. 20) rounded once to fp32.
* Section 3.3, Eq. 23: s_j = ||r[:, j]||_2 over the current token batch.  The
  oracle's score is s_j^2 = sum_i r_ij^2 as the fp64 value nearest to the
  exact real sum (ties to even): each r_ij is an fp32 value m 2^e (integer m <
  2^24), so the sum is accumulated exactly in integers and rounded once.  No
  summation order enters the definition; any fp64 summation of the same terms
  lies within (rows - 1) 2^-53 relative of it.
* Section 3.3, Eq. 24: the selected set S is the k channels with the largest
  score (ties -> smaller channel index), listed in ascending channel order.
  k is an absolute count.
* MXFP4 (page thelatestinai.com/papers/2607.15810, Rollout-ResQ abstract
  "open-standard MXFP4"; the power-of-two scale of the MXFP4 error-split
  abstract on the same page): 32-element blocks, scale 2^e with
  e = floor(log2 amax_b) - 2 (2 = largest E2M1 exponent), clamped to
  [-127, 127], stored as the E8M0 byte e + 127; amax_b == 0 -> byte 0 and zero
  magnitudes.  No tensor scale.
"""
from __future__ import annotations

import dataclasses

import numpy as np

from .formats import E2M1_MAGNITUDES, E4M3_VALUES, bf16_bits_to_f64, f32_to_bf16_bits

_E2M1 = np.array(E2M1_MAGNITUDES, dtype=np.float64)
# midpoints between consecutive E2M1 magnitudes and whether a tie goes up
# (ties go to the even code: the upper neighbour's code c+1 is even)
_E2M1_MIDS = (_E2M1[:-1] + _E2M1[1:]) / 2.0          # 0.25 .. 5
_E2M1_TIE_UP = np.array([((c + 1) % 2 == 0) for c in range(7)])
_E4M3_MIDS = (E4M3_VALUES[:-1] + E4M3_VALUES[1:]) / 2.0
_E4M3_TIE_UP = np.array([((c + 1) % 2 == 0) for c in range(126)])


@dataclasses.dataclass
class QuantResult:
    fmt: str                    # "nvfp4" | "mxfp4"
    codes: np.ndarray           # uint8 [M, K/2]; element 2i low nibble, 2i+1 high nibble
    scales: np.ndarray          # uint8 [M, K/16] E4M3 codes (nvfp4) | [M, K/32] E8M0 (mxfp4)
    tensor_scale: np.float32    # nvfp4 s_t (fp32); mxfp4: 1.0
    resid: np.ndarray           # float32 [M, K]: RN32(x - dequant)
    mag: np.ndarray             # uint8 [M, K] magnitude codes 0..7 (unpacked, for tests)
    sign: np.ndarray            # bool [M, K]


def nvfp4_tensor_scale(x64: np.ndarray) -> np.float32:
    amax = float(np.max(np.abs(x64))) if x64.size else 0.0
    if amax == 0.0:
        return np.float32(1.0)
    # amax (bf16) / 2688 rounded once to fp32: the fp64 quotient is not an fp32
    # midpoint (2688 = 21 * 2^7 and amax has 8 significant bits), so rounding
    # the fp64 quotient to fp32 equals rounding the exact quotient.
    q = amax / 2688.0
    return np.float32(q)


def _round_to_table(num: np.ndarray, thresholds: np.ndarray, tie_up: np.ndarray) -> np.ndarray:
    """Index of the nearest table entry given the exact midpoint thresholds.

    ``thresholds`` broadcast against ``num`` on a trailing axis; entry m is the
    exact value of the midpoint between table entries m and m+1 (already
    multiplied by the scale).  Passing a threshold strictly, or meeting it
    exactly when the tie goes up, moves one entry up; saturates at the top.
    """
    n = num[..., None]
    up = (n > thresholds) | ((n == thresholds) & tie_up)
    return up.sum(axis=-1).astype(np.uint8)


def _rn32_difference(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """RN32(a - b) for fp64 a, b, with a single rounding of the exact difference."""
    d = a - b
    # exact error of the fp64 subtraction (Knuth's TwoSum)
    bv = d - a
    err = (a - (d - bv)) + (-b - bv)
    f = d.astype(np.float32)
    # d is an fp32 midpoint only if d - f == +-half an fp32 ulp; then the
    # rounding direction of the exact value is the sign of err.
    diff = d - f.astype(np.float64)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(-np.inf))
    half_up = (up.astype(np.float64) - f.astype(np.float64)) / 2.0
    half_dn = (f.astype(np.float64) - dn.astype(np.float64)) / 2.0
    mid_above = (diff > 0) & (diff == half_up)     # d halfway between f and up
    mid_below = (diff < 0) & (-diff == half_dn)    # d halfway between dn and f
    fix = np.where(mid_above & (err > 0), up, f)
    fix = np.where(mid_above & (err < 0), f, fix)
    fix = np.where(mid_below & (err < 0), dn, fix)
    fix = np.where(mid_below & (err > 0), f, fix)
    return fix.astype(np.float32)


def _pack(mag: np.ndarray, sign: np.ndarray) -> np.ndarray:
    nib = (mag.astype(np.uint8) | (sign.astype(np.uint8) << 3))
    lo = nib[:, 0::2]
    hi = nib[:, 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def _nvfp4_rows(x: np.ndarray, st: float):
    M, K = x.shape
    blk = np.abs(x).reshape(M, K // 16, 16)
    amax_b = blk.max(axis=2)
    # E4M3 block scale: nearest to amax_b / (6 s_t); threshold = (6 s_t) * mid, exact
    sb_code = _round_to_table(amax_b, (6.0 * st) * _E4M3_MIDS, _E4M3_TIE_UP)
    sb = E4M3_VALUES[sb_code]                                   # [M, K/16]
    # E2M1 code: nearest to |x| / (sb s_t); threshold = (mid * sb) * s_t, exact
    thr = (_E2M1_MIDS[None, None, :] * sb[..., None]) * st     # [M, K/16, 7]
    mag = _round_to_table(blk, thr[:, :, None, :], _E2M1_TIE_UP)  # [M, K/16, 16]
    mag = np.where((sb == 0.0)[..., None], np.uint8(0), mag).reshape(M, K)
    sign = np.signbit(x)
    deq = np.where(sign, -1.0, 1.0) * (_E2M1[mag] * np.repeat(sb, 16, axis=1)) * st
    resid = _rn32_difference(x, deq)
    return _pack(mag, sign), sb_code.astype(np.uint8), resid, mag.astype(np.uint8), sign


_ROW_CHUNK = 512


def _by_rows(fn, x: np.ndarray, *args):
    """Apply a row-independent step to row chunks (bounded memory); same result."""
    parts = [fn(x[i:i + _ROW_CHUNK], *args) for i in range(0, max(1, x.shape[0]), _ROW_CHUNK)]
    return [np.concatenate([p[j] for p in parts], axis=0) for j in range(len(parts[0]))]


def nvfp4_quantize(x_bits: np.ndarray, tensor_scale: float | None = None) -> QuantResult:
    """Quantize bf16 bits [M, K] (K % 16 == 0) to NVFP4 with the residual.

    ``tensor_scale`` given -> used as s_t (a caller-supplied FP32 scale);
    otherwise s_t comes from the tensor's absolute maximum.
    """
    x = bf16_bits_to_f64(x_bits)
    M, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    s_t = nvfp4_tensor_scale(x) if tensor_scale is None else np.float32(tensor_scale)
    codes, scales, resid, mag, sign = _by_rows(_nvfp4_rows, x, float(s_t))
    return QuantResult("nvfp4", codes, scales, s_t, resid, mag, sign)


def _mxfp4_rows(x: np.ndarray):
    M, K = x.shape
    blk = np.abs(x).reshape(M, K // 32, 32)
    amax_b = blk.max(axis=2)
    # floor(log2 amax) from frexp: amax = m * 2^p with m in [0.5, 1) -> p - 1
    _, p = np.frexp(amax_b)
    ex = np.clip(p.astype(np.int64) - 1 - 2, -127, 127)
    code = np.where(amax_b == 0.0, 0, ex + 127).astype(np.uint8)
    scale = np.where(amax_b == 0.0, 0.0, np.ldexp(1.0, ex))
    thr = _E2M1_MIDS[None, None, :] * scale[..., None]         # exact (power of two)
    mag = _round_to_table(blk, thr[:, :, None, :], _E2M1_TIE_UP)
    mag = np.where((amax_b == 0.0)[..., None], np.uint8(0), mag).reshape(M, K)
    sign = np.signbit(x)
    deq = np.where(sign, -1.0, 1.0) * _E2M1[mag] * np.repeat(scale, 32, axis=1)
    resid = _rn32_difference(x, deq)
    return _pack(mag, sign), code, resid, mag.astype(np.uint8), sign


def mxfp4_quantize(x_bits: np.ndarray) -> QuantResult:
    """Quantize bf16 bits [M, K] (K % 32 == 0) to MXFP4 with the residual."""
    x = bf16_bits_to_f64(x_bits)
    if x.shape[1] % 32:
        raise ValueError("K must be a multiple of 32")
    codes, scales, resid, mag, sign = _by_rows(_mxfp4_rows, x)
    return QuantResult("mxfp4", codes, scales, np.float32(1.0), resid, mag, sign)


def _unpack(codes: np.ndarray):
    lo = codes & 0xF
    hi = codes >> 4
    nib = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    nib[:, 0::2] = lo
    nib[:, 1::2] = hi
    return nib


def block_values(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """Per-element c * block_scale in fp64 (no tensor scale); exact."""
    nib = _unpack(codes)
    val = _E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    if fmt == "nvfp4":
        sb = E4M3_VALUES[scales.astype(np.int64)]
        return val * np.repeat(sb, 16, axis=1)
    if fmt == "mxfp4":
        e = scales.astype(np.int64) - 127
        sc = np.ldexp(1.0, e)
        return val * np.repeat(sc, 32, axis=1)
    raise ValueError(fmt)


def dequantize(q: QuantResult) -> np.ndarray:
    return block_values(q.codes, q.scales, q.fmt) * float(q.tensor_scale)


def nvfp4_qdq(x_bits: np.ndarray, tensor_scale=None) -> np.ndarray:
    """Trainer-side weight fake quantization (QUADS section 3.2, Eq. 12): the
    trainer quantizes and dequantizes its weight with the rollout quantizer's
    own block layout and rounding, so the values are c sb s_t of this module's
    NVFP4 quantization, exact in fp64 (at most 6 + 24 significant bits).
    Eq. 13's straight-through backward is the identity on the gradient."""
    return dequantize(nvfp4_quantize(x_bits, tensor_scale=tensor_scale))


def channel_scores(resid: np.ndarray) -> np.ndarray:
    """s_j^2 = sum_i r_ij^2 per channel j (Eq. 23 squared): the fp64 value
    nearest to the exact sum.

    Every fp32 residual is m * 2^e with an integer 0 <= m < 2^24 and
    e = max(E, 1) - 150 (E the biased exponent field), so r^2 = m^2 * 2^(2e)
    with m^2 < 2^48.  The squares are binned by e per channel; within a bin
    the integer m^2 values are summed exactly (split in two 24-bit halves so
    each half's running sum stays an integer below 2^53 for fewer than 2^29
    rows); the bins are then combined as one Python integer and converted to
    fp64 with a single correctly rounded conversion.
    """
    r = np.ascontiguousarray(resid, dtype=np.float32)
    M, K = r.shape
    NE = 254                                   # e = -149 .. 104
    hi = np.zeros(K * NE, dtype=np.float64)
    lo = np.zeros(K * NE, dtype=np.float64)
    col = np.arange(K, dtype=np.int64)[None, :] * NE
    for i0 in range(0, M, 1024):
        bits = r[i0:i0 + 1024].view(np.uint32)
        ef = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64)
        mant = (bits & np.uint32(0x7FFFFF)).astype(np.int64)
        m = np.where(ef > 0, mant | 0x800000, mant)
        sq = m * m                             # < 2^48, exact in int64
        b = (col + (np.maximum(ef, 1) - 1)).ravel()
        hi += np.bincount(b, weights=(sq >> 24).ravel().astype(np.float64), minlength=K * NE)
        lo += np.bincount(b, weights=(sq & 0xFFFFFF).ravel().astype(np.float64), minlength=K * NE)
    hi = hi.reshape(K, NE)
    lo = lo.reshape(K, NE)
    out = np.zeros(K, dtype=np.float64)
    for j in range(K):
        nz = np.nonzero((hi[j] != 0) | (lo[j] != 0))[0]
        if nz.size == 0:
            continue
        base = int(nz[0])
        total = 0
        for t in nz:                            # bin t holds multiples of 2^(2(t - 149))
            c = (int(hi[j, t]) << 24) + int(lo[j, t])
            total += c << (2 * (int(t) - base))
        # one rounding: Python's int -> float conversion and int / int true
        # division are both correctly rounded (nearest, ties to even)
        sh = 2 * (base - 149)
        out[j] = float(total << sh) if sh >= 0 else total / (1 << -sh)
    return out


def select_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """k largest scores, ties -> smaller index; returned in ascending index order."""
    K = scores.shape[0]
    if not 0 <= k <= K:
        raise ValueError("k out of range")
    order = sorted(range(K), key=lambda j: (-scores[j], j))
    return np.array(sorted(order[:k]), dtype=np.int32)


def residual_gather(resid: np.ndarray, S: np.ndarray) -> np.ndarray:
    """R[i, t] = bf16(r[i, S_t]) (round to nearest even), as bf16 bits [M, k]."""
    return f32_to_bf16_bits(resid[:, np.asarray(S, dtype=np.int64)])
