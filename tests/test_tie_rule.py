"""The tie rule the GPU quantizer uses for an in-call tensor scale (no GPU).

With s_t = RN32(a / 2688) for a bf16 tensor amax a, the quantize kernel
decides every element whose x / (s s_t) falls within 2^-20 of an E2M1
rounding midpoint by one rule for the whole launch: up in magnitude when s_t
was rounded down, down when it was rounded up, to the even code when the
quotient was exact.  That rests on two facts, checked here with exact
rational arithmetic over every bf16 amax mantissa, every E4M3 block scale
and every midpoint, for the bf16 x nearest each midpoint:

* an element that close to a midpoint is an exact tie, x * 2688 == mid * a * s;
* for an exact tie, |x| - mid * s * s_t has the sign of a / 2688 - s_t.

The window checked (2^-18) is wider than the kernel's bracket (2^-20 plus
its reciprocal error).  The amax exponent only scales s_t by a power of two,
so a in [1, 2) covers every normal amax.
"""
import struct
from fractions import Fraction as F

import numpy as np

MIDPOINTS = [F(1, 4), F(3, 4), F(5, 4), F(7, 4), F(5, 2), F(7, 2), F(5)]


def _rn32(q: F) -> F:
    """Correctly rounded fp32 value of a positive rational in the normal range."""
    f32 = np.float32(float(q))
    cands = [np.nextafter(f32, np.float32(0)), f32, np.nextafter(f32, np.float32(np.inf))]

    def key(v):
        bits = int(np.frombuffer(np.float32(v).tobytes(), np.uint32)[0])
        return (abs(F(float(v)) - q), bits & 1)

    return F(float(min(cands, key=key)))


def _bf16_near(t: F):
    """The bf16 values around t (positive)."""
    b = struct.unpack("<I", struct.pack("<f", float(t)))[0] >> 16
    out = []
    for d in (-1, 0, 1, 2):
        v = struct.unpack("<f", struct.pack("<I", ((b + d) & 0xFFFF) << 16))[0]
        if v > 0:
            out.append(F(v))
    return out


def _e4m3_values():
    vals = []
    for c in range(1, 127):
        e, m = c >> 3, c & 7
        vals.append(F(m, 8) / 64 if e == 0 else (1 + F(m, 8)) * F(2) ** (e - 7))
    return vals


def test_near_midpoint_elements_are_exact_ties_with_one_direction():
    scales = _e4m3_values()
    near = 0
    for am in range(128):
        a = 1 + F(am, 128)
        st = _rn32(a / 2688)
        rule = "up" if st < a / 2688 else ("down" if st > a / 2688 else "even")
        for s in scales:
            S = s * st
            for mid in MIDPOINTS:
                for x in _bf16_near(mid * S):
                    if abs(x / S - mid) > mid / 2 ** 18:
                        continue
                    near += 1
                    assert x * 2688 == mid * a * s, (a, s, x, mid)
                    t = mid * s * st
                    got = "up" if x > t else ("down" if x < t else "even")
                    assert got == rule, (a, s, x, mid, got, rule)
    # the structure is common: thousands of (amax, scale, midpoint) ties
    assert near > 10000


def test_each_direction_occurs():
    """All three outcomes of s_t = RN32(a / 2688) occur among bf16 amax values
    (the even case needs a mantissa divisible by 21, e.g. 1 + 40/128 = 168/128)."""
    seen = set()
    for am in range(128):
        a = 1 + F(am, 128)
        st = _rn32(a / 2688)
        seen.add("up" if st < a / 2688 else ("down" if st > a / 2688 else "even"))
    assert seen == {"up", "down", "even"}
