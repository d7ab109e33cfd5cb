"""Number formats used by the oracle (test infrastructure only).

E2M1 magnitudes: QUADS page, section 2.2 paragraph "FP4" ({0,0.5,1,1.5,2,3,4,6}
per sign).  E4M3: section 2.2 paragraph "FP8" (four exponent bits, three
mantissa bits, largest magnitude 448); the variant with no infinities whose
all-ones code is NaN, so codes 0..126 are the non-negative finite values.
"""
from __future__ import annotations

import numpy as np

# code (3 magnitude bits) -> value; sign is the fourth bit of the nibble
E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_value(nibble: int) -> float:
    mag = E2M1_MAGNITUDES[nibble & 7]
    return -mag if nibble & 8 else mag


def e4m3_value(code: int) -> float:
    """Value of a non-negative E4M3 code 0..126 (exponent bias 7, subnormals at e=0)."""
    if not 0 <= code <= 126:
        raise ValueError("E4M3 code out of the finite non-negative range")
    e, m = code >> 3, code & 7
    if e == 0:
        return m * 2.0 ** -9
    return 2.0 ** (e - 7) * (1.0 + m / 8.0)


E4M3_VALUES = np.array([e4m3_value(c) for c in range(127)], dtype=np.float64)
E4M3_MAX = float(E4M3_VALUES[-1])  # 448


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_f32(a: np.ndarray) -> np.ndarray:
    """Round to nearest even fp32 (numpy's cast rounds to nearest even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even (finite values)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits with ONE rounding to nearest even.

    The value is split into the bf16 candidates below and above it and the
    nearer one is kept (ties to the even bit pattern); no intermediate fp32.
    """
    a = np.asarray(a, dtype=np.float64)
    # truncate to bf16 toward zero: build from fp32 truncation of the fp64 value
    f = a.astype(np.float32)
    # fp32 rounding may have gone past the value; step back toward zero if so
    f = np.where(np.abs(f.astype(np.float64)) > np.abs(a),
                 np.nextafter(f, np.float32(0)), f)
    t = (f.view(np.uint32) & np.uint32(0xFFFF0000))          # truncated bf16 (toward 0)
    lo = t.view(np.float32).astype(np.float64)               # |lo| <= |a|
    hi_bits = t + np.uint32(0x10000)                         # next bf16 away from zero
    hi = hi_bits.view(np.float32).astype(np.float64)
    d_lo = np.abs(a - lo)
    d_hi = np.abs(hi - a)
    even_lo = ((t >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~even_lo)
    out = np.where(take_hi, hi_bits, t) >> np.uint32(16)
    return out.astype(np.uint16)
