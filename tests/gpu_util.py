"""Helpers for the GPU parity tests: moving bit patterns to and from the device
and the GEMM tolerance of the parity criterion."""
import sys

import numpy as np
import torch


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy array (bf16 bit patterns as uint16 are sent as int16) -> cuda tensor."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int16:
        return t.numpy().view(np.uint16)
    return t.numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    """max_ij |y - ref| / max(|ref_ij|, rms(ref))  (elementwise relative, rms floor)."""
    ref = ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 1.0
    den = np.maximum(np.abs(ref), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(y.astype(np.float64) - ref) / den)) if ref.size else 0.0


GEMM_TOL = 1e-3


def check_bf16_output(y_bits: np.ndarray, ref: np.ndarray, tol: float = GEMM_TOL):
    """bf16 output: within tol (rms floor) plus one bf16 ulp of the reference."""
    y = bf16_to_f64(y_bits)
    ref = ref.astype(np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 1.0
    den = np.maximum(np.abs(ref), rms)
    ulp = np.abs(ref) * 2.0 ** -8
    ok = np.abs(y - ref) <= tol * den + ulp
    assert ok.all(), f"bf16 output off at {np.argwhere(~ok)[:5].tolist()}"


_CACHE = {}


def cached(key, fn):
    """fn() computed once per test process (large oracle results and inputs
    that several tests share)."""
    if key not in _CACHE:
        _CACHE[key] = fn()
    return _CACHE[key]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
