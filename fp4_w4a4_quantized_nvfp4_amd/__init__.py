"""Python binding of libq4rac (NVFP4 W4A4 GEMM with Residual Activation Compensation).

Argument marshalling only: every step runs in the HIP kernels of
``libq4rac.so``; PyTorch supplies device memory and the current stream.  The
library must have been built (``python -m fp4_w4a4_quantized_nvfp4_amd.build``);
importing the functions without it raises instead of falling back to anything.

Function names and argument meaning follow ``include/q4rac.h``.  bf16 tensors
may be passed as ``torch.bfloat16`` or as ``int16``/``uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

__all__ = [
    "Q4Error", "library_path", "lib",
    "nvfp4_quantize", "mxfp4_quantize", "nvfp4_qdq", "q4_select_channels", "q4_residual_gather",
    "w4a4_gemm", "rac_gemm", "rac_gemm_eq21", "q4_moe_route", "q4_moe_sort", "q4_transpose_bf16",
    "q4_moe_pack_w13", "q4_scale_records", "moe_w4a4_grouped_gemm", "moe_workspace_layout",
    "prepare_weight",
    "prepare_moe_weights", "NVFP4", "MXFP4", "OUT_F32", "OUT_BF16",
]

NVFP4, MXFP4 = 0, 1
OUT_F32, OUT_BF16 = 0, 1
MOE_WS_FIELDS = 16
MAX_TOPK = 1024

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libq4rac.so")


class Q4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"q4rac status {status}: {msg}")
        self.status = status


_LIB = None
_P = C.c_void_p
_I64, _I32, _SZ = C.c_int64, C.c_int32, C.c_size_t

_SIGS = {
    "q4_last_error": (C.c_char_p, []),
    "q4_version": (_I32, []),
    "q4_quantize_workspace_size": (_SZ, [_I64, _I64, _I32]),
    "nvfp4_quantize": (_I32, [_P, _I64, _I64, _P, _P, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "mxfp4_quantize": (_I32, [_P, _I64, _I64, _P, _P, _P, _I32, _P, _P, _SZ, _P]),
    "nvfp4_quantize_noalloc_max_scratch": (_SZ, []),
    "nvfp4_quantize_noalloc": (_I32, [_P, _I64, _I64, _P, _P, _P, _P, _P, _I32, _P, _P]),
    "nvfp4_qdq_workspace_size": (_SZ, [_I64, _I64]),
    "nvfp4_qdq": (_I32, [_P, _I64, _I64, _P, _P, _I32, _P, _P, _SZ, _P]),
    "q4_select_workspace_size": (_SZ, [_I64]),
    "q4_select_channels": (_I32, [_P, _I64, _I32, _P, _P, _SZ, _P]),
    "q4_residual_gather": (_I32, [_I32, _P, _I64, _I64, _P, _P, _P, _P, _I32, _P, _I64, _P, _P]),
    "w4a4_gemm": (_I32, [_I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _I32, _P]),
    "rac_gemm_workspace_size": (_SZ, [_I64, _I64, _I64, _I32]),
    "rac_gemm": (_I32, [_I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P,
                        _I32, _P, _SZ, _P, _P]),
    "rac_gemm_eq21_workspace_size": (_SZ, [_I64, _I64, _I64, _I32]),
    "rac_gemm_eq21": (_I32, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32,
                             _P, _P, _SZ, _P, _P]),
    "q4_moe_route": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P]),
    "q4_moe_sort_workspace_size": (_SZ, [_I64, _I32, _I32]),
    "q4_moe_sort": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _SZ, _P, _P]),
    "q4_transpose_bf16": (_I32, [_P, _I64, _I64, _I64, _P, _P]),
    "q4_moe_pack_w13": (_I32, [_P, _I32, _I32, _I32, _P, _P]),
    "q4_scale_records_size": (_SZ, [_I32, _I64, _I64, _I64]),
    "q4_scale_records": (_I32, [_I32, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "moe_workspace_size": (_SZ, [_I32, _I64, _I32, _I32, _I32, _I32, _I32]),
    "moe_workspace_layout": (_I32, [_I32, _I64, _I32, _I32, _I32, _I32, _I32, _P]),
    "moe_w4a4_grouped_gemm": (_I32, [_I32, _P, _I64, _I32, _P, _P, _I32, _I32, _I32, _P, _P, _P,
                                     _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _P, _SZ,
                                     _P, _P]),
    "moe_w4a4_grouped_gemm_ex": (_I32, [_I32, _P, _I64, _I32, _P, _P, _I32, _I32, _I32, _P, _P,
                                        _P, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P, _I32, _P,
                                        _SZ, _P, C.c_uint32, _P]),
}


def lib():
    """The loaded library (ctypes).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m fp4_w4a4_quantized_nvfp4_amd.build`")
        L = C.CDLL(path)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int):
    if status != 0:
        raise Q4Error(status, lib().q4_last_error().decode())


_BF16_TYPES = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t, dtype=None, shape=None, name="tensor"):
    """Device pointer of a contiguous tensor, after checking its dtype (a torch
    dtype or a tuple of them) and shape (None entries are free)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"q4rac: '{name}' must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"q4rac: '{name}' must be contiguous")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise TypeError(f"q4rac: '{name}' has dtype {t.dtype}, expected {dtype}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(d) != int(w)
                                        for d, w in zip(t.shape, shape)):
            raise ValueError(f"q4rac: '{name}' has shape {tuple(t.shape)}, expected "
                             f"{tuple('*' if w is None else w for w in shape)}")
    return t.data_ptr()


def _on(stream):
    """Run the body with `stream` current, so temporaries allocated there are
    stream-ordered with the kernels that use them (freed only after them)."""
    return torch.cuda.stream(stream) if stream is not None else _NullCtx()


class _NullCtx:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _bf16(t, name="x"):
    if t.dtype in _BF16_TYPES:
        return t
    raise TypeError(f"q4rac: '{name}' must be bf16 (torch.bfloat16 or 16-bit bit patterns), "
                    f"got {t.dtype}")


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


def _status(status):
    return _ptr(status, torch.int32, (1,), "status")


def _qshape(q, rows, K, name):
    """Check a quantized operand dict against rows x K."""
    blk = 16 if q["fmt"] == NVFP4 else 32
    _ptr(q["codes"], torch.uint8, (rows, K // 2), name + " codes")
    _ptr(q["scales"], torch.uint8, (rows, K // blk), name + " scales")
    if q["fmt"] == NVFP4:
        _ptr(q["tensor_scale"], torch.float32, (None,), name + " tensor_scale")


# ------------------------------------------------------------------ quantizer
def _quantize(fmt, x, tensor_scale_in=None, topk=0, want_scores=True, stream=None):
    with _on(stream):
        return _quantize_body(fmt, x, tensor_scale_in, topk, want_scores)


def _quantize_body(fmt, x, tensor_scale_in, topk, want_scores, stream=None):
    x = _bf16(x)
    if x.dim() != 2:
        raise ValueError("q4rac: x must be 2-D [rows, cols]")
    rows, cols = x.shape
    _ptr(tensor_scale_in, torch.float32, (1,), "tensor_scale_in")
    dev = x.device
    L = lib()
    blk = 16 if fmt == NVFP4 else 32
    codes = _empty((rows, cols // 2), torch.uint8, dev)
    scales = _empty((rows, max(cols // blk, 0)), torch.uint8, dev)
    ts = _empty((1,), torch.float32, dev) if fmt == NVFP4 else None
    score = _empty((cols,), torch.float64, dev) if want_scores else None
    idx = _empty((topk,), torch.int32, dev) if topk > 0 else None
    wsb = L.q4_quantize_workspace_size(rows, cols, fmt)
    ws = _empty((max(wsb, 1),), torch.uint8, dev)
    if fmt == NVFP4:
        st = L.nvfp4_quantize(_ptr(x), rows, cols, _ptr(tensor_scale_in), _ptr(codes), _ptr(scales),
                              _ptr(ts), _ptr(score), topk, _ptr(idx), _ptr(ws), wsb, _stream(stream))
    else:
        st = L.mxfp4_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(score), topk,
                              _ptr(idx), _ptr(ws), wsb, _stream(stream))
    _check(st)
    return {"fmt": fmt, "codes": codes, "scales": scales, "tensor_scale": ts,
            "chan_score": score, "chan_idx": idx}


def nvfp4_quantize(x, tensor_scale_in=None, topk=0, want_scores=True, stream=None):
    """NVFP4 quantization of bf16 x [rows, cols] -> dict of device tensors."""
    return _quantize(NVFP4, x, tensor_scale_in, topk, want_scores, stream)


def mxfp4_quantize(x, topk=0, want_scores=True, stream=None):
    return _quantize(MXFP4, x, None, topk, want_scores, stream)


def nvfp4_qdq(x, tensor_scale_in=None, out_dtype=OUT_F32, stream=None, want_scale=False):
    """Weight fake quantization: the values c sb s_t of nvfp4_quantize(x), fp32 or
    bf16; with want_scale also the tensor scale used."""
    with _on(stream):
        return _nvfp4_qdq_body(x, tensor_scale_in, out_dtype, want_scale)


def _nvfp4_qdq_body(x, tensor_scale_in, out_dtype, want_scale, stream=None):
    x = _bf16(x)
    _ptr(tensor_scale_in, torch.float32, (1,), "tensor_scale_in")
    rows, cols = x.shape
    L = lib()
    y = _empty((rows, cols), torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, x.device)
    ts = _empty((1,), torch.float32, x.device)
    wsb = L.nvfp4_qdq_workspace_size(rows, cols)
    ws = _empty((max(wsb, 1),), torch.uint8, x.device)
    _check(L.nvfp4_qdq(_ptr(x), rows, cols, _ptr(tensor_scale_in), _ptr(y), out_dtype, _ptr(ts),
                       _ptr(ws), wsb, _stream(stream)))
    return (y, ts) if want_scale else y


def q4_select_channels(chan_score, topk, stream=None):
    with _on(stream):
        cols = chan_score.shape[0]
        _ptr(chan_score, torch.float64, (cols,), "chan_score")
        idx = _empty((topk,), torch.int32, chan_score.device)
        _check(lib().q4_select_channels(_ptr(chan_score), cols, topk, _ptr(idx) if topk else None,
                                        None, 0, _stream(stream)))
        return idx


def q4_residual_gather(x, q, chan_idx, ld_r=None, stream=None, status=None):
    with _on(stream):
        x = _bf16(x)
        rows, cols = x.shape
        _qshape(q, rows, cols, "q")
        k = 0 if chan_idx is None else int(chan_idx.shape[0])
        ld_r = max(k, 1) if ld_r is None else ld_r
        R = _empty((rows, ld_r), torch.int16, x.device)
        _check(lib().q4_residual_gather(q["fmt"], _ptr(x), rows, cols, _ptr(q["codes"]),
                                        _ptr(q["scales"]), _ptr(q["tensor_scale"]),
                                        _ptr(chan_idx, torch.int32, (k,), "chan_idx") if k else None,
                                        k, _ptr(R), ld_r, _status(status), _stream(stream)))
        return R


# ------------------------------------------------------------------ GEMM
def w4a4_gemm(A, W, out_dtype=OUT_F32, stream=None):
    """Y = W4A4(A, W) for quantized dicts A [M, K] and W [N, K]."""
    with _on(stream):
        return _w4a4_gemm_body(A, W, out_dtype, stream)


def _w4a4_gemm_body(A, W, out_dtype, stream):
    M = A["codes"].shape[0]
    N = W["codes"].shape[0]
    K = A["codes"].shape[1] * 2
    if A["fmt"] != W["fmt"]:
        raise ValueError("q4rac: A and W must share a format")
    _qshape(A, M, K, "A")
    _qshape(W, N, K, "W")
    Y = _empty((M, N), torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
               A["codes"].device)
    _check(lib().w4a4_gemm(A["fmt"], M, N, K, _ptr(A["codes"]), _ptr(A["scales"]),
                           _ptr(A["tensor_scale"]), _ptr(W["codes"]), _ptr(W["scales"]),
                           _ptr(W["tensor_scale"]), _ptr(Y), out_dtype, _stream(stream)))
    return Y


def _out_check(Y, M, N, out_dtype):
    _ptr(Y, torch.float32 if out_dtype == OUT_F32 else _BF16_TYPES, (M, N), "Y")


def rac_gemm(x, A, W, w_hi_t, chan_set, out_dtype=OUT_F32, stream=None, Y=None, workspace=None,
             status=None):
    """Y = W4A4(A, W) + residual(x on chan_set) @ W_hi[:, chan_set]^T.  ``status``
    (optional int32 [1] device tensor) receives 0, or 1 for an invalid channel set."""
    with _on(stream):
        x = _bf16(x)
        M, K = x.shape
        N = W["codes"].shape[0]
        if A["fmt"] != W["fmt"]:
            raise ValueError("q4rac: A and W must share a format")
        _qshape(A, M, K, "A")
        _qshape(W, N, K, "W")
        k = 0 if chan_set is None else int(chan_set.shape[0])
        L = lib()
        if Y is None:
            Y = _empty((M, N), torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, x.device)
        _out_check(Y, M, N, out_dtype)
        wsb = L.rac_gemm_workspace_size(M, N, K, k)
        if workspace is None or workspace.numel() < wsb:
            workspace = _empty((max(wsb, 1),), torch.uint8, x.device)
        _check(L.rac_gemm(A["fmt"], M, N, K, _ptr(x), _ptr(A["codes"]), _ptr(A["scales"]),
                          _ptr(A["tensor_scale"]), _ptr(W["codes"]), _ptr(W["scales"]),
                          _ptr(W["tensor_scale"]),
                          _ptr(_bf16(w_hi_t, "w_hi_t"), None, (K, N), "w_hi_t") if k else None,
                          _ptr(chan_set, torch.int32, (k,), "chan_set") if k else None, k,
                          _ptr(Y), out_dtype, _ptr(workspace, torch.uint8), wsb,
                          _status(status), _stream(stream)))
        return Y


def rac_gemm_eq21(x, A, W, chan_set, out_dtype=OUT_F32, stream=None, Y=None, workspace=None,
                  resid_tensor_scale=None, status=None):
    """Page-literal compensation: Y = (Q(x) - M_S * Q(Q(x) - x)) @ Q(W)^T for NVFP4
    operands A (of x) and W; resid_tensor_scale (fp32 [1], optional) receives the
    residual's tensor scale, status (int32 [1], optional) 0 or 1 (invalid set)."""
    with _on(stream):
        x = _bf16(x)
        M, K = x.shape
        N = W["codes"].shape[0]
        if A["fmt"] != NVFP4 or W["fmt"] != NVFP4:
            raise ValueError("q4rac: rac_gemm_eq21 takes NVFP4 operands")
        _qshape(A, M, K, "A")
        _qshape(W, N, K, "W")
        k = 0 if chan_set is None else int(chan_set.shape[0])
        L = lib()
        if Y is None:
            Y = _empty((M, N), torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, x.device)
        _out_check(Y, M, N, out_dtype)
        wsb = L.rac_gemm_eq21_workspace_size(M, N, K, k)
        if workspace is None or workspace.numel() < wsb:
            workspace = _empty((max(wsb, 1),), torch.uint8, x.device)
        _check(L.rac_gemm_eq21(M, N, K, _ptr(x), _ptr(A["codes"]), _ptr(A["scales"]),
                               _ptr(A["tensor_scale"]), _ptr(W["codes"]), _ptr(W["scales"]),
                               _ptr(W["tensor_scale"]),
                               _ptr(chan_set, torch.int32, (k,), "chan_set") if k else None, k,
                               _ptr(Y), out_dtype,
                               _ptr(resid_tensor_scale, torch.float32, (1,), "resid_tensor_scale"),
                               _ptr(workspace, torch.uint8), wsb, _status(status),
                               _stream(stream)))
        return Y


def q4_transpose_bf16(x, stream=None):
    """rows x cols -> cols x rows; batch x rows x cols -> cols x batch x rows
    (channel-major, the matrices interleaved)."""
    x = _bf16(x)
    batch = x.shape[0] if x.dim() == 3 else 1
    rows, cols = x.shape[-2], x.shape[-1]
    out = _empty((cols, batch, rows) if x.dim() == 3 else (cols, rows), x.dtype, x.device)
    _check(lib().q4_transpose_bf16(_ptr(x), batch, rows, cols, _ptr(out), _stream(stream)))
    return out


def prepare_weight(w, fmt=NVFP4, stream=None):
    """Offline weight preparation: quantize W [N, K] and build W_hi^T [K, N]."""
    q = _quantize(fmt, w, None, 0, False, stream)
    q["w_hi_t"] = q4_transpose_bf16(w, stream)
    return q


# ------------------------------------------------------------------ MoE
def q4_moe_route(logits, topk, stream=None):
    with _on(stream):
        T, E = logits.shape
        _ptr(logits, torch.float32, (T, E), "logits")
        idx = _empty((T, topk), torch.int32, logits.device)
        w = _empty((T, topk), torch.float32, logits.device)
        _check(lib().q4_moe_route(_ptr(logits), T, E, topk, _ptr(idx), _ptr(w), _stream(stream)))
        return idx, w


def q4_moe_sort(topk_idx, E, stream=None, status=None):
    with _on(stream):
        T, k = topk_idx.shape
        _ptr(topk_idx, torch.int32, (T, k), "topk_idx")
        L = lib()
        perm = _empty((T * k,), torch.int32, topk_idx.device)
        offsets = _empty((E + 1,), torch.int32, topk_idx.device)
        wsb = L.q4_moe_sort_workspace_size(T, E, k)
        ws = _empty((max(wsb, 1),), torch.uint8, topk_idx.device)
        _check(L.q4_moe_sort(_ptr(topk_idx), T, E, k, _ptr(perm), _ptr(offsets), _ptr(ws), wsb,
                             _status(status), _stream(stream)))
        return perm, offsets


def q4_moe_pack_w13(w13, stream=None):
    """[E, 2F, H] logical (gate rows, then up rows) -> packed 32-row groups."""
    w13 = _bf16(w13)
    E, F2, H = w13.shape
    out = torch.empty_like(w13)
    _check(lib().q4_moe_pack_w13(_ptr(w13), E, F2 // 2, H, _ptr(out), _stream(stream)))
    return out


def _quantize_stacked(fmt, w, stream=None):
    """Quantize each expert [E, R, C] with its own tensor scale; stacked outputs."""
    E, R, Cc = w.shape
    blk = 16 if fmt == NVFP4 else 32
    dev = w.device
    codes = _empty((E, R, Cc // 2), torch.uint8, dev)
    scales = _empty((E, R, Cc // blk), torch.uint8, dev)
    ts = _empty((E,), torch.float32, dev) if fmt == NVFP4 else None
    L = lib()
    wsb = L.q4_quantize_workspace_size(R, Cc, fmt)
    ws = _empty((max(wsb, 1),), torch.uint8, dev)
    s = _stream(stream)
    for e in range(E):
        if fmt == NVFP4:
            st = L.nvfp4_quantize(_ptr(w[e]), R, Cc, None, _ptr(codes[e]), _ptr(scales[e]),
                                  ts[e:e + 1].data_ptr(), None, 0, None, _ptr(ws), wsb, s)
        else:
            st = L.mxfp4_quantize(_ptr(w[e]), R, Cc, _ptr(codes[e]), _ptr(scales[e]), None, 0,
                                  None, _ptr(ws), wsb, s)
        _check(st)
    return {"fmt": fmt, "codes": codes, "scales": scales, "tensor_scale": ts}


def q4_scale_records(scales, K, fmt=NVFP4, stream=None):
    """Scale records of stacked scales uint8 [batch, rows, K/16] (NVFP4) or
    [batch, rows, K/32] (MXFP4), K % 128 == 0, as one flat uint8 buffer:
    NVFP4 [batch, K/128, rows_pad, 16] fp16 records followed by [batch, K/128,
    rows_pad, 8] raw E4M3 records; MXFP4 [batch, K/128, rows_pad, 4] E8M0
    bytes; rows_pad = rows rounded up to 256."""
    with _on(stream):
        if scales.dim() != 3:
            raise ValueError("q4rac: scales must be [batch, rows, K/16 or K/32]")
        b, rows = scales.shape[0], scales.shape[1]
        blk = 16 if fmt == NVFP4 else 32
        _ptr(scales, torch.uint8, (b, rows, K // blk), "scales")
        L = lib()
        n = L.q4_scale_records_size(fmt, b, rows, K)
        if n == 0:
            raise Q4Error(f"q4_scale_records: K = {K} is not a positive multiple of 128")
        out = _empty((n,), torch.uint8, scales.device)
        _check(L.q4_scale_records(fmt, _ptr(scales), b, rows, K, _ptr(out), n, _stream(stream)))
        return out


def prepare_moe_weights(w13, w2, fmt=NVFP4, with_hi=True, stream=None, scale_records=True):
    """Offline expert preparation from logical bf16 w13 [E, 2F, H] and w2 [E, H, F].
    With H and F multiples of 128: also the weights' scale records
    ("scale_records"), which the grouped GEMMs read instead of the raw scales
    (same results)."""
    w13p = q4_moe_pack_w13(w13, stream)
    out = {"fmt": fmt, "w13": _quantize_stacked(fmt, w13p, stream),
           "w2": _quantize_stacked(fmt, _bf16(w2), stream),
           "E": w13.shape[0], "F": w13.shape[1] // 2, "H": w13.shape[2]}
    H, F = out["H"], out["F"]
    if scale_records and H % 128 == 0 and F % 128 == 0:
        out["w13"]["scale_records"] = q4_scale_records(out["w13"]["scales"], H, fmt, stream)
        out["w2"]["scale_records"] = q4_scale_records(out["w2"]["scales"], F, fmt, stream)
    if with_hi:
        out["w13_hi_t"] = q4_transpose_bf16(w13p, stream)
        out["w2_hi_t"] = q4_transpose_bf16(_bf16(w2), stream)
    return out


def moe_workspace_layout(fmt, T, E, H, F, topk, rac_k):
    L = lib()
    offs = (C.c_size_t * MOE_WS_FIELDS)()
    _check(L.moe_workspace_layout(fmt, T, E, H, F, topk, rac_k, offs))
    return list(offs), L.moe_workspace_size(fmt, T, E, H, F, topk, rac_k)


MOE_FUSE_H_QUANT = 1


def moe_w4a4_grouped_gemm(tokens, topk_idx, topk_w, experts, rac_k, out_dtype=OUT_BF16,
                          workspace=None, stream=None, Y=None, status=None, h_tensor_scale=None,
                          fuse_h=False):
    """Token-sorted grouped W4A4+RAC SwiGLU expert layer; returns (Y, workspace).
    ``status`` (optional int32 [1]) receives 0, or 1 for an expert index
    outside [0, E).  ``h_tensor_scale`` (optional fp32 [1], NVFP4) supplies
    h's tensor scale, so h's quantization needs no amax pass.  ``fuse_h``
    (with ``h_tensor_scale``): on prefill shapes, quantize h inside the W13
    GEMM's epilogue instead of in a separate pass (moe_w4a4_grouped_gemm_ex,
    Q4_MOE_FUSE_H_QUANT)."""
    with _on(stream):
        tokens = _bf16(tokens, "tokens")
        T, H = tokens.shape
        topk = topk_idx.shape[1]
        fmt = experts["fmt"]
        E, F = experts["E"], experts["F"]
        if experts["H"] != H:
            raise ValueError(f"q4rac: tokens have {H} channels, the experts {experts['H']}")
        _ptr(topk_idx, torch.int32, (T, topk), "topk_idx")
        _ptr(topk_w, torch.float32, (T, topk), "topk_w")
        w13, w2 = experts["w13"], experts["w2"]
        blk = 16 if fmt == NVFP4 else 32
        _ptr(w13["codes"], torch.uint8, (E, 2 * F, H // 2), "w13 codes")
        _ptr(w13["scales"], torch.uint8, (E, 2 * F, H // blk), "w13 scales")
        _ptr(w2["codes"], torch.uint8, (E, H, F // 2), "w2 codes")
        _ptr(w2["scales"], torch.uint8, (E, H, F // blk), "w2 scales")
        if fmt == NVFP4:
            _ptr(w13["tensor_scale"], torch.float32, (E,), "w13 tensor_scale")
            _ptr(w2["tensor_scale"], torch.float32, (E,), "w2 tensor_scale")
        rec13 = rec2 = None
        L = lib()
        if w13.get("scale_records") is not None:
            rec13 = _ptr(w13["scale_records"], torch.uint8,
                         (L.q4_scale_records_size(fmt, E, 2 * F, H),), "w13 scale_records")
        if w2.get("scale_records") is not None:
            rec2 = _ptr(w2["scale_records"], torch.uint8,
                        (L.q4_scale_records_size(fmt, E, H, F),), "w2 scale_records")
        wsb = L.moe_workspace_size(fmt, T, E, H, F, topk, rac_k)
        if workspace is None or workspace.numel() < wsb:
            workspace = _empty((max(wsb, 1),), torch.uint8, tokens.device)
        if Y is None:
            Y = _empty((T, H), torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
                       tokens.device)
        _out_check(Y, T, H, out_dtype)
        _check(L.moe_w4a4_grouped_gemm_ex(
            fmt, _ptr(tokens), T, H, _ptr(topk_idx), _ptr(topk_w), topk, E, F,
            _ptr(w13["codes"]), _ptr(w13["scales"]), _ptr(w13["tensor_scale"]),
            _ptr(w2["codes"]), _ptr(w2["scales"]), _ptr(w2["tensor_scale"]),
            _ptr(experts.get("w13_hi_t"), _BF16_TYPES, (H, E, 2 * F), "w13_hi_t") if rac_k else None,
            _ptr(experts.get("w2_hi_t"), _BF16_TYPES, (F, E, H), "w2_hi_t") if rac_k else None,
            rec13, rec2, _ptr(h_tensor_scale, torch.float32, (1,), "h_tensor_scale"),
            rac_k, _ptr(Y), out_dtype, _ptr(workspace, torch.uint8), wsb,
            _status(status), MOE_FUSE_H_QUANT if fuse_h else 0,
            _stream(stream)))
        return Y, workspace
