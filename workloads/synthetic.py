"""Seeded synthetic workloads (shapes and distributions only, no method arithmetic).

The QUADS page (arXiv 2607.15810, section 3.3, Figure 4a) shows activation
quantization residuals concentrated in a few persistent hidden channels that
form vertical bands across tokens.  The generators reproduce that structure
with outlier channels that are fixed for every token of a tensor.  The model
and datasets of the page are not available, so these tensors stand in for
them; the shapes and distributions follow the five workloads below.

Random streams: numpy ``PCG64`` seeded with
``SeedSequence(20261202, spawn_key=(workload_index, tensor_id, [expert]))``.
fp32 samples are rounded to bf16 with round-to-nearest-even on the bit
pattern; bf16 tensors are carried as ``uint16`` arrays of bit patterns.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

ROOT_SEED = 20261202

# tensor ids inside one workload's seed space
_T_X, _T_W, _T_OUTLIER_CH, _T_OUTLIER_MUL, _T_LOGITS, _T_W13, _T_W2 = range(7)


@dataclasses.dataclass(frozen=True)
class Workload:
    index: int
    name: str
    rows: int                 # tokens (M, or T for MoE)
    cols: int                 # hidden size K (= H for MoE)
    dist: str                 # "normal" or "t3"
    n_outlier: int            # number of fixed outlier channels
    outlier_mul: tuple        # (lo, hi) multiplier range; lo == hi -> fixed
    n_out: int = 0            # dense: W rows (N); 0 -> no weight
    topk_channels: int = 0    # k of the channel selection
    out_dtype: str = "f32"    # dense output type
    experts: int = 0          # MoE: experts
    ffn: int = 0              # MoE: expert FFN width F
    route_topk: int = 0       # MoE: experts per token
    weight_std: float = 0.02

    @property
    def is_moe(self) -> bool:
        return self.experts > 0


WORKLOADS = {
    "dense_64x512": Workload(0, "dense_64x512", 64, 512, "normal", 4, (50.0, 50.0),
                             n_out=512, topk_channels=16, out_dtype="f32"),
    "quant_16384x7168": Workload(1, "quant_16384x7168", 16384, 7168, "t3", 72, (20.0, 100.0),
                                 topk_channels=64),
    "dense_8192x14336x4096": Workload(2, "dense_8192x14336x4096", 8192, 4096, "normal", 20,
                                      (50.0, 50.0), n_out=14336, topk_channels=128,
                                      out_dtype="bf16"),
    "moe_prefill_8192": Workload(3, "moe_prefill_8192", 8192, 2048, "normal", 10, (50.0, 50.0),
                                 topk_channels=64, out_dtype="bf16", experts=128, ffn=768,
                                 route_topk=8),
    "moe_decode_256": Workload(4, "moe_decode_256", 256, 4096, "t3", 41, (20.0, 100.0),
                               topk_channels=64, out_dtype="bf16", experts=128, ffn=1536,
                               route_topk=8),
    # selection-ratio sweep (k = 12.5 .. 75 % of the channels, the page's range):
    # the dense prefill distribution on a 1024-channel projection
    "sweep_8192x4096x1024": Workload(5, "sweep_8192x4096x1024", 8192, 1024, "normal", 5,
                                     (50.0, 50.0), n_out=4096, topk_channels=128,
                                     out_dtype="f32"),
}


def rng_for(workload_index: int, tensor_id: int, *extra: int) -> np.random.Generator:
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=(workload_index, tensor_id) + tuple(extra))
    return np.random.Generator(np.random.PCG64(ss))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _outliers(wl: Workload, cols: int):
    r = rng_for(wl.index, _T_OUTLIER_CH)
    ch = np.sort(r.choice(cols, size=wl.n_outlier, replace=False)).astype(np.int64)
    lo, hi = wl.outlier_mul
    if lo == hi:
        mul = np.full(wl.n_outlier, lo, dtype=np.float32)
    else:
        mul = rng_for(wl.index, _T_OUTLIER_MUL).uniform(lo, hi, size=wl.n_outlier).astype(np.float32)
    return ch, mul


def make_activations(wl: Workload, rows: int | None = None) -> np.ndarray:
    """bf16 bits [rows x cols]; base N(0,1) or Student-t(3), outlier channels scaled."""
    rows = wl.rows if rows is None else rows
    r = rng_for(wl.index, _T_X)
    if wl.dist == "normal":
        x = r.standard_normal((rows, wl.cols), dtype=np.float32)
    elif wl.dist == "t3":
        x = r.standard_t(3, size=(rows, wl.cols)).astype(np.float32)
    else:
        raise ValueError(wl.dist)
    ch, mul = _outliers(wl, wl.cols)
    x[:, ch] *= mul[None, :]
    return bf16_bits_from_f32(x)


def make_weight(wl: Workload) -> np.ndarray:
    """Dense weight, bf16 bits [N out x K in], N(0, std)."""
    r = rng_for(wl.index, _T_W)
    w = r.standard_normal((wl.n_out, wl.cols), dtype=np.float32) * np.float32(wl.weight_std)
    return bf16_bits_from_f32(w)


def make_logits(wl: Workload) -> np.ndarray:
    """Router logits fp32 [T x E], N(0,1)."""
    return rng_for(wl.index, _T_LOGITS).standard_normal((wl.rows, wl.experts), dtype=np.float32)


def _expert_weight(wl: Workload, tid: int, e: int, shape) -> np.ndarray:
    r = rng_for(wl.index, tid, e)
    w = r.standard_normal(shape, dtype=np.float32) * np.float32(wl.weight_std)
    return bf16_bits_from_f32(w)


def make_moe_weights(wl: Workload, experts: list | None = None, threads: int | None = None):
    """Expert weights in logical layout, bf16 bits.

    w13: [E, 2F, H]: rows 0..F-1 are the gate projection, rows F..2F-1 the up
    projection.  w2: [E, H, F].  ``experts`` restricts generation to a subset
    (any expert can be regenerated on its own).
    """
    E, H, F = wl.experts, wl.cols, wl.ffn
    ids = list(range(E)) if experts is None else list(experts)
    w13 = np.empty((len(ids), 2 * F, H), dtype=np.uint16)
    w2 = np.empty((len(ids), H, F), dtype=np.uint16)

    def one(i_e):
        i, e = i_e
        w13[i] = _expert_weight(wl, _T_W13, e, (2 * F, H))
        w2[i] = _expert_weight(wl, _T_W2, e, (H, F))

    n = threads or min(8, len(os.sched_getaffinity(0)))
    with _cf.ThreadPoolExecutor(max_workers=max(1, n)) as ex:
        list(ex.map(one, enumerate(ids)))
    return w13, w2


def make_inputs(name: str, rows: int | None = None, with_weights: bool = True) -> dict:
    wl = WORKLOADS[name]
    out = {"workload": wl, "x": make_activations(wl, rows)}
    if wl.n_out and with_weights:
        out["w"] = make_weight(wl)
    if wl.is_moe:
        out["logits"] = make_logits(wl) if rows is None else make_logits(wl)[:rows]
        if with_weights:
            out["w13"], out["w2"] = make_moe_weights(wl)
    return out
