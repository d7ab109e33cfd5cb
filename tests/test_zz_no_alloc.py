"""The no-allocation quantize entry point (static device scratch) against the
workspace entry point, through the C ABI: identical codes, scales, tensor
scale, channel scores and selection on two calls in a row, the second with a
smaller input; a shape beyond the static maximum is refused before launch."""
import ctypes as C

import numpy as np
import pytest
import torch

from workloads import bf16_bits_from_f32
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def _x(rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols)).astype(np.float32)
    x[:, rng.choice(cols, 5, replace=False)] *= 60.0
    return dev(bf16_bits_from_f32(x))


def _outputs(rows, cols, topk):
    d = torch.device("cuda")
    return {"codes": torch.empty((rows, cols // 2), dtype=torch.uint8, device=d),
            "scales": torch.empty((rows, cols // 16), dtype=torch.uint8, device=d),
            "ts": torch.empty((1,), dtype=torch.float32, device=d),
            "score": torch.empty((cols,), dtype=torch.float64, device=d),
            "idx": torch.empty((max(topk, 1),), dtype=torch.int32, device=d)}


def _run(L, x, topk, noalloc, ts_in=None):
    rows, cols = x.shape
    o = _outputs(rows, cols, topk)
    sp = torch.cuda.current_stream().cuda_stream
    tin = None if ts_in is None else ts_in.data_ptr()
    args = (x.data_ptr(), rows, cols, tin, o["codes"].data_ptr(), o["scales"].data_ptr(),
            o["ts"].data_ptr(), o["score"].data_ptr(), topk, o["idx"].data_ptr())
    if noalloc:
        st = L.nvfp4_quantize_noalloc(*args, sp)
    else:
        wsb = L.q4_quantize_workspace_size(rows, cols, 0)
        ws = torch.empty((wsb,), dtype=torch.uint8, device="cuda")
        st = L.nvfp4_quantize(*args, ws.data_ptr(), wsb, sp)
        o["ws"] = ws
    assert st == 0, L.q4_last_error().decode()
    return o


def _same(a, b, topk):
    for key in ("codes", "scales", "ts", "score"):
        assert torch.equal(a[key], b[key]), key
    if topk:
        assert torch.equal(a["idx"][:topk], b["idx"][:topk])


def test_noalloc_matches_workspace_entry_point():
    import fp4_w4a4_quantized_nvfp4_amd as m
    L = m.lib()
    assert L.nvfp4_quantize_noalloc_max_scratch() == 24 << 20
    # first a large call, then a smaller one: the second must not see the
    # first call's partial sums
    for rows, cols, topk, seed in ((4096, 7168, 64, 1), (300, 1024, 40, 2), (16384, 7168, 64, 3)):
        say(f"noalloc quantize {rows}x{cols} topk={topk}")
        x = _x(rows, cols, seed)
        ref = _run(L, x, topk, noalloc=False)
        got = _run(L, x, topk, noalloc=True)
        torch.cuda.synchronize()
        _same(got, ref, topk)
    # a supplied tensor scale
    x = _x(512, 2048, 4)
    tin = torch.tensor([0.03], dtype=torch.float32, device="cuda")
    ref = _run(L, x, 16, noalloc=False, ts_in=tin)
    got = _run(L, x, 16, noalloc=True, ts_in=tin)
    torch.cuda.synchronize()
    _same(got, ref, 16)


def test_noalloc_refuses_oversized_shape():
    import fp4_w4a4_quantized_nvfp4_amd as m
    L = m.lib()
    fake = C.c_void_p(0x100000)
    # 262144 rows x 8192 channels: 1024 row groups of fp64 partial sums, 64 MiB
    st = L.nvfp4_quantize_noalloc(fake, 262144, 8192, None, fake, fake, fake, None, 0, None, None)
    assert st == 4 and "static" in L.q4_last_error().decode()
    assert L.nvfp4_quantize_noalloc(fake, 4, 24, None, fake, fake, fake, None, 0, None, None) == 2
