"""The C-ABI library loads, exports every entry point of include/q4rac.h and
rejects bad arguments on the host before any launch (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "q4rac.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


@pytest.fixture(scope="module")
def L():
    import fp4_w4a4_quantized_nvfp4_amd as m
    return m.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 19
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_binding_covers_header():
    import fp4_w4a4_quantized_nvfp4_amd as m
    assert set(_declared()) <= set(m._SIGS)


def _err(L):
    return L.q4_last_error().decode()


def test_shape_and_pointer_errors(L):
    fake = C.c_void_p(0x100000)          # aligned, never dereferenced on error paths
    odd = C.c_void_p(0x100004)
    # cols not a multiple of 16
    assert L.nvfp4_quantize(fake, 4, 24, None, fake, fake, fake, None, 0, None, fake, 1 << 30, None) == 2
    assert "cols % 16" in _err(L)
    # topk beyond cols
    assert L.nvfp4_quantize(fake, 4, 32, None, fake, fake, fake, None, 33, fake, fake, 1 << 30, None) == 1
    # channels beyond 2^24 (quantizers, weight QDQ), K beyond 2^24 (GEMMs, MoE H and F)
    big = (1 << 24) + 32
    assert L.nvfp4_quantize(fake, 4, big, None, fake, fake, fake, None, 0, None, fake, 1 << 40, None) == 2
    assert "2^24" in _err(L)
    assert L.nvfp4_quantize(fake, 4, 1 << 24, None, fake, fake, fake, None, 0, None, fake, 8, None) == 4
    assert L.mxfp4_quantize(fake, 4, big, fake, fake, None, 0, None, fake, 1 << 40, None) == 2
    assert L.nvfp4_quantize_noalloc(fake, 4, big, None, fake, fake, fake, None, 0, None, None) == 2
    assert L.nvfp4_qdq(fake, 4, big, None, fake, 0, fake, fake, 1 << 40, None) == 2
    assert L.w4a4_gemm(0, 8, 8, big, fake, fake, fake, fake, fake, fake, fake, 0, None) == 2
    assert L.moe_w4a4_grouped_gemm(0, fake, 4, big, fake, fake, 2, 4, 64, fake, fake, fake, fake,
                                   fake, fake, fake, fake, None, None, None, 0, fake, 1, fake,
                                   1 << 40, None, None) == 2
    # misaligned input
    assert L.nvfp4_quantize(odd, 4, 32, None, fake, fake, fake, None, 0, None, fake, 1 << 30, None) == 3
    # workspace too small
    assert L.nvfp4_quantize(fake, 4, 32, None, fake, fake, fake, None, 0, None, fake, 8, None) == 4
    # MXFP4 needs cols % 32
    assert L.mxfp4_quantize(fake, 4, 48, fake, fake, None, 0, None, fake, 1 << 30, None) == 2
    # GEMM: K % 32, bad format, missing tensor scale, MXFP4 with tensor scale
    assert L.w4a4_gemm(0, 8, 8, 48, fake, fake, fake, fake, fake, fake, fake, 0, None) == 2
    assert L.w4a4_gemm(7, 8, 8, 64, fake, fake, fake, fake, fake, fake, fake, 0, None) == 1
    assert L.w4a4_gemm(0, 8, 8, 64, fake, fake, None, fake, fake, fake, fake, 0, None) == 1
    assert L.w4a4_gemm(1, 8, 8, 64, fake, fake, fake, fake, fake, None, fake, 0, None) == 1
    assert L.w4a4_gemm(0, 8, 8, 64, fake, fake, fake, fake, fake, fake, fake, 5, None) == 1
    # RAC: k > K, missing workspace, misaligned status word
    assert L.rac_gemm(0, 8, 8, 64, fake, fake, fake, fake, fake, fake, fake, fake, fake, 65,
                      fake, 0, fake, 1 << 30, None, None) == 1
    assert L.rac_gemm(0, 8, 8, 64, fake, fake, fake, fake, fake, fake, fake, fake, fake, 16,
                      fake, 0, None, 0, None, None) == 4
    assert L.rac_gemm(0, 8, 8, 64, fake, fake, fake, fake, fake, fake, fake, fake, fake, 16,
                      fake, 0, fake, 1 << 30, C.c_void_p(0x100002), None) == 3
    assert "status" in _err(L)
    # Eq. 21 compensation: K % 32, k > K, missing workspace, misaligned scale output,
    # missing tensor scale (NVFP4 only)
    assert L.rac_gemm_eq21(8, 8, 48, fake, fake, fake, fake, fake, fake, fake, fake, 16, fake, 0,
                           None, fake, 1 << 30, None, None) == 2
    assert L.rac_gemm_eq21(8, 8, 64, fake, fake, fake, fake, fake, fake, fake, fake, 65, fake, 0,
                           None, fake, 1 << 30, None, None) == 1
    assert L.rac_gemm_eq21(8, 8, 64, fake, fake, fake, fake, fake, fake, fake, fake, 16, fake, 0,
                           None, None, 0, None, None) == 4
    assert L.rac_gemm_eq21(8, 8, 64, fake, fake, fake, fake, fake, fake, fake, fake, 16, fake, 0,
                           C.c_void_p(0x100002), fake, 1 << 30, None, None) == 3
    assert L.rac_gemm_eq21(8, 8, 64, fake, fake, fake, None, fake, fake, fake, fake, 16, fake, 0,
                           None, fake, 1 << 30, None, None) == 1
    assert "a_ts" in _err(L)
    # residual gather: ld_r < k
    assert L.q4_residual_gather(0, fake, 4, 64, fake, fake, fake, fake, 8, fake, 4, None, None) == 1
    # MoE: bad E, F % 32, topk > E
    assert L.q4_moe_route(fake, 4, 0, 1, fake, fake, None) == 2
    assert L.q4_moe_route(fake, 4, 8, 9, fake, fake, None) == 1
    assert L.moe_w4a4_grouped_gemm(0, fake, 4, 64, fake, fake, 2, 4, 48, fake, fake, fake, fake,
                                   fake, fake, fake, fake, None, None, None, 0, fake, 1, fake,
                                   1 << 30, None, None) == 2
    # MoE: a supplied h tensor scale is NVFP4 only
    assert L.moe_w4a4_grouped_gemm(1, fake, 4, 64, fake, fake, 2, 4, 64, fake, fake, None, fake,
                                   fake, None, fake, fake, None, None, fake, 0, fake, 1, fake,
                                   1 << 30, None, None) == 1
    assert "tensor scale" in _err(L)
    # MoE option flags: unknown bits; h fused into the W13 epilogue needs a supplied s_h
    assert L.moe_w4a4_grouped_gemm_ex(0, fake, 4, 64, fake, fake, 2, 4, 64, fake, fake, fake, fake,
                                      fake, fake, fake, fake, None, None, fake, 0, fake, 1, fake,
                                      1 << 30, None, 2, None) == 1
    assert "flags" in _err(L)
    assert L.moe_w4a4_grouped_gemm_ex(0, fake, 4, 64, fake, fake, 2, 4, 64, fake, fake, fake, fake,
                                      fake, fake, fake, fake, None, None, None, 0, fake, 1, fake,
                                      1 << 30, None, 1, None) == 1
    assert "h_tensor_scale" in _err(L)
    # scale records: K % 128, short output, format
    assert L.q4_scale_records(0, fake, 2, 64, 96, fake, 1 << 20, None) == 2
    assert L.q4_scale_records(0, fake, 2, 64, 256, fake, 100, None) == 4
    assert L.q4_scale_records(2, fake, 2, 64, 256, fake, 1 << 20, None) == 1
    assert L.q4_scale_records_size(0, 2, 300, 256) == 2 * 2 * 512 * (16 + 8)
    assert L.q4_scale_records_size(1, 2, 300, 256) == 2 * 2 * 512 * 4
    # sort: topk > 16, misaligned status
    assert L.q4_moe_sort(fake, 4, 32, 17, fake, fake, fake, 1 << 20, None, None) == 1
    assert L.q4_moe_sort(fake, 4, 32, 2, fake, fake, fake, 1 << 20, C.c_void_p(0x100002), None) == 3
    assert L.q4_moe_pack_w13(fake, 2, 40, 64, fake, None) == 2


def test_workspace_sizes(L):
    assert L.q4_quantize_workspace_size(16384, 7168, 0) >= 64 * 7168 * 8
    assert L.rac_gemm_workspace_size(8192, 14336, 4096, 128) >= (8192 + 14336) * 128 * 2
    # Eq. 21: R' and W' [rows][kp] bf16 first, then amax partials, s_R and the records
    assert L.rac_gemm_eq21_workspace_size(8192, 14336, 4096, 128) >= \
        L.rac_gemm_workspace_size(8192, 14336, 4096, 128) + 1024 * 4
    assert L.rac_gemm_eq21_workspace_size(64, 512, 512, 20) >= (64 + 512) * 32 * 2
    offs = (C.c_size_t * 16)()
    assert L.moe_workspace_layout(0, 8192, 128, 2048, 768, 8, 64, offs) == 0
    vals = list(offs)
    assert vals == sorted(vals) and len(set(vals)) == 16
    assert L.moe_workspace_size(0, 8192, 128, 2048, 768, 8, 64) > vals[-1]
