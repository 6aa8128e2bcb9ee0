"""The C-ABI library: it loads, exports every symbol the header declares, and
rejects invalid arguments on the host before touching a GPU (these calls
never reach a launch, so they run without a GPU)."""

import ctypes
import os
import re

import pytest

import precision_gemm_nvfp4_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4_resq.h")

FAKE = ctypes.c_void_p(0x1000)          # aligned, never dereferenced: validation fails first


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(P.LIB_PATH):
        pytest.skip("library not built")
    return P.load()


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert len(declared) == 27      # 18 operations, 7 workspace queries, version, last error
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(P.exported_symbols()) == declared
    assert lib.nvfp4_version() >= 100


def test_workspace_sizes(lib):
    assert lib.nvfp4_quantize_workspace_size(16384, 4096) >= 256 * 4   # one partial per amax workgroup, at most 256
    n = lib.resq_select_and_requant_workspace_size(2048, 131072, 128, 64)
    assert n >= (131072 // 128 + 128) * 2048 * 4 + 131072 * 64 * 4
    assert lib.qdq_weights_workspace_size(512, 3072, 4096) >= 512 * 4


def err(lib):
    return lib.nvfp4_last_error().decode()


def test_quantize_noalloc_validation(lib):
    """The no-allocation quantize validates like nvfp4_quantize, before it
    looks up its device scratch (so these run without a GPU)."""
    f = lib.nvfp4_quantize_noalloc
    assert f(None, 0, 4, 32, 32, None, FAKE, FAKE, None, None, None) == -1
    assert "x is NULL" in err(lib) and "noalloc" in err(lib)
    assert f(FAKE, 0, 4, 30, 32, None, FAKE, FAKE, None, None, None) == -1
    assert "multiple of 16" in err(lib)
    assert f(FAKE, 0, 4, 32, 20, None, FAKE, FAKE, None, None, None) == -1
    assert f(FAKE, 7, 4, 32, 32, None, FAKE, FAKE, None, None, None) == -2
    assert f(FAKE, 0, 4, 32, 32, None, None, FAKE, None, None, None) == -1
    assert f(FAKE, 0, 4, 32, 32, None, ctypes.c_void_p(0x1004), FAKE, None, None, None) == -1
    assert "aligned" in err(lib)


def test_quantize_validation(lib):
    assert lib.nvfp4_quantize(None, 0, 4, 32, 32, None, FAKE, FAKE, None, None, FAKE, 4096, None) == -1
    assert "x is NULL" in err(lib)
    assert lib.nvfp4_quantize(FAKE, 0, 4, 30, 32, None, FAKE, FAKE, None, None, FAKE, 4096, None) == -1
    assert "multiple of 16" in err(lib)
    assert lib.nvfp4_quantize(FAKE, 0, 4, 32, 20, None, FAKE, FAKE, None, None, FAKE, 4096, None) == -1
    assert lib.nvfp4_quantize(FAKE, 7, 4, 32, 32, None, FAKE, FAKE, None, None, FAKE, 4096, None) == -2
    assert lib.nvfp4_quantize(FAKE, 0, 4, 32, 36, None, FAKE, FAKE, None, None, FAKE, 4096, None) == -1
    assert "16 bytes" in err(lib)
    assert lib.nvfp4_quantize(FAKE, 0, 4, 32, 32, None, FAKE, FAKE, None, None, None, 0, None) == -3
    assert lib.nvfp4_quantize(ctypes.c_void_p(0x1004), 0, 4, 32, 32, None, FAKE, FAKE, None, None,
                              FAKE, 4096, None) == -1
    assert "aligned" in err(lib)


def test_resq_validation(lib):
    f = lib.resq_select_and_requant
    base = dict(x=FAKE, dtype=0, x_rows=256, K=512, ldx=512, row_index=None, codes=FAKE, scales=FAKE,
                g=FAKE, unit_offsets=FAKE, U=2, rows_total=256, k=64, tile_partials=None,
                sel=FAKE, rc=FAKE, rs=FAKE, rg=FAKE, ws=FAKE, ws_bytes=1 << 30, stream=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())

    assert call(k=24) == -1 and "k=24" in err(lib)
    assert call(k=1024) == -1
    assert call(K=32768, ldx=32768) == -2
    assert call(unit_offsets=None) == -1
    assert call(tile_partials=FAKE, row_index=FAKE) == -1
    assert call(tile_partials=FAKE, U=3) == -1
    assert call(ws_bytes=16) == -3
    assert call(ws=None) == -3


def test_gemm_validation(lib):
    f = lib.moe_w4a4_grouped_gemm
    base = dict(ac=FAKE, as_=FAKE, ag=FAKE, ari=None, a_rows=128, go=FAKE, E=4, rows=128, K=512,
                wc=FAKE, ws_=FAKE, wg=FAKE, N=256, sel=None, rc=None, rs=None, rg=None, kc=0,
                epi=0, rw=None, si=None, out_rows=0, out=FAKE, ldo=256, amax=None, ws=None,
                ws_bytes=0, stream=None)

    def call(**kw):
        a = dict(base, **kw)
        return f(*a.values())

    assert call(K=520) == -1 and "multiple of 64" in err(lib)
    assert call(K=48) == -1 and "multiple of 64" in err(lib)      # K % 16 == 0 is not enough
    assert call(a_rows=1 << 22, K=4096) == -2 and "4 GiB" in err(lib)
    assert call(sel=FAKE, kc=24, rc=FAKE, rs=FAKE, rg=FAKE) == -1
    assert call(sel=FAKE, kc=64, rg=None, rc=FAKE, rs=FAKE) == -1
    assert call(epi=1, N=255) == -1
    assert call(epi=2) == -1 and "scatter" in err(lib)
    assert call(epi=2, rw=FAKE, si=FAKE, out_rows=64) == -3 and "workspace" in err(lib)
    assert call(epi=9) == -1
    assert call(ldo=100) == -1
    assert call(out=None) == -1
    assert call(E=0) == -1


def test_qdq_and_guided_validation(lib):
    assert lib.qdq_weights(FAKE, 2, 16, 40, FAKE, None, None, None, FAKE, 4096, None) == -1
    assert lib.qdq_weights(FAKE, 2, 16, 32, FAKE, None, None, None, FAKE, 4096, None) == -1
    assert "in-place" in err(lib)
    assert lib.qdq_weights(FAKE, 2, 16, 32, ctypes.c_void_p(0x2000), None, None, None, None, 0,
                           None) == -3
    assert lib.guided_round(FAKE, 0, 4, 32, 32, None, FAKE, FAKE, FAKE, None, None, None) == -1
    assert lib.guided_round(FAKE, 0, 4, 24, 24, FAKE, FAKE, FAKE, FAKE, None, None, None) == -1


def test_guidance_record_validation(lib):
    assert lib.guidance_record_pack(None, 4, 32, FAKE, None) == -1
    assert "NULL" in err(lib)
    assert lib.guidance_record_pack(FAKE, 4, 24, FAKE, None) == -1
    assert "multiple of 16" in err(lib)
    assert lib.guidance_record_pack(FAKE, 4, 32, ctypes.c_void_p(0x1008), None) == -1
    assert "aligned" in err(lib)
    assert lib.guided_round_record(FAKE, 0, 4, 32, 32, None, FAKE, FAKE, FAKE, None, None, None) == -1
    assert lib.guided_round_record(FAKE, 0, 4, 24, 24, FAKE, FAKE, FAKE, FAKE, None, None, None) == -1
    assert lib.guided_round_record(FAKE, 3, 4, 32, 32, FAKE, FAKE, FAKE, FAKE, None, None, None) == -2



def test_mxfp4_validation(lib):
    assert lib.mxfp4_quantize(FAKE, 0, 4, 48, 48, FAKE, FAKE, None, None) == -1
    assert "multiple of 32" in err(lib)
    assert lib.mxfp4_quantize(None, 0, 4, 64, 64, FAKE, FAKE, None, None) == -1
    ws = lib.mxfp4_resq_select_and_requant_workspace_size(128, 8, 1, 32)
    assert ws == lib.resq_select_and_requant_workspace_size(128, 8, 1, 32)
    # k must be a multiple of 32 in MXFP4
    assert lib.mxfp4_resq_select_and_requant(FAKE, 0, 8, 128, 128, None, FAKE, FAKE, FAKE, 1, 8, 16,
                                             None, FAKE, FAKE, FAKE, FAKE, ws, None) == -1
    assert "multiple of 32" in err(lib)
    # the GEMM needs K % 128 == 0, kc % 32 == 0 and 4-byte aligned scales
    args = [FAKE, FAKE, None, 8, FAKE, 1, 8, 192, FAKE, FAKE, 256, None, None, None, 0, 0,
            None, None, 0, FAKE, 256, None, None, 0, None]
    assert lib.moe_mxfp4_grouped_gemm(*args) == -1
    assert "multiple of 128" in err(lib)
    args[7] = 256
    args[11], args[12], args[13], args[14] = FAKE, FAKE, FAKE, 48
    assert lib.moe_mxfp4_grouped_gemm(*args) == -1
    assert "kc=48" in err(lib)
    args[11], args[12], args[13], args[14] = None, None, None, 0
    args[9] = ctypes.c_void_p(0x1002)
    assert lib.moe_mxfp4_grouped_gemm(*args) == -1
    assert "4-byte aligned" in err(lib)


def test_w4a8_validation(lib):
    assert lib.mxfp8_quantize(FAKE, 0, 4, 48, 48, FAKE, FAKE, None) == -1
    assert "multiple of 32" in err(lib)
    args = [FAKE, FAKE, None, 8, FAKE, 1, 8, 192, FAKE, FAKE, 256, 0, None, None, 0, FAKE, 256,
            None, None, 0, None]
    assert lib.moe_mxfp4_w4a8_grouped_gemm(*args) == -1
    assert "multiple of 128" in err(lib)
    args[7] = 256
    args[11] = 2                    # scatter without row weights
    assert lib.moe_mxfp4_w4a8_grouped_gemm(*args) == -1
    assert "scatter" in err(lib)


def test_masked_validation(lib):
    # the dense-mask residual step shares the compact one's checks
    args = [FAKE, 0, 8, 64, 64, None, FAKE, FAKE, FAKE, FAKE, 1, 8, 24, None, FAKE, FAKE, FAKE,
            FAKE, FAKE, 1 << 20, None]
    assert lib.resq_mask_select_and_requant(*args) == -1
    assert "multiple of 16" in err(lib)
    args[3], args[4] = 32768, 32768
    args[12] = 32
    assert lib.resq_mask_select_and_requant(*args) == -2
    assert "16384" in err(lib)
    g = [FAKE, FAKE, FAKE, FAKE, 1, 8, 96, FAKE, FAKE, FAKE, 64, FAKE, 64, None]
    assert lib.moe_w4a4_masked_comp_gemm(*g) == -1
    assert "multiple of 64" in err(lib)
    g[6] = 128
    g[12] = 32                      # ldo < N
    assert lib.moe_w4a4_masked_comp_gemm(*g) == -1
    assert "ldo" in err(lib)
    g[12] = 64
    g[2] = None
    assert lib.moe_w4a4_masked_comp_gemm(*g) == -1
    assert "NULL" in err(lib)


def test_mxfp4_trainer_validation(lib):
    assert lib.mxfp4_qdq_weights(FAKE, 2, 8, 48, FAKE, None, None, None) == -1
    assert "multiple of 32" in err(lib)
    assert lib.mxfp4_qdq_weights(FAKE, 2, 8, 64, FAKE, None, None, None) == -1
    assert "in-place" in err(lib)
    assert lib.mxfp4_guided_round(FAKE, 0, 4, 48, 48, FAKE, FAKE, FAKE, None, None, None) == -1
    assert "multiple of 32" in err(lib)
    assert lib.mxfp4_guided_round(FAKE, 0, 4, 64, 64, None, FAKE, FAKE, None, None, None) == -1
    assert "NULL" in err(lib)
    assert lib.mxfp4_guided_round_record(FAKE, 0, 4, 48, 48, FAKE, FAKE, FAKE, None, None, None) == -1
    assert "multiple of 32" in err(lib)
