"""The MXFP4 entry points (include/mxfp4.h) on the host: exported, sized, and
rejecting bad arguments before any HIP call (no call here passes validation)."""
import ctypes
import os
import re

import pytest

import w4a16_dequant_gemm_amd as w4
from w4a16_dequant_gemm_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x10000)
FAKE_MIS = ctypes.c_void_p(0x10008)
INV, UNS = w4.W4A16_ERR_INVALID_ARG, w4.W4A16_ERR_UNSUPPORTED


@pytest.fixture(scope="module")
def mx():
    if not os.path.exists(hipbuild.LIB):
        hipbuild.build()
    from w4a16_dequant_gemm_amd import mxfp4
    mxfp4._lib()
    return mxfp4


def test_exports_every_declared_symbol(mx):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mxfp4.h")).read(),
                  flags=re.S)
    names = sorted(set(re.findall(r"\b(mxfp4_[a-z0-9_]+)\s*\(", text)))
    assert len(names) == 4
    lib = w4.load_library()
    for name in names:
        assert hasattr(lib, name)
    assert sorted(mx.C_FUNCTIONS_MXFP4) == names


@pytest.mark.parametrize("K,N,expect", [
    (8192, 28672, 8192 * 28672 // 2 + 8192 * 28672 // 32 + 16), (256, 128, 256 * 64 + 1024 + 16),
    (100, 128, 0), (256, 64, 0), (0, 128, 0)])
def test_packed_bytes(mx, K, N, expect):
    assert mx.mxfp4_packed_bytes(K, N) == expect


def test_rejects_before_any_launch(mx):
    lib = w4.load_library()

    def gemm(xq=FAKE, xs=FAKE, p=FAKE, pb=1 << 40, Y=FAKE, M=4, N=256, K=512, flags=0):
        return lib.mxfp4_gemm(xq, xs, p, pb, Y, M, N, K, flags, None)
    assert gemm(M=0) == INV
    assert gemm(xs=None) == INV
    assert gemm(Y=FAKE_MIS) == INV
    assert gemm(flags=0x2) == INV
    assert gemm(flags=0x40) == INV
    assert gemm(N=200) == UNS
    assert gemm(K=320) == UNS
    assert gemm(pb=1000) == INV
    assert lib.mxfp4_repack(FAKE, None, 256, 128, FAKE, 1 << 30, None) == INV
    assert lib.mxfp4_repack(FAKE, FAKE, 256, 128, FAKE, 100, None) == INV
    assert lib.mxfp4_repack(FAKE, FAKE, 256, 96, FAKE, 1 << 30, None) == UNS
    assert lib.mxfp4_quantize_rows(FAKE, FAKE, FAKE, 0, 256, 0, None) == INV
    assert lib.mxfp4_quantize_rows(FAKE, FAKE, FAKE, 2, 300, 0, None) == UNS
    assert lib.mxfp4_quantize_rows(FAKE, FAKE, FAKE, 2, 256, 4, None) == INV
    assert lib.mxfp4_quantize_rows(FAKE, FAKE_MIS, FAKE, 2, 256, 0, None) == INV


def test_plan_hint_names(mx):
    assert mx.plan_flags_mx(("tiled", 2)) == 0x20 | (2 << 8)
    with pytest.raises(ValueError):
        mx.plan_flags_mx("decode")
