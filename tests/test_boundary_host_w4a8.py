"""The W4A8 entry points (include/w4a8.h) on the host: exported, sized, and
rejecting bad arguments before any HIP call (no call here passes
validation, so these run without a GPU)."""
import ctypes
import os
import re

import pytest

import w4a16_dequant_gemm_amd as w4
from w4a16_dequant_gemm_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a8.h")

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced (validation fails first)
FAKE_MIS = ctypes.c_void_p(0x10008)    # misaligned
NULL = None
INV, UNS = w4.W4A16_ERR_INVALID_ARG, w4.W4A16_ERR_UNSUPPORTED


@pytest.fixture(scope="module")
def w8():
    if not os.path.exists(hipbuild.LIB):
        hipbuild.build()
    from w4a16_dequant_gemm_amd import w4a8
    w4a8._lib()
    return w4a8


def test_exports_every_declared_symbol(w8):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(w4a8_[a-z0-9_]+)\s*\(", text)))
    assert len(names) == 5
    lib = w4.load_library()
    for name in names:
        assert hasattr(lib, name), f"{name} declared in w4a8.h but not exported"
    assert sorted(w8.C_FUNCTIONS_W4A8) == names


@pytest.mark.parametrize("K,N,G,expect", [
    (8192, 28672, 128, 8192 * 28672 // 2 + 64 * 28672 * 2 + 28672 * 4 + 16),
    (256, 128, 32, 256 * 128 // 2 + 8 * 128 * 2 + 128 * 4 + 16),
    (131072, 128, 64, 131072 * 128 // 2 + 2048 * 128 * 2 + 128 * 4 + 16),
    (131072 + 256, 128, 128, 0),      # beyond the int32-safe K
    (100, 128, 128, 0), (256, 64, 128, 0), (256, 128, 256, 0), (256, 128, 48, 0),
])
def test_packed_bytes(w8, K, N, G, expect):
    assert w8.w4a8_packed_bytes(K, N, G) == expect


def _gemm(X=FAKE, sx=FAKE, packed=FAKE, pbytes=1 << 40, Y=FAKE, M=4, N=256, K=512, G=128,
          flags=0):
    lib = w4.load_library()
    return lib.w4a8_gemm(X, sx, packed, pbytes, Y, M, N, K, G, flags, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(M=0), INV), (dict(M=1 << 31), INV), (dict(X=NULL), INV), (dict(packed=NULL), INV),
    (dict(Y=NULL), INV), (dict(X=FAKE_MIS), INV), (dict(Y=FAKE_MIS), INV),
    (dict(sx=NULL), INV),                       # fp16 output needs sx
    (dict(sx=NULL, flags=0x3), INV),            # no output kind 3
    (dict(flags=0x4), INV), (dict(flags=0x40), INV),
    (dict(N=200), UNS), (dict(K=384), UNS), (dict(K=300), INV), (dict(G=256), UNS),
    (dict(G=0), INV), (dict(K=131072 + 256), UNS), (dict(pbytes=100), INV),
])
def test_gemm_rejects_before_any_launch(w8, kw, expect):
    assert _gemm(**kw) == expect


def test_repack_dequant_quantize_reject(w8):
    lib = w4.load_library()
    ok = dict(q=FAKE, s=FAKE, a=FAKE, sw=FAKE, K=256, N=128, G=64, p=FAKE, pb=1 << 30)

    def rep(**kw):
        c = {**ok, **kw}
        return lib.w4a8_repack(c["q"], c["s"], c["a"], c["sw"], c["K"], c["N"], c["G"], c["p"],
                               c["pb"], None)
    assert rep(q=NULL) == INV
    assert rep(sw=FAKE_MIS) == INV
    assert rep(pb=1000) == INV
    assert rep(N=100) == UNS
    assert rep(K=200) == INV
    assert rep(G=16) == UNS
    assert lib.w4a8_dequant(FAKE, 10, FAKE, 256, 128, 64, None) == INV
    assert lib.w4a8_dequant(NULL, 1 << 30, FAKE, 256, 128, 64, None) == INV
    assert lib.w4a8_dequant(FAKE, 1 << 30, FAKE, 256, 96, 64, None) == UNS
    assert lib.w4a8_quantize_rows(FAKE, FAKE, FAKE, 0, 256, 0, None) == INV
    assert lib.w4a8_quantize_rows(FAKE, FAKE, FAKE, 4, 100, 0, None) == UNS
    assert lib.w4a8_quantize_rows(FAKE, FAKE, FAKE, 4, 256, 2, None) == INV
    assert lib.w4a8_quantize_rows(FAKE, FAKE, FAKE_MIS, 4, 256, 0, None) == INV


def test_plan_hint_names(w8):
    assert w8.plan_flags_w8(None) == 0
    assert w8.plan_flags_w8("tiled") == 0x20
    assert w8.plan_flags_w8(("stream", 4)) == 0x10 | (4 << 8)
    with pytest.raises(ValueError):
        w8.plan_flags_w8("wide")


def test_bindings_reject_bad_tensors_before_any_launch(w8):
    """The Python bindings check what the C side cannot see (device, dtype,
    element count, contiguity); these CPU tensors fail those checks, so no
    pointer ever reaches a kernel."""
    import torch
    from w4a16_dequant_gemm_amd import mxfp4 as mx
    K, N, G = 256, 128, 64
    qw = torch.zeros((K // 8, N), dtype=torch.int32)
    s8 = torch.zeros((K // G, N), dtype=torch.uint8)
    with pytest.raises(w4.W4A16Error):
        w8.w4a8_repack(qw, s8, s8, torch.zeros(N), K, N, G)            # CPU tensors
    with pytest.raises(w4.W4A16Error):
        w8.w4a8_repack(qw[:4], s8, s8, torch.zeros(N), K, N, G)        # short qweight
    with pytest.raises(w4.W4A16Error):
        w8.w4a8_quantize_rows(torch.zeros((2, K), dtype=torch.float32))
    with pytest.raises(w4.W4A16Error):
        mx.mxfp4_repack(qw, torch.zeros((K // 32, N), dtype=torch.uint8), K, N)
    with pytest.raises(w4.W4A16Error):
        mx.mxfp4_quantize_rows(torch.zeros((2, K), dtype=torch.float16))
    packed = w8.PackedW8(torch.zeros(10, dtype=torch.uint8), K, N, G)
    with pytest.raises(w4.W4A16Error):
        w8.w4a8_gemm(torch.zeros((2, K), dtype=torch.int8), None, packed, out="fp16")
    pm = mx.PackedMX(torch.zeros(10, dtype=torch.uint8), K, N)
    with pytest.raises(w4.W4A16Error):
        mx.mxfp4_gemm(torch.zeros((2, K), dtype=torch.uint8), torch.zeros((2, K // 32),
                      dtype=torch.uint8), pm)
