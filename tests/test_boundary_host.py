"""The C-ABI library on the host: it loads, exports every entry point the
header declares, and rejects bad arguments before any HIP call (so these
run without a GPU: no call here passes validation)."""
import ctypes
import os
import re

import pytest

import w4a16_dequant_gemm_amd as w4
from w4a16_dequant_gemm_amd import build as hipbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced (validation fails first)
FAKE_MIS = ctypes.c_void_p(0x10008)    # misaligned
NULL = None


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(hipbuild.LIB):
        hipbuild.build()
    return w4.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a16_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), f"{name} declared in w4a16.h but not exported"
    assert sorted(w4.C_FUNCTIONS) == names


def test_versions_and_status_strings(lib):
    assert w4.w4a16_abi_version() == 1
    assert w4.w4a16_layout_version() == 2
    for s in range(5):
        assert isinstance(w4.status_string(s), str) and w4.status_string(s)
    assert w4.status_string(99) == "unknown status"


@pytest.mark.parametrize("K,N,G,flags,expect", [
    (4096, 4096, 128, w4.W4A16_FP16, 4096 * 4096 // 2 + 32 * 4096 * 2 + 32 * 4096 // 2 + 16),
    (8192, 28672, 128, w4.W4A16_FP16, 8192 * 28672 // 2 + 64 * 28672 * 2 + 64 * 28672 // 2 + 16),
    (8192, 28672, 128, w4.W4A16_BF16 | w4.W4A16_SYM, 8192 * 28672 // 2 + 64 * 28672 * 2 + 16),
    (8192, 28672, 32, w4.W4A16_FP16, 8192 * 28672 // 2 + 256 * 28672 * 2 + 256 * 28672 // 2 + 16),
    (256, 128, 32, w4.W4A16_FP16, 256 * 128 // 2 + 8 * 128 * 2 + 8 * 128 // 2 + 16),
    (4352, 128, 64, w4.W4A16_BF16, 4352 * 128 // 2 + 68 * 128 * 2 + 68 * 128 // 2 + 16),
    (4096, 4000, 128, 0, 0),      # N % 128
    (4224, 4096, 128, 0, 0),      # K % 256
    (96, 128, 32, 0, 0),          # K % 256
    (4096, 4096, 100, 0, 0),      # G unsupported
    (4100, 4096, 128, 0, 0),      # K % G
    (0, 4096, 128, 0, 0),
    (4096, 4096, 128, 0x4, 0),    # unknown flag bit
])
def test_packed_bytes_is_the_algorithmic_weight_bytes_plus_trailer(lib, K, N, G, flags, expect):
    assert w4.w4a16_packed_bytes(K, N, G, flags) == expect


def test_workspace_bytes(lib):
    assert w4.w4a16_workspace_bytes(0, 4096, 4096, 128, 0) == 0
    assert w4.w4a16_workspace_bytes(1, 4096, 4096, 128, 0x8) == 0
    for M, N, K in [(1, 28672, 8192), (8, 28672, 8192), (32, 28672, 8192), (33, 28672, 8192),
                    (128, 28672, 8192), (4096, 28672, 8192), (2, 128, 1 << 20), (32, 128, 1 << 20),
                    (1, 4096, 4096), (16, 8192, 28672)]:
        ws = w4.w4a16_workspace_bytes(M, N, K, 128, 0)
        Mp = -(-M // 32) * 32
        assert 0 <= ws <= max(64 * Mp * N, 262144 * M) + 65536
        assert ws == 0 or ws > 65536


def test_plan_hints(lib):
    """Plan hints are accepted where a plan is made (workspace size, GEMM) and
    nowhere else; the decode kernel needs a workspace only when the tiles do
    not divide evenly over the workgroups (the left-over tiles are split along
    K); a hint that does not apply to the shape falls back to the default
    choice."""
    f = w4.W4A16_FP16
    assert w4.plan_flags(None) == 0
    assert w4.plan_flags("decode") == 0x10 and w4.plan_flags(("splitk", 3)) == 0x320
    for bad in ("fast", ("tiled", 256), ("decode", -1)):
        with pytest.raises(ValueError):
            w4.plan_flags(bad)
    # 256 tiles of 32 columns over 256 workgroups: nothing to split
    assert w4.w4a16_workspace_bytes(4, 8192, 8192, 128, f | w4.plan_flags("decode")) == 0
    assert w4.w4a16_workspace_bytes(4, 8192, 8192, 128, f) == 0           # decode by default
    # 896 tiles: 3 rounds, then 128 tiles in two halves of K each: one counter
    # area plus 2 x 128 partial tiles of 8 rows x 32 columns (fp32)
    assert w4.w4a16_workspace_bytes(4, 28672, 8192, 128, f) == 65536 + 2 * 128 * 1024
    assert w4.w4a16_workspace_bytes(4, 28672, 8192, 128, f | w4.plan_flags(("decode", 224))) == 0
    # 128 tiles over 256 workgroups: whole tiles up to K = 8192 (no workspace),
    # split in halves beyond, or when the workgroup count is forced
    assert w4.w4a16_workspace_bytes(1, 4096, 4096, 128, f) == 0
    assert w4.w4a16_workspace_bytes(4, 4096, 8192, 128, f) == 0
    assert w4.w4a16_workspace_bytes(1, 4096, 16384, 128, f) == 65536 + 2 * 128 * 1024
    assert w4.w4a16_workspace_bytes(1, 2048, 4096, 128, f) == 0
    assert w4.w4a16_workspace_bytes(1, 2048, 4096, 128, f | w4.plan_flags(("decode", 255))) > 0
    # wide kernel: 224 blocks of 128 columns fill the workgroups, no workspace;
    # 64 blocks are split into 4 parts (4 tiles x 2 row tiles x 16 x 64 floats each)
    assert w4.w4a16_workspace_bytes(64, 28672, 8192, 128, f | w4.plan_flags("wide")) == 0
    assert w4.w4a16_workspace_bytes(64, 8192, 8192, 128, f | w4.plan_flags("wide")) == \
        65536 + 64 * 4 * (4 * 2 * 16 * 64 * 4)
    assert w4.plan_flags("wide") == 0x40
    assert w4.w4a16_workspace_bytes(4, 4096, 8192, 128, f | w4.plan_flags(("tiled", 4))) > 0
    # decode holds X in LDS: M = 8 rows of K = 16384 do not fit, the hint is ignored
    assert w4.w4a16_workspace_bytes(8, 4096, 1 << 14, 128, f | w4.plan_flags("decode")) == \
        w4.w4a16_workspace_bytes(8, 4096, 1 << 14, 128, f)
    assert w4.w4a16_packed_bytes(4096, 4096, 128, f | 0x10) == 0
    assert lib.w4a16_repack(FAKE, FAKE, FAKE, 256, 256, 128, 0x10, FAKE, 1 << 30, None) == \
        w4.W4A16_ERR_INVALID_ARG


def gemm(lib, X=FAKE, packed=FAKE, pbytes=1 << 40, Y=FAKE, M=8, N=4096, K=4096, G=128, flags=0,
         ws=FAKE, wsb=1 << 40):
    return lib.w4a16_gemm(X, packed, pbytes, Y, M, N, K, G, flags, ws, wsb, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(M=0), w4.W4A16_ERR_INVALID_ARG),
    (dict(M=-1), w4.W4A16_ERR_INVALID_ARG),
    (dict(K=4100), w4.W4A16_ERR_INVALID_ARG),            # K % G
    (dict(K=0), w4.W4A16_ERR_INVALID_ARG),
    (dict(N=0), w4.W4A16_ERR_INVALID_ARG),
    (dict(N=4000), w4.W4A16_ERR_UNSUPPORTED),            # N % 128
    (dict(K=4224), w4.W4A16_ERR_UNSUPPORTED),            # K % 256
    (dict(flags=0x80), w4.W4A16_ERR_INVALID_ARG),        # neither a blob flag nor a plan hint

    (dict(G=256), w4.W4A16_ERR_UNSUPPORTED),
    (dict(G=16), w4.W4A16_ERR_UNSUPPORTED),
    (dict(G=100), w4.W4A16_ERR_INVALID_ARG),             # does not divide K
    (dict(flags=0x4), w4.W4A16_ERR_INVALID_ARG),
    (dict(X=NULL), w4.W4A16_ERR_INVALID_ARG),
    (dict(Y=NULL), w4.W4A16_ERR_INVALID_ARG),
    (dict(packed=NULL), w4.W4A16_ERR_INVALID_ARG),
    (dict(X=FAKE_MIS), w4.W4A16_ERR_INVALID_ARG),
    (dict(Y=FAKE_MIS), w4.W4A16_ERR_INVALID_ARG),
    (dict(packed=FAKE_MIS), w4.W4A16_ERR_INVALID_ARG),
    (dict(pbytes=100), w4.W4A16_ERR_INVALID_ARG),        # blob too small
    (dict(M=16, K=8192, N=4096, ws=NULL), w4.W4A16_ERR_WORKSPACE),
    (dict(M=16, K=8192, N=4096, wsb=16), w4.W4A16_ERR_WORKSPACE),
    (dict(M=16, K=8192, N=4096, ws=FAKE_MIS), w4.W4A16_ERR_WORKSPACE),
    (dict(M=1 << 31), w4.W4A16_ERR_INVALID_ARG),
])
def test_gemm_rejects_before_any_launch(lib, kw, expect):
    if kw.get("ws", FAKE) is not FAKE or kw.get("wsb", 1) == 16:
        # these need a plan that uses a workspace
        assert w4.w4a16_workspace_bytes(16, 4096, 8192, 128, 0) > 0
    assert gemm(lib, **kw) == expect


@pytest.mark.parametrize("fn", ["repack", "unrepack"])
@pytest.mark.parametrize("case,expect", [
    ("sym_with_zeros", w4.W4A16_ERR_INVALID_ARG),
    ("asym_without_zeros", w4.W4A16_ERR_INVALID_ARG),
    ("short_blob", w4.W4A16_ERR_INVALID_ARG),
    ("null_qweight", w4.W4A16_ERR_INVALID_ARG),
    ("misaligned_scales", w4.W4A16_ERR_INVALID_ARG),
    ("bad_n", w4.W4A16_ERR_UNSUPPORTED),
    ("bad_k", w4.W4A16_ERR_INVALID_ARG),
    ("k_not_256", w4.W4A16_ERR_UNSUPPORTED),
])
def test_repack_rejects(lib, fn, case, expect):
    K, N, G = 256, 256, 128
    flags, zeros, pbytes, qw, sc = 0, FAKE, 1 << 30, FAKE, FAKE
    if case == "sym_with_zeros":
        flags = w4.W4A16_SYM
    elif case == "asym_without_zeros":
        zeros = NULL
    elif case == "short_blob":
        pbytes = w4.w4a16_packed_bytes(K, N, G, 0) - 1
    elif case == "null_qweight":
        qw = NULL
    elif case == "misaligned_scales":
        sc = FAKE_MIS
    elif case == "bad_n":
        N = 200
    elif case == "bad_k":
        K = 200
    elif case == "k_not_256":
        K = 384
    if fn == "repack":
        rc = lib.w4a16_repack(qw, sc, zeros, K, N, G, flags, FAKE, pbytes, None)
    else:
        rc = lib.w4a16_unrepack(FAKE, pbytes, qw, sc, zeros, K, N, G, flags, None)
    assert rc == expect


def test_dequant_and_probe_reject(lib):
    assert lib.w4a16_dequant(FAKE, 1 << 30, NULL, 256, 256, 128, 0, None) == w4.W4A16_ERR_INVALID_ARG
    assert lib.w4a16_dequant(FAKE, 10, FAKE, 256, 256, 128, 0, None) == w4.W4A16_ERR_INVALID_ARG
    assert lib.w4a16_dequant(FAKE, 1 << 30, FAKE, 256, 200, 128, 0, None) == w4.W4A16_ERR_UNSUPPORTED
    assert lib.w4a16_mfma_layout_probe(FAKE, FAKE, NULL, 0, None) == w4.W4A16_ERR_INVALID_ARG
    assert lib.w4a16_mfma_layout_probe(FAKE, FAKE, FAKE, 0x2, None) == w4.W4A16_ERR_INVALID_ARG
    ob = lib.w4a16_read_probe_out_bytes()
    assert ob == 256 * 512 * 16
    assert lib.w4a16_read_probe(FAKE, 1000, FAKE, ob, None) == w4.W4A16_ERR_INVALID_ARG     # not 1 KiB
    assert lib.w4a16_read_probe(FAKE, 0, FAKE, ob, None) == w4.W4A16_ERR_INVALID_ARG
    assert lib.w4a16_read_probe(FAKE, 4096, FAKE, ob - 16, None) == w4.W4A16_ERR_INVALID_ARG
    assert lib.w4a16_read_probe(FAKE_MIS, 4096, FAKE, ob, None) == w4.W4A16_ERR_INVALID_ARG
    assert lib.w4a16_read_probe(NULL, 4096, FAKE, ob, None) == w4.W4A16_ERR_INVALID_ARG


def test_python_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        saved = w4._lib
        w4._lib = None
        try:
            w4.load_library(str(tmp_path / "nope.so"))
        finally:
            w4._lib = saved


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "w4a16_dequant_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "w4a16_oracle" not in text and "liboracle" not in text, f


def test_noalloc_rejects_before_any_launch(lib):
    """w4a16_gemm_noalloc validates like w4a16_gemm_ex and refuses a shape whose
    plan needs more scratch than its static array, before any HIP call."""
    def call(X=FAKE, packed=FAKE, pbytes=1 << 40, Y=FAKE, M=8, N=4096, K=4096, G=128, flags=0):
        return lib.w4a16_gemm_noalloc(X, packed, pbytes, Y, M, N, K, G, flags, None, None)
    M, N, K, G = 128, 28672, 8192, 64
    assert w4.w4a16_workspace_bytes(M, N, K, G, 0) > w4.W4A16_NOALLOC_SCRATCH_BYTES
    assert call(M=M, N=N, K=K, G=G) == w4.W4A16_ERR_WORKSPACE
    assert call(M=0) == w4.W4A16_ERR_INVALID_ARG
    assert call(X=NULL) == w4.W4A16_ERR_INVALID_ARG
    assert call(Y=FAKE_MIS) == w4.W4A16_ERR_INVALID_ARG
    assert call(N=4000) == w4.W4A16_ERR_UNSUPPORTED
    assert call(pbytes=100) == w4.W4A16_ERR_INVALID_ARG
