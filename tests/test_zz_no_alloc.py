"""w4a16_gemm_noalloc (through the C ABI) against w4a16_gemm_ex with a caller
workspace: the same kernels, so the outputs must be equal bit for bit, and
both within the tolerance of the oracle.  Two calls in a row on the static
scratch, the second with a smaller problem, so the second call runs on what
the first left in the scratch; then the same with an epilogue.
"""
import numpy as np
import pytest

import oracle
import w4a16_synth as synth
from gpu_helpers import TOL, OnDevice, lib, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lib()


# (label, M, K, N, G, dtype, sym, plan hint): each needs scratch, the second of
# each pair is smaller than the first
PAIRS = [
    (("tiled-split", 70, 4096, 1024, 128, "fp16", False, ("tiled", 4)),
     ("splitk-shared", 5, 2048, 512, 64, "fp16", False, ("splitk", 3))),
    (("splitk-shared", 9, 8192, 4096, 128, "bf16", True, "splitk"),
     ("tiled-split", 40, 1024, 256, 32, "bf16", True, ("tiled", 2))),
]


def run_pair(pair, with_epilogue):
    w4 = lib()
    for label, M, K, N, G, dtype, sym, plan in pair:
        p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=M * 7 + N)
        say(f"noalloc {label}: M={M} K={K} N={N} G={G} {dtype} sym={sym} ep={with_epilogue}")
        need = w4.w4a16_workspace_bytes(M, N, K, G, w4.flags_of(dtype, sym) | w4.plan_flags(plan))
        assert 0 < need <= w4.W4A16_NOALLOC_SCRATCH_BYTES, (label, need)
        d = OnDevice(p)
        kw = dict(plan=plan)
        if with_epilogue:
            rng = np.random.default_rng(N)
            kw.update(col_scale=torch.from_numpy(rng.uniform(-1, 1, N).astype(np.float32)).cuda(),
                      bias=torch.from_numpy(rng.normal(0, 0.5, N)).to(d.X.dtype).cuda(),
                      activation="silu")
        Y_ref = d.w4.w4a16_gemm_ex(d.X, d.packed, **kw)
        Y = torch.full((M, N), float("nan"), dtype=d.X.dtype, device=d.X.device)
        w4.w4a16_gemm_noalloc(d.X, d.packed, Y, **kw)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16)), label
        if not with_epilogue:
            Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, sym)
            rel, zero_ok = oracle.max_rel_error(d.y_float(Y), Yref, B)
            assert zero_ok and rel <= TOL[dtype], (label, rel)


@pytest.mark.parametrize("i", range(len(PAIRS)))
def test_noalloc_equals_workspace_path(i):
    run_pair(PAIRS[i], with_epilogue=False)


@pytest.mark.parametrize("i", range(len(PAIRS)))
def test_noalloc_equals_workspace_path_with_epilogue(i):
    run_pair(PAIRS[i], with_epilogue=True)


def test_noalloc_without_scratch_need():
    """A shape whose plan needs no scratch (whole column blocks per workgroup)."""
    w4 = lib()
    p = synth.make_problem(2, 1024, 28672, G=128, dtype="fp16", sym=False, seed=3)
    assert w4.w4a16_workspace_bytes(2, 28672, 1024, 128, 0) == 0
    d = OnDevice(p)
    Y = torch.empty((2, 28672), dtype=torch.float16, device="cuda")
    w4.w4a16_gemm_noalloc(d.X, d.packed, Y)
    Y_ref = d.gemm()
    assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16))


def test_noalloc_rejects_a_shape_beyond_the_scratch():
    w4 = lib()
    M, K, N = 128, 8192, 28672
    assert w4.w4a16_workspace_bytes(M, N, K, 64, 0) > w4.W4A16_NOALLOC_SCRATCH_BYTES
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    blob = torch.zeros(w4.w4a16_packed_bytes(K, N, 64, 0), dtype=torch.uint8, device="cuda")
    packed = w4.PackedW4(blob, K, N, 64, 0, w4.w4a16_layout_version())
    Y = torch.zeros((M, N), dtype=torch.float16, device="cuda")
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_gemm_noalloc(X, packed, Y)
    assert e.value.status == w4.W4A16_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(Y.count_nonzero()) == 0   # nothing was launched
