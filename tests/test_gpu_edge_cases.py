"""GPU edge cases of the fused product (through the C ABI): degenerate weights
and scales, non-finite activations, and the smallest legal shape.

* q = z everywhere, or every scale 0: every dequantized weight is 0, so Y is
  exactly 0 (up to the sign of zero) whatever X is.
* A NaN in one activation row: IEEE arithmetic makes that output row NaN; every
  other row is unaffected, bit for bit (no partial sum crosses rows in any
  reduction, inside a wave, between waves or between workgroups).
* The smallest shape the library accepts (K = 256, N = 128) against the
  oracle, with every group size.
"""
import numpy as np
import pytest

import oracle
import w4a16_synth as synth
from gpu_helpers import OnDevice, assert_gemm_close, lib, same_bits, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lib()


# (plan hint, M, K, N, G)
CASES = [
    ("decode", 1, 2048, 512, 128),
    (("decode", 2), 8, 1024, 384, 64),
    (("decode", 3), 7, 1024, 256, 32),
    ("splitk", 1, 2048, 512, 128),
    (("splitk", 3), 7, 1024, 256, 64),
    (("splitk", 2), 30, 1024, 384, 32),
    ("wide", 40, 2048, 512, 128),
    (("wide", 16), 100, 1024, 384, 64),
    ("tiled", 48, 2048, 512, 128),
    (("tiled", 2), 130, 1024, 1024, 64),
]
IDS = [f"{c[0] if isinstance(c[0], str) else c[0][0]}-m{c[1]}" for c in CASES]


def bits_of_problem_with(p, qweight=None, scales=None, zeros=None, X=None):
    return synth.Problem(p.M, p.K, p.N, p.G, p.dtype, p.sym,
                         p.X if X is None else X,
                         p.qweight if qweight is None else qweight,
                         p.scales if scales is None else scales,
                         p.zeros if zeros is None else zeros)


def run(p, plan):
    d = OnDevice(p)
    Y = d.gemm(plan=plan)
    return d, d.w4.bits_of(Y)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_q_equal_z_everywhere_gives_zero(case):
    variant, M, K, N, G = case
    p = synth.make_problem(M, K, N, G=G, dtype="fp16", sym=False, seed=M + N)
    # every nibble equal to its group's zero point
    q = np.repeat(p.zeros, G, axis=0)                   # [K][N]
    qw = synth.pack_nibbles(q)
    say(f"q == z: {variant} M={M} K={K} N={N} G={G}")
    _, Yb = run(bits_of_problem_with(p, qweight=qw), variant)
    assert same_bits(Yb, np.zeros_like(Yb))


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_zero_scales_give_zero(case):
    variant, M, K, N, G = case
    p = synth.make_problem(M, K, N, G=G, dtype="bf16", sym=True, seed=M + 2 * N)
    say(f"zero scales: {variant} M={M} K={K} N={N} G={G}")
    _, Yb = run(bits_of_problem_with(p, scales=np.zeros_like(p.scales)), variant)
    assert same_bits(Yb, np.zeros_like(Yb))


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_nan_row_stays_in_its_row(case):
    variant, M, K, N, G = case
    p = synth.make_problem(M, K, N, G=G, dtype="fp16", sym=False, seed=3 * M + N)
    r = M // 2
    Xn = p.X.copy()
    Xn[r, K // 3] = 0x7E00                               # fp16 quiet NaN
    say(f"NaN row {r}: {variant} M={M} K={K} N={N} G={G}")
    _, Y0 = run(p, variant)
    _, Y1 = run(bits_of_problem_with(p, X=Xn), variant)
    row = Y1[r].astype(np.uint32)
    assert np.all(((row & 0x7C00) == 0x7C00) & ((row & 0x03FF) != 0)), "row with a NaN input"
    others = np.delete(np.arange(M), r)
    assert np.array_equal(Y0[others], Y1[others])


@pytest.mark.parametrize("variant", ["decode", "splitk", "tiled"])
@pytest.mark.parametrize("G", [32, 64, 128])
@pytest.mark.parametrize("dtype,sym", [("fp16", False), ("bf16", True)])
def test_smallest_shape(variant, G, dtype, sym):
    M, K, N = 3, 256, 128
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=11 + G)
    say(f"smallest shape: {variant} G={G} {dtype}")
    d, Yb = run(p, variant)
    Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, sym)
    assert_gemm_close(p, oracle.bits_to_float(Yb, dtype), Yref, B, "smallest shape")
