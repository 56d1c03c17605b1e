"""GPU parity of the MXFP4 route (include/mxfp4.h) against the CPU oracle
(oracle/mxfp4.py), through the C ABI.

Bar:
  * bit-exact: the E4M3 codes and E8M0 scales of the activation quantiser
    (an integer decision per element, taken on both sides from the same exact
    values with the same rounding rule);
  * the product: max |Y - y| / B <= 2e-3 (fp16 output) or 1e-2 (bf16 output),
    with y the oracle's sum and B = sum |xa| |w|; Y == 0 wherever B == 0.  The
    matrix unit accumulates in fp32 (a relative error of about K * 2^-24 of B
    at worst) and the output is rounded once (half an ulp: 2^-11 or 2^-8 of
    |y| <= B).
"""
import numpy as np
import pytest

from oracle import mxfp4 as omx
import w4a16_synth as synth
from gpu_helpers import lib, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
TOL = {"fp16": 2e-3, "bf16": 1e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lib()


def mxmod():
    from w4a16_dequant_gemm_amd import mxfp4
    return mxfp4


def check_shapes_mx(p):
    assert p.xq.shape == (p.M, p.K) and p.xq.dtype == np.uint8
    assert p.xs.shape == (p.M, p.K // 32) and p.xs.dtype == np.uint8
    assert p.qweight.shape == (p.K // 8, p.N) and p.qweight.dtype == np.uint32
    assert p.ws.shape == (p.K // 32, p.N) and p.ws.dtype == np.uint8
    assert p.N % 128 == 0 and p.K % 256 == 0


class OnDeviceMX:
    def __init__(self, p):
        check_shapes_mx(p)
        self.mx = mxmod()
        self.p = p
        d = "cuda"
        self.xq = torch.from_numpy(p.xq).to(d)
        self.xs = torch.from_numpy(p.xs).to(d)
        self.packed = self.mx.mxfp4_repack(torch.from_numpy(p.qweight.view(np.int32)).to(d),
                                           torch.from_numpy(p.ws).to(d), p.K, p.N)

    def gemm(self, out, plan=None, xq=None, xs=None):
        Y = self.mx.mxfp4_gemm(self.xq if xq is None else xq, self.xs if xs is None else xs,
                               self.packed, out=out, plan=plan)
        torch.cuda.synchronize()
        return Y


def y_float(Y):
    return Y.float().cpu().numpy().astype(np.float64)


def assert_close(Yg, y, B, dt, what=""):
    zero = B == 0
    assert np.all(Yg[zero] == 0), f"{what}: an output with bound 0 is not 0"
    rel = np.max(np.abs(Yg - y)[~zero] / B[~zero]) if np.any(~zero) else 0.0
    assert rel <= TOL[dt], f"{what}: max|Y-y|/B = {rel:.3e} > {TOL[dt]}"
    return rel


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("M,K", [(1, 256), (5, 1024), (40, 4096), (3, 8192)])
def test_quantize_rows_bit_exact(dtype, M, K):
    say(f"mxfp4 quantize rows {dtype} M={M} K={K}")
    bits = synth.make_activations(M, K, dtype, seed=M + K, outlier_frac=0.01)
    x = omx_bits_to_float(bits, dtype)
    if M > 2:
        bits[1, 32:64] = 0                      # a block of zeros
        bits[2, :32] = bits[2, :32] & 0x8000    # a block of signed zeros
        x = omx_bits_to_float(bits, dtype)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    X = torch.from_numpy(bits.view(np.int16)).to("cuda").view(tdt)
    xq, xs = mxmod().mxfp4_quantize_rows(X)
    torch.cuda.synchronize()
    want_q, want_s = omx.quantize_rows(x)
    assert np.array_equal(xs.cpu().numpy(), want_s)
    assert np.array_equal(xq.cpu().numpy(), want_q)


def omx_bits_to_float(bits, dtype):
    from oracle import w4a8 as o8
    return o8.bits_to_float(bits, dtype)


def test_quantize_rows_saturation_and_ties():
    """Blocks built to hit saturation (amax just under the next power of two)
    and exact E4M3 ties."""
    K = 256
    x = np.zeros((2, K))
    x[0, :32] = 1.9375                          # scales to 496: saturates to 448
    x[0, 32:64] = np.linspace(-1.0, 1.0, 32)
    x[0, 64] = 1.0
    x[0, 65:96] = 1.0 + 1.0 / 16                # 272: halfway between 256 and 288 -> 256
    x[0, 96] = 1.0
    x[0, 97:128] = 1.0 + 3.0 / 16               # 304: halfway 288/320 -> 320 (even code)
    x[1, :] = np.ldexp(1.0, -20) * np.arange(K) # tiny values (fp16 subnormal range)
    bits = x.astype(np.float16).view(np.uint16)
    xf = omx_bits_to_float(bits, "fp16")
    X = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.float16)
    say("mxfp4 quantize saturation and ties")
    xq, xs = mxmod().mxfp4_quantize_rows(X)
    torch.cuda.synchronize()
    want_q, want_s = omx.quantize_rows(xf)
    assert np.array_equal(xs.cpu().numpy(), want_s)
    assert np.array_equal(xq.cpu().numpy(), want_q)
    assert want_q[0, 0] == 0x7E


GEMM_CASES = [  # (M, K, N, plan)
    (1, 256, 128, None), (1, 1024, 384, None), (7, 2048, 256, None), (17, 512, 128, ("stream", 2)),
    (32, 1024, 256, ("stream", 4)), (31, 2048, 128, ("stream", 8)), (48, 512, 256, ("stream", 2)),
    (3, 512, 384, "tiled"), (33, 512, 384, None), (64, 1024, 256, None), (100, 1024, 256, None),
    (130, 768, 640, None), (200, 512, 384, ("tiled", 3)), (300, 512, 128, None),
    (40, 1024, 640, ("tiled", 1)), (513, 1024, 384, None), (1000, 512, 640, None),
    (300, 768, 640, ("tiled", 4)), (33, 1024, 128, ("tiled", 4)), (600, 512, 384, ("tiled", 1)),
    # the block-diagonal streaming form (M <= 8) with every parts count
    (2, 512, 128, ("stream", 4)), (4, 1024, 256, ("stream", 2)), (8, 2048, 384, ("stream", 8)),
    (5, 4096, 640, None), (6, 8192, 128, None),
]


@pytest.mark.parametrize("M,K,N,plan", GEMM_CASES)
def test_gemm_against_oracle(M, K, N, plan):
    say(f"mxfp4 gemm M={M} K={K} N={N} plan={plan}")
    p = synth.make_mxfp4_problem(M, K, N, seed=M * 3 + K + N)
    d = OnDeviceMX(p)
    _, y, B = omx.gemm(p.xq, p.xs, p.qweight, p.ws, M, N, K, "fp16")
    for dt in ("fp16", "bf16"):
        assert_close(y_float(d.gemm(dt, plan=plan)), y, B, dt, f"M={M} {dt}")


def test_plans_agree_bitwise():
    """The kernels differ in how they split K only across parts (stream) or
    not at all (tiled): fixed summation orders, repeatable bit for bit."""
    M, K, N = 24, 2048, 384
    p = synth.make_mxfp4_problem(M, K, N, seed=9)
    d = OnDeviceMX(p)
    say("mxfp4 repeatability")
    for pl in (("stream", 2), ("stream", 8), "tiled"):
        a = d.gemm("fp16", plan=pl).cpu().numpy()
        b = d.gemm("fp16", plan=pl).cpu().numpy()
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_chain_quantize_then_gemm():
    M, K, N = 20, 4096, 512
    bits = synth.make_activations(M, K, "bf16", seed=6, outlier_frac=0.001)
    qw, ws = synth.make_mxfp4_weights(K, N, seed=6)
    xq0, xs0 = omx.quantize_rows(omx_bits_to_float(bits, "bf16"))
    p = synth.ProblemMX(M, K, N, xq0, xs0, qw, ws)
    d = OnDeviceMX(p)
    X = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    say("mxfp4 chain")
    xq, xs = d.mx.mxfp4_quantize_rows(X)
    Y = d.gemm("bf16", xq=xq, xs=xs)
    _, y, B = omx.gemm(xq0, xs0, qw, ws, M, N, K, "bf16")
    assert_close(y_float(Y), y, B, "bf16", "chain")


@pytest.mark.parametrize("name", sorted(synth.MXFP4_WORKLOADS))
def test_full_size_workload(name):
    cfg = synth.MXFP4_WORKLOADS[name]
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    say(f"mxfp4 full size {name}")
    p = synth.make_mxfp4_problem(seed=0, **cfg)
    d = OnDeviceMX(p)
    Yg = y_float(d.gemm("fp16"))
    if M <= 128:
        _, y, B = omx.gemm(p.xq, p.xs, p.qweight, p.ws, M, N, K, "fp16")
        assert_close(Yg, y, B, "fp16", name)
        return
    rng = np.random.default_rng(2)
    rows = np.sort(rng.choice(M, 64, replace=False))
    cols = np.sort(rng.choice(N, 256, replace=False))
    _, y, B = omx.gemm_rows_cols(p.xq, p.xs, p.qweight, p.ws, M, N, K, rows, np.arange(N))
    assert_close(Yg[rows], y, B, "fp16", name + " rows")
    _, y, B = omx.gemm_rows_cols(p.xq, p.xs, p.qweight, p.ws, M, N, K, np.arange(M), cols)
    assert_close(Yg[:, cols], y, B, "fp16", name + " cols")
