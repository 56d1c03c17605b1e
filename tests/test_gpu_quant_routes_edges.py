"""Edge cases and HIP-graph capture of the W4A8 and MXFP4 routes, through the
C ABI: graph replays equal eager calls bit for bit (with eager work and
synchronisations between replays), all-zero activations give exact zeros,
one-hot activation rows reproduce the int8 weights exactly, a NaN in one MX
activation row stays in that row and a NaN MX weight scale in its column."""
import numpy as np
import pytest

from oracle import mxfp4 as omx
from oracle import w4a8 as o8
import w4a16_synth as synth
from gpu_helpers import lib, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lib()


def _w8(p):
    from w4a16_dequant_gemm_amd import w4a8 as w8
    d = "cuda"
    packed = w8.w4a8_repack(torch.from_numpy(p.qweight.view(np.int32)).to(d),
                            torch.from_numpy(p.s8).to(d), torch.from_numpy(p.a).to(d),
                            torch.from_numpy(p.sw).to(d), p.K, p.N, p.G)
    return w8, packed


def _mx(p):
    from w4a16_dequant_gemm_amd import mxfp4 as mx
    packed = mx.mxfp4_repack(torch.from_numpy(p.qweight.view(np.int32)).to("cuda"),
                             torch.from_numpy(p.ws).to("cuda"), p.K, p.N)
    return mx, packed


@pytest.mark.parametrize("M", [1, 24, 200])
def test_graph_replay_equals_eager(M):
    K, N, G = 1024, 256, 128
    p8 = synth.make_w4a8_problem(M, K, N, G, seed=M)
    w8, pk8 = _w8(p8)
    pm = synth.make_mxfp4_problem(M, K, N, seed=M)
    mx, pkm = _mx(pm)
    xq = torch.from_numpy(p8.xq).cuda()
    sx = torch.from_numpy(p8.sx).cuda()
    mq = torch.from_numpy(pm.xq).cuda()
    ms = torch.from_numpy(pm.xs).cuda()
    say(f"quant routes graph M={M}")
    Y8 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Ym = torch.empty((M, N), dtype=torch.float16, device="cuda")
    eager8 = w8.w4a8_gemm(xq, sx, pk8, out="bf16").clone()
    eagerm = mx.mxfp4_gemm(mq, ms, pkm, out="fp16").clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):      # warm up on the capture stream
        w8.w4a8_gemm(xq, sx, pk8, out="bf16", Y=Y8)
        mx.mxfp4_gemm(mq, ms, pkm, out="fp16", Y=Ym)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        w8.w4a8_gemm(xq, sx, pk8, out="bf16", Y=Y8)
        mx.mxfp4_gemm(mq, ms, pkm, out="fp16", Y=Ym)
    for r in range(3):
        Y8.zero_()
        Ym.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y8.view(torch.int16), eager8.view(torch.int16)), f"replay {r}"
        assert torch.equal(Ym.view(torch.int16), eagerm.view(torch.int16)), f"replay {r}"
        w8.w4a8_gemm(xq, sx, pk8, out="bf16")     # eager work between replays
        torch.cuda.synchronize()


def test_zero_activations_give_exact_zeros():
    M, K, N, G = 40, 512, 384, 64
    p8 = synth.make_w4a8_problem(M, K, N, G, seed=3)
    w8, pk8 = _w8(p8)
    z = torch.zeros((M, K), dtype=torch.int8, device="cuda")
    sx = torch.from_numpy(p8.sx).cuda()
    say("quant routes zero activations")
    assert torch.count_nonzero(w8.w4a8_gemm(z, sx, pk8, out="i32")) == 0
    Y = w8.w4a8_gemm(z, sx, pk8, out="fp16").view(torch.int16)
    assert torch.count_nonzero(Y & 0x7FFF) == 0
    pm = synth.make_mxfp4_problem(M, K, N, seed=3)
    mx, pkm = _mx(pm)
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    xq, xs = mx.mxfp4_quantize_rows(X)
    assert torch.count_nonzero(xq) == 0 and torch.count_nonzero(xs) == 0
    Ym = mx.mxfp4_gemm(xq, xs, pkm, out="bf16").view(torch.int16)
    assert torch.count_nonzero(Ym & 0x7FFF) == 0


def test_one_hot_rows_reproduce_int8_weights():
    """xq row m one-hot at k = k_m with value 1 and sx = sw = 1 (int32 output):
    row m of the product is row k_m of the int8 weights, exactly, on both kernels."""
    K, N, G = 768, 384, 32
    for M, plan in ((16, "stream"), (100, "tiled")):
        p = synth.make_w4a8_problem(M, K, N, G, seed=M)
        w8, pk = _w8(p)
        rng = np.random.default_rng(M)
        ks = rng.choice(K, M, replace=False)
        xq = np.zeros((M, K), np.int8)
        xq[np.arange(M), ks] = 1
        say(f"w4a8 one-hot rows M={M} plan={plan}")
        Y = w8.w4a8_gemm(torch.from_numpy(xq).cuda(), None, pk, out="i32",
                         plan=plan).cpu().numpy()
        w = o8.weight_int8(p.qweight, p.s8, p.a, K, N, G).astype(np.int64)
        assert np.array_equal(Y.astype(np.int64), w[ks])


@pytest.mark.parametrize("M,row", [(12, 5), (3, 1), (1, 0)])
def test_mx_nan_activation_stays_in_its_row(M, row):
    K, N = 512, 256
    p = synth.make_mxfp4_problem(M, K, N, seed=7)
    mx, pk = _mx(p)
    xq = p.xq.copy()
    xq[row, 100] = 0x7F                    # E4M3 NaN
    say(f"mxfp4 NaN row M={M}")
    Y = mx.mxfp4_gemm(torch.from_numpy(xq).cuda(), torch.from_numpy(p.xs).cuda(), pk,
                      out="fp16").float().cpu().numpy()
    Y0 = mx.mxfp4_gemm(torch.from_numpy(p.xq).cuda(), torch.from_numpy(p.xs).cuda(), pk,
                       out="fp16").float().cpu().numpy()
    assert np.all(np.isnan(Y[row]))
    others = np.arange(M) != row
    assert np.array_equal(Y[others], Y0[others])
    _, y, B = omx.gemm(p.xq, p.xs, p.qweight, p.ws, M, N, K, "fp16")
    assert np.max(np.abs(Y0 - y) / np.where(B > 0, B, 1)) <= 2e-3


@pytest.mark.parametrize("M", [1, 3, 12])
def test_mx_nan_weight_scale_stays_in_its_column(M):
    """An E8M0 NaN (0xFF) weight scale makes its own column NaN and no other:
    the repack flags it, and the small-M kernel then keeps each column's
    scales to itself."""
    K, N = 512, 256
    p = synth.make_mxfp4_problem(M, K, N, seed=8)
    mx, pk0 = _mx(p)
    ws = p.ws.copy()
    ws[3, 37] = 0xFF                       # block 3 of column 37
    pk = mx.mxfp4_repack(torch.from_numpy(p.qweight.view(np.int32)).to("cuda"),
                         torch.from_numpy(ws).to("cuda"), K, N)
    say(f"mxfp4 NaN weight scale M={M}")
    xq = torch.from_numpy(p.xq).cuda()
    xs = torch.from_numpy(p.xs).cuda()
    Y = mx.mxfp4_gemm(xq, xs, pk, out="fp16").float().cpu().numpy()
    Y0 = mx.mxfp4_gemm(xq, xs, pk0, out="fp16").float().cpu().numpy()
    assert np.all(np.isnan(Y[:, 37]))
    others = np.arange(N) != 37
    assert not np.any(np.isnan(Y[:, others]))
    assert np.array_equal(Y[:, others], Y0[:, others])
