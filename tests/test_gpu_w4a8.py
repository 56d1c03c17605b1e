"""GPU parity of the W4A8 route (include/w4a8.h) against the CPU oracle
(oracle/w4a8.py), through the C ABI.

Bar:
  * bit-exact: the int8 weights of a blob (w4a8_dequant), the int8
    activations and their fp32 row scales (w4a8_quantize_rows), and the int32
    accumulators (W4A8_OUT_I32) -- all integer work, or decisions taken in
    fp32 on both sides;
  * fp16 / bf16 outputs: within one unit in the last place of the oracle's
    value.  The kernel's fp32 steps (int32 -> fp32, times sx, times sw) stay
    within 3 * 2^-24 relative of the exact product, far below half an ulp of
    either output dtype, so after one rounding the two sides can differ only
    where the exact value sits within that distance of a rounding boundary:
    by one ulp at most.
"""
import numpy as np
import pytest

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


def w8mod():
    from w4a16_dequant_gemm_amd import w4a8
    return w4a8


def check_shapes_w8(p):
    """Host-side check of the operand shapes the kernels assume, before a launch."""
    assert p.xq.shape == (p.M, p.K) and p.xq.dtype == np.int8
    assert p.sx.shape == (p.M,) and p.sx.dtype == np.float32
    assert p.qweight.shape == (p.K // 8, p.N) and p.qweight.dtype == np.uint32
    assert p.s8.shape == (p.K // p.G, p.N) and p.a.shape == (p.K // p.G, p.N)
    assert p.sw.shape == (p.N,) and p.sw.dtype == np.float32
    assert p.N % 128 == 0 and p.K % 256 == 0 and p.G in (32, 64, 128) and p.K <= 131072


class OnDeviceW8:
    def __init__(self, p):
        check_shapes_w8(p)
        self.w8 = w8mod()
        self.p = p
        d = "cuda"
        self.xq = torch.from_numpy(p.xq).to(d)
        self.sx = torch.from_numpy(p.sx).to(d)
        qw = torch.from_numpy(p.qweight.view(np.int32)).to(d)
        s8 = torch.from_numpy(p.s8).to(d)
        a = torch.from_numpy(p.a).to(d)
        sw = torch.from_numpy(p.sw).to(d)
        self.packed = self.w8.w4a8_repack(qw, s8, a, sw, p.K, p.N, p.G)

    def gemm(self, out, plan=None, xq=None, sx=None):
        Y = self.w8.w4a8_gemm(self.xq if xq is None else xq, self.sx if sx is None else sx,
                              self.packed, out=out, plan=plan)
        torch.cuda.synchronize()
        return Y


def to_np_bits(Y):
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def assert_within_one_ulp(got_bits, want_bits, dtype, what=""):
    g = o8.bits_to_float(got_bits, dtype)
    w = o8.bits_to_float(want_bits, dtype)
    both_inf = np.isinf(g) & np.isinf(w) & (np.sign(g) == np.sign(w))
    d = np.where(both_inf, 0.0, np.abs(g - w))
    u = o8.ulp(np.maximum(np.abs(g), np.abs(w)), dtype)
    bad = ~(d <= u)
    assert not np.any(bad), (f"{what}: {int(bad.sum())} outputs differ by more than one ulp, "
                             f"first at {np.argwhere(bad)[0]}: {g[bad][0]} vs {w[bad][0]}")
    return int(np.count_nonzero(got_bits != want_bits))


SHAPES = [  # (K, N, G)
    (256, 128, 32), (512, 384, 64), (1024, 256, 128), (768, 640, 128), (2048, 128, 32),
]


@pytest.mark.parametrize("K,N,G", SHAPES)
def test_dequant_bit_exact(K, N, G):
    say(f"w4a8 dequant K={K} N={N} G={G}")
    p = synth.make_w4a8_problem(1, K, N, G, seed=K + N + G)
    d = OnDeviceW8(p)
    W = d.w8.w4a8_dequant(d.packed)
    torch.cuda.synchronize()
    want = o8.weight_int8(p.qweight, p.s8, p.a, K, N, G)
    assert np.array_equal(W.cpu().numpy(), want)
    assert d.w8.trailer_flags(d.packed) == 0


def test_dequant_every_code_scale_offset():
    """Every (q, s8, a) of the format once: s8 0..16, a 0..255-15*s8, q 0..15."""
    cases = [(s, a) for s in range(17) for a in range(0, 256 - 15 * s)]
    N = 128
    G = 32
    ngroups = -(-len(cases) // N)
    ngroups += (-ngroups) % 8          # K = 32 * ngroups must be a multiple of 256
    K = G * ngroups
    s8 = np.zeros((ngroups, N), np.uint8)
    a = np.zeros((ngroups, N), np.uint8)
    for i, (s, off) in enumerate(cases):
        s8[i // N, i % N] = s
        a[i // N, i % N] = off
    q = ((np.arange(K)[:, None] + np.arange(N)[None, :]) % 16).astype(np.uint8)   # all codes per group
    qw = synth.pack_nibbles(q)
    sw = np.ones(N, np.float32)
    p = synth.ProblemW8(1, K, N, G, np.zeros((1, K), np.int8), np.ones(1, np.float32), qw, s8, a,
                        sw)
    say(f"w4a8 dequant exhaustive K={K} N={N}")
    d = OnDeviceW8(p)
    W = d.w8.w4a8_dequant(d.packed)
    torch.cuda.synchronize()
    assert np.array_equal(W.cpu().numpy(), o8.weight_int8(qw, s8, a, K, N, G))


def test_trailer_flags_a_group_outside_the_format():
    p = synth.make_w4a8_problem(1, 256, 128, 64, seed=3)
    s8 = p.s8.copy()
    a = p.a.copy()
    s8[2, 77] = 16
    a[2, 77] = 20                      # 20 + 15*16 = 260 > 255
    p2 = synth.ProblemW8(p.M, p.K, p.N, p.G, p.xq, p.sx, p.qweight, s8, a, p.sw)
    say("w4a8 trailer overflow flag")
    d = OnDeviceW8(p2)
    torch.cuda.synchronize()
    assert d.w8.trailer_flags(d.packed) & d.w8.W4A8_TRAILER_OVERFLOW


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("M,K", [(1, 256), (7, 1024), (33, 4096), (3, 8192)])
def test_quantize_rows_bit_exact(dtype, M, K):
    say(f"w4a8 quantize rows {dtype} M={M} K={K}")
    bits = synth.make_activations(M, K, dtype, seed=M * K, outlier_frac=0.001)
    if M > 2:
        bits[1, :] = 0                 # a row of zeros
        bits[2, :] = 0x8000            # a row of negative zeros
    x = o8.bits_to_float(bits, dtype)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    X = torch.from_numpy(bits.view(np.int16)).to("cuda").view(tdt)
    xq, sx = w8mod().w4a8_quantize_rows(X)
    torch.cuda.synchronize()
    want_q, want_s = o8.quantize_rows(x)
    assert np.array_equal(sx.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(xq.cpu().numpy(), want_q)


# (M, K, N, G, plan)
GEMM_CASES = [
    (1, 256, 128, 32, None), (1, 1024, 384, 128, None), (5, 2048, 256, 64, None),
    (17, 512, 128, 128, ("stream", 2)), (32, 1024, 256, 32, ("stream", 4)),
    (31, 2048, 128, 64, ("stream", 8)), (33, 512, 384, 128, None), (64, 1024, 256, 64, None),
    (64, 768, 128, 32, ("stream", 8)), (3, 512, 384, 128, "tiled"),
    (65, 512, 384, 128, None), (100, 1024, 256, 32, None), (130, 768, 640, 64, None),
    (300, 512, 128, 128, None), (513, 1024, 384, 128, None), (600, 256, 256, 32, None),
    (1000, 512, 640, 64, None), (200, 512, 384, 32, ("tiled", 3)),
    (40, 1024, 640, 64, ("tiled", 1)), (130, 512, 384, 128, ("tiled", 2)),
    (257, 768, 128, 64, ("tiled", 1)), (48, 512, 256, 64, ("stream", 2)),
    (600, 512, 384, 128, ("tiled", 4)), (300, 768, 640, 32, ("tiled", 4)),
    (33, 1024, 128, 64, ("tiled", 4)), (300, 256, 384, 32, ("tiled", 5)),
    (600, 512, 640, 128, ("tiled", 5)),
    # the block-diagonal streaming form (M <= 4) with every parts count
    (2, 1024, 256, 64, ("stream", 2)), (4, 2048, 384, 32, ("stream", 8)),
    (3, 512, 128, 128, ("stream", 4)), (4, 8192, 128, 128, None),
]


@pytest.mark.parametrize("M,K,N,G,plan", GEMM_CASES)
def test_gemm_int32_bit_exact_and_scaled_outputs(M, K, N, G, plan):
    say(f"w4a8 gemm M={M} K={K} N={N} G={G} plan={plan}")
    p = synth.make_w4a8_problem(M, K, N, G, seed=M * 7 + K + N + G)
    d = OnDeviceW8(p)
    _, acc = o8.gemm(p.xq, p.sx, p.qweight, p.s8, p.a, p.sw, M, N, K, G, "i32")
    Yi = d.gemm("i32", plan=plan).cpu().numpy()
    assert np.array_equal(Yi.astype(np.int64), acc)
    for dt in ("fp16", "bf16"):
        Yref = o8.scale_output(acc, p.sx, p.sw, dt)
        Yg = to_np_bits(d.gemm(dt, plan=plan))
        assert_within_one_ulp(Yg, Yref, dt, f"M={M} {dt}")


def test_stream_and_tiled_agree_bitwise():
    M, K, N, G = 48, 2048, 384, 128
    p = synth.make_w4a8_problem(M, K, N, G, seed=21)
    d = OnDeviceW8(p)
    say("w4a8 stream vs tiled")
    outs = [to_np_bits(d.gemm("fp16", plan=pl)) for pl in
            (("stream", 2), ("stream", 4), ("stream", 8), "tiled")]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_chain_quantize_then_gemm():
    """fp16 activations -> per-row int8 -> W4A8 GEMM, against the oracle chain."""
    M, K, N, G = 20, 4096, 512, 128
    bits = synth.make_activations(M, K, "fp16", seed=4, outlier_frac=0.001)
    qw, s8, a, sw = synth.make_w4a8_weights(K, N, G, seed=4)
    xq0, sx0 = o8.quantize_rows(o8.bits_to_float(bits, "fp16"))
    p = synth.ProblemW8(M, K, N, G, xq0, sx0, qw, s8, a, sw)
    d = OnDeviceW8(p)
    X = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.float16)
    say("w4a8 chain")
    xq, sx = d.w8.w4a8_quantize_rows(X)
    Y = d.gemm("fp16", xq=xq, sx=sx)
    Yref, _ = o8.gemm(xq0, sx0, qw, s8, a, sw, M, N, K, G, "fp16")
    assert_within_one_ulp(to_np_bits(Y), Yref, "fp16", "chain")


@pytest.mark.parametrize("name", sorted(synth.W4A8_WORKLOADS))
def test_full_size_workload(name):
    """The benchmark workloads at full size: every output for M <= 128; for
    the prefill, 64 whole rows and 256 whole columns."""
    cfg = synth.W4A8_WORKLOADS[name]
    M, K, N, G = cfg["M"], cfg["K"], cfg["N"], cfg["G"]
    say(f"w4a8 full size {name}")
    p = synth.make_w4a8_problem(seed=0, **cfg)
    d = OnDeviceW8(p)
    Yi = d.gemm("i32").cpu().numpy().astype(np.int64)
    Yg = to_np_bits(d.gemm("fp16"))
    w8 = o8.weight_int8(p.qweight, p.s8, p.a, K, N, G)
    if M <= 128:
        acc = o8.accumulate(p.xq, w8)
        assert np.array_equal(Yi, acc)
        assert_within_one_ulp(Yg, o8.scale_output(acc, p.sx, p.sw, "fp16"), "fp16", name)
        return
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(M, 64, replace=False))
    cols = np.sort(rng.choice(N, 256, replace=False))
    acc_r = o8.accumulate(p.xq[rows], w8)
    assert np.array_equal(Yi[rows], acc_r)
    assert_within_one_ulp(Yg[rows], o8.scale_output(acc_r, p.sx[rows], p.sw, "fp16"), "fp16",
                          name + " rows")
    acc_c = o8.accumulate(p.xq, np.ascontiguousarray(w8[:, cols]))
    assert np.array_equal(Yi[:, cols], acc_c)
    assert_within_one_ulp(Yg[:, cols], o8.scale_output(acc_c, p.sx, p.sw[cols], "fp16"), "fp16",
                          name + " cols")


def test_back_to_back_and_reuse():
    """Two calls of different M on one blob, then the first again: same bits."""
    M, K, N, G = 80, 1024, 256, 64
    p = synth.make_w4a8_problem(M, K, N, G, seed=30)
    d = OnDeviceW8(p)
    say("w4a8 back to back")
    y1 = to_np_bits(d.gemm("bf16"))
    y2 = to_np_bits(d.gemm("bf16", xq=d.xq[:7].contiguous(), sx=d.sx[:7].contiguous()))
    y3 = to_np_bits(d.gemm("bf16"))
    assert np.array_equal(y1, y3)
    # other kernel, same exact integer sums and the same fp32 epilogue: same bits
    assert np.array_equal(y2, y1[:7])
    _, acc = o8.gemm(p.xq[:7], p.sx[:7], p.qweight, p.s8, p.a, p.sw, 7, N, K, G, "i32")
    assert_within_one_ulp(y2, o8.scale_output(acc, p.sx[:7], p.sw, "bf16"), "bf16", "M=7")


def test_largest_k_extreme_sum():
    """K = 131072 with xq = -127 and every weight -128 (q = 0, a = 0): the
    largest sum the format allows, 127 * 128 * K < 2^31, exact in int32."""
    M, K, N, G = 2, 131072, 128, 128
    xq = np.full((M, K), -127, np.int8)
    xq[1, ::2] = 127
    qw = np.zeros((K // 8, N), np.uint32)
    s8 = np.full((K // G, N), 16, np.uint8)
    a = np.zeros((K // G, N), np.uint8)
    p = synth.ProblemW8(M, K, N, G, xq, np.ones(M, np.float32), qw, s8, a, np.ones(N, np.float32))
    say("w4a8 extreme sum K=131072")
    d = OnDeviceW8(p)
    Yi = d.gemm("i32").cpu().numpy().astype(np.int64)
    assert np.all(Yi[0] == 127 * 128 * K) and np.all(Yi[1] == 0)
