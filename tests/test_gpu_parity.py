"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar: bit-exact for unpacked/dequantized weights (and the repack round trip);
max |Y - Y_ref| / B <= 2e-3 (fp16) or 1e-2 (bf16) for the product, with
B = sum_k |X||deq| and Y == 0 wherever B == 0.
"""
import numpy as np
import pytest

import oracle
import w4a16_synth as synth
from gpu_helpers import (OnDevice, assert_gemm_close, column_slice, lib, same_bits, say)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    lib()


# ---------------------------------------------------------------------------
# operand layout of v_mfma_f32_32x32x16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_mfma_operand_layout(dtype):
    """Random small integers (exact in both formats): D == A.B exactly; also
    one-hot A rows and B columns, so a swapped row/column/k placement fails."""
    w4 = lib()
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    flags = w4.W4A16_BF16 if dtype == "bf16" else 0
    rng = np.random.default_rng(0)
    cases = [(rng.integers(-4, 5, (32, 16)), rng.integers(-4, 5, (16, 32)))]
    for i in range(4):
        A = np.zeros((32, 16))
        B = np.zeros((16, 32))
        A[np.arange(32), (np.arange(32) * 3 + i) % 16] = np.arange(1, 33)
        B[np.arange(16), (np.arange(16) * 5 + i) % 32] = 1 + np.arange(16) / 16
        cases.append((A, B))
    for A, B in cases:
        say(f"mfma probe {dtype}")
        Ad = torch.tensor(A, dtype=tdt, device="cuda").contiguous()
        Bd = torch.tensor(B, dtype=tdt, device="cuda").contiguous()
        D = w4.w4a16_mfma_layout_probe(Ad, Bd, flags)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(D.cpu().numpy(), (A @ B).astype(np.float32))


# ---------------------------------------------------------------------------
# repack, dequant
# ---------------------------------------------------------------------------

SHAPES = [  # (K, N, G, dtype, sym)
    (256, 128, 128, "fp16", False),
    (512, 384, 64, "bf16", False),
    (256, 256, 32, "fp16", True),
    (768, 640, 32, "bf16", True),
    (1024, 512, 128, "bf16", False),
]


@pytest.mark.parametrize("K,N,G,dtype,sym", SHAPES)
def test_repack_round_trip(K, N, G, dtype, sym):
    w4 = lib()
    p = synth.make_problem(1, K, N, G=G, dtype=dtype, sym=sym, seed=K + N)
    say(f"repack round trip K={K} N={N} G={G} {dtype} sym={sym}")
    d = OnDevice(p)
    qw, sc, zr = w4.w4a16_unrepack(d.packed)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(qw.cpu().numpy().view(np.uint32), p.qweight)
    np.testing.assert_array_equal(w4.bits_of(sc), p.scales)
    if sym:
        assert zr is None
    else:
        np.testing.assert_array_equal(zr.cpu().numpy(), p.zeros)


@pytest.mark.parametrize("K,N,G,dtype,sym", SHAPES)
def test_dequant_bit_exact(K, N, G, dtype, sym):
    w4 = lib()
    p = synth.make_problem(1, K, N, G=G, dtype=dtype, sym=sym, seed=7 * K + N)
    say(f"dequant K={K} N={N} G={G} {dtype} sym={sym}")
    d = OnDevice(p)
    got = w4.bits_of(w4.w4a16_dequant(d.packed))
    want = oracle.dequant(p.qweight, p.scales, p.zeros, K, N, G, dtype, sym)
    assert same_bits(got, want)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_dequant_exhaustive_scales(dtype):
    """Every (q, z) pair with every non-negative finite scale pattern (subnormals
    included), through the library's device dequantization."""
    w4 = lib()
    G, N = 32, 4096
    scales_all = np.arange(0, 0x7C00 if dtype == "fp16" else 0x7F80, dtype=np.uint16)
    combos = 16 * scales_all.size                      # (z, s) pairs
    per_body = 256 // G                                # K must be a multiple of 256
    NG = -(-combos // (N * per_body)) * per_body
    K = NG * G
    zs = np.repeat(np.arange(16, dtype=np.uint8), scales_all.size)
    ss = np.tile(scales_all, 16)
    pad = NG * N - combos
    zs = np.concatenate([zs, np.zeros(pad, np.uint8)]).reshape(NG, N)
    ss = np.concatenate([ss, np.full(pad, 0x3C00 if dtype == "fp16" else 0x3F80, np.uint16)])
    ss = ss.reshape(NG, N)
    q = np.tile((np.arange(K) % 16).astype(np.uint8)[:, None], (1, N))   # every q in each group
    p = synth.Problem(1, K, N, G, dtype, False, np.zeros((1, K), np.uint16),
                      synth.pack_nibbles(q), ss, zs)
    say(f"exhaustive dequant {dtype} K={K} N={N}")
    d = OnDevice(p)
    got = w4.bits_of(w4.w4a16_dequant(d.packed))
    want = oracle.dequant(p.qweight, p.scales, p.zeros, K, N, G, dtype, False)
    g0 = np.where(got == 0x8000, 0, got)
    w0 = np.where(want == 0x8000, 0, want)
    bad = np.argwhere(g0 != w0)
    if bad.size:
        rows = []
        for k, n in bad[:12]:
            rows.append(f"q={k % 16} z={zs[k // G, n]} s=0x{int(ss[k // G, n]):04X} "
                        f"got=0x{int(got[k, n]):04X} want=0x{int(want[k, n]):04X}")
        svals = np.unique(ss[bad[:, 0] // G, bad[:, 1]])
        pytest.fail(f"{len(bad)} mismatches; scale patterns 0x{int(svals.min()):04X}.."
                    f"0x{int(svals.max()):04X} ({svals.size} distinct); first: " + "; ".join(rows))


# ---------------------------------------------------------------------------
# the fused product
# ---------------------------------------------------------------------------

def one_hot_rows(M, K, dtype):
    one = 0x3C00 if dtype == "fp16" else 0x3F80
    ks = (np.arange(M) * 37 + 5) % K
    X = np.zeros((M, K), dtype=np.uint16)
    X[np.arange(M), ks] = one
    return X, ks


@pytest.mark.parametrize("variant,M", [("decode", 1), ("decode", 8), ("decode", 5),
                                       ("splitk", 1), ("splitk", 7), ("splitk", 32),
                                       ("wide", 33), ("wide", 64), ("wide", 100), ("wide", 128),
                                       ("tiled", 20), ("tiled", 64), ("tiled", 130)])
@pytest.mark.parametrize("K,N,G,dtype,sym", [(512, 384, 128, "fp16", False),
                                             (256, 256, 32, "bf16", False),
                                             (768, 640, 64, "fp16", True)])
def test_gemm_one_hot_rows_are_dequantized_weights(variant, M, K, N, G, dtype, sym):
    """X = rows of the identity: Y[m] must equal deq[k_m] bit for bit, through the
    real GEMM kernels (one exact product, fp32 sums of zeros)."""
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=M + K)
    p.X, ks = one_hot_rows(M, K, dtype)
    say(f"one-hot {variant} M={M} K={K} N={N} G={G} {dtype} sym={sym}")
    d = OnDevice(p)
    Y = d.w4.bits_of(d.gemm(plan=variant))
    deq = oracle.dequant(p.qweight, p.scales, p.zeros, K, N, G, dtype, sym)
    assert same_bits(Y, deq[ks])


@pytest.mark.parametrize("variant,M", [("decode", 3), ("splitk", 3), ("wide", 70), ("tiled", 70)])
def test_gemm_exact_bf16_form_for_huge_scales(variant, M):
    """bf16 scales so large that -z*s overflows fp32 (z = 15, s near 2^125) while
    every (q - z) * s stays finite (q in {14, 15}): the repack flags the blob and
    both kernels must still return the dequantized weights bit for bit."""
    w4 = lib()
    K, N, G = 512, 256, 64
    rng = np.random.default_rng(M)
    q = rng.integers(14, 16, size=(K, N)).astype(np.uint8)
    scales = rng.integers(0x7E00, 0x7E80, size=(K // G, N)).astype(np.uint16)   # 2^125..2^126
    zeros = np.full((K // G, N), 15, dtype=np.uint8)
    X, ks = one_hot_rows(M, K, "bf16")
    p = synth.Problem(M, K, N, G, "bf16", False, X, synth.pack_nibbles(q), scales, zeros)
    say(f"exact bf16 form {variant} M={M}")
    d = OnDevice(p)
    flags_word = int(d.packed.data[-8:-4].view(torch.int32).cpu()[0])
    assert flags_word & 1, "repack did not flag the blob"
    Y = w4.bits_of(d.gemm(plan=variant))
    deq = oracle.dequant(p.qweight, p.scales, p.zeros, K, N, G, "bf16", False)
    assert same_bits(Y, deq[ks])
    assert same_bits(w4.bits_of(w4.w4a16_dequant(d.packed)), deq)


SMALL = [  # (K, N, G, dtype, sym)
    (256, 256, 128, "fp16", False),
    (512, 384, 32, "bf16", True),
    (768, 128, 64, "bf16", False),
    (1280, 512, 32, "fp16", False),
    (2048, 640, 128, "fp16", True),
]


@pytest.mark.parametrize("K,N,G,dtype,sym", SMALL)
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 13, 16, 17, 31, 32, 33, 47, 64, 65, 100, 128, 129, 200])
def test_gemm_matches_oracle(M, K, N, G, dtype, sym):
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=3 * M + K, outlier_frac=0.01)
    say(f"gemm M={M} K={K} N={N} G={G} {dtype} sym={sym}")
    d = OnDevice(p)
    Yg = d.y_float(d.gemm())
    Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, sym)
    assert_gemm_close(p, Yg, Yref, B, f"M={M}")


@pytest.mark.parametrize("variant,M,param", [("decode", 1, 1), ("decode", 5, 3), ("decode", 8, 7),
                                             ("decode", 6, 2), ("decode", 2, 255), ("decode", 3, 16),
                                             ("splitk", 4, 1), ("splitk", 4, 3), ("splitk", 30, 16),
                                             ("splitk", 1, 7), ("splitk", 9, 100), ("splitk", 2, 255),
                                             ("wide", 48, 1), ("wide", 64, 3), ("wide", 70, 16),
                                             ("wide", 128, 255), ("wide", 40, 255),
                                             ("tiled", 8, 1), ("tiled", 32, 2), ("tiled", 96, 5),
                                             ("tiled", 200, 16)])
def test_gemm_forced_variant_and_param(variant, M, param):
    """Forced kernel and work split.  decode: `param` workgroups share the 20
    output tiles (1 = one workgroup runs every item in turn, so the item slots
    are reused many times; 3, 7, 16: left-over tiles split along K in two
    halves, the split items first; 255: every tile in two halves); split-K:
    8*param workgroups (2040 = more than there are batches); wide: `param`
    workgroups (1 and 3: every block in turn; 16 and 255: each of the five
    blocks' K split into parts that meet in the workspace); tiled: `param`
    K-splits."""
    K, N, G = 4096, 640, 64
    p = synth.make_problem(M, K, N, G=G, dtype="bf16", sym=False, seed=M)
    say(f"forced {variant} param={param} M={M}")
    d = OnDevice(p)
    Y1 = d.gemm(plan=(variant, param))
    Y2 = d.gemm(plan=(variant, param))
    Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, "bf16", False)
    assert_gemm_close(p, d.y_float(Y1), Yref, B, f"{variant} param={param}")
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16)), "not bitwise reproducible"


def test_workspace_counters_return_to_zero():
    """Calls of different shapes share one workspace; every result stays right and
    the counters are zero after each call."""
    w4 = lib()
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    # shapes whose tile counts differ, in an order where a later call has more
    # tiles than an earlier one wrote partial sums for
    for i, (M, K, N, var) in enumerate([(1, 8192, 1024, "splitk"), (9, 2048, 512, "splitk"),
                                        (40, 4096, 1024, "tiled"), (3, 8192, 1024, "splitk"),
                                        (70, 8192, 384, "tiled"), (2, 8192, 4096, "splitk"),
                                        (1, 4096, 256, "splitk"), (5, 8192, 8192, "splitk"),
                                        (1, 4096, 1024, ("decode", 255)),
                                        (8, 8192, 2048, ("decode", 255)),
                                        (64, 4096, 512, "wide"), (100, 2048, 1024, "wide"),
                                        (4, 2048, 512, "splitk")]):
        p = synth.make_problem(M, K, N, G=128, seed=i)
        say(f"workspace reuse call {i}: M={M} K={K} N={N} {var}")
        need = w4.w4a16_workspace_bytes(M, N, K, 128, w4.plan_flags(var))
        assert need > 0
        d = OnDevice(p)
        Y = w4.w4a16_gemm(d.X, d.packed, workspace=ws, plan=var)
        torch.cuda.synchronize()
        Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, 128, "fp16", False)
        assert_gemm_close(p, d.y_float(Y), Yref, B, f"call {i}")
        # counter area: the first 64 KiB of every workspace, all zero between calls
        assert int(ws[:65536].count_nonzero()) == 0, "counters not reset"


# ---------------------------------------------------------------------------
# full-size workloads (sampled outputs)
# ---------------------------------------------------------------------------

_weights = {}


def full_problem(name):
    cfg = dict(synth.WORKLOADS[name])
    key = (cfg["K"], cfg["N"], cfg["G"], cfg["dtype"], cfg["sym"])
    if key not in _weights:
        _weights.clear()
        _weights[key] = synth.make_weights(cfg["K"], cfg["N"], cfg["G"], cfg["dtype"], cfg["sym"], 0)
    qw, sc, zr, _ = _weights[key]
    X = synth.make_activations(cfg["M"], cfg["K"], cfg["dtype"], 0, cfg.get("outlier_frac", 0.0))
    return synth.Problem(cfg["M"], cfg["K"], cfg["N"], cfg["G"], cfg["dtype"], cfg["sym"], X, qw,
                         sc, zr)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_full_size_workload(name):
    """Launch configuration of the benchmark at the workload's real size.  Up to
    M = 128 every output element is compared with the oracle; above, rows are
    sampled (the prefill test below covers those shapes densely).  One
    128-column slice of the dequantized weights is compared bit for bit."""
    w4 = lib()
    p = full_problem(name)
    say(f"full-size {name}: M={p.M} K={p.K} N={p.N} G={p.G} {p.dtype} sym={p.sym}")
    d = OnDevice(p)
    Y = d.gemm()
    rng = np.random.default_rng(1)
    if p.M <= 128:
        Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, p.M, p.N, p.K, p.G, p.dtype,
                              p.sym)
        assert_gemm_close(p, d.y_float(Y), Yref, B, name)
    else:
        n_s = 384
        ms = np.concatenate([rng.integers(0, p.M, n_s), np.full(32, p.M - 1), np.zeros(32, int)])
        ns = np.concatenate([rng.integers(0, p.N, n_s), rng.integers(0, p.N, 32),
                             np.arange(32) + p.N - 32])
        Yref, B = oracle.gemm_at(p.X, p.qweight, p.scales, p.zeros, p.M, p.N, p.K, p.G, p.dtype,
                                 p.sym, ms, ns)
        assert_gemm_close(p, d.y_float(Y)[ms, ns], Yref, B, name)
    # dequant: one column block, bit-exact
    nb = int(rng.integers(0, p.N // 128))
    cols = np.arange(nb * 128, nb * 128 + 128)
    deq = w4.w4a16_dequant(d.packed)
    torch.cuda.synchronize()
    got = w4.bits_of(deq[:, nb * 128: nb * 128 + 128])
    del deq
    sl = column_slice(p, cols)
    want = oracle.dequant(sl.qweight, sl.scales, sl.zeros, p.K, 128, p.G, p.dtype, p.sym)
    assert same_bits(got, want)


@pytest.mark.parametrize("M,dtype,sym", [(3, "fp16", False), (8, "bf16", True), (8, "fp16", False)])
def test_full_size_ffn_down_small_m(M, dtype, sym):
    """The FFN-down shape (K = 28672, N = 8192) at decode M: X does not fit the
    decode kernel's LDS, so the default plan runs the split-K kernel's 8-row
    (block-diagonal 16x16x32) form; every output is compared with the oracle."""
    lib()
    K, N, G = 28672, 8192, 128
    p = synth.make_problem(M, K, N, G, dtype, sym, seed=11 + M, outlier_frac=0.001)
    say(f"full-size FFN-down M={M} {dtype} sym={sym}")
    d = OnDevice(p)
    Y = d.gemm()
    Yref, B = oracle.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, sym)
    assert_gemm_close(p, d.y_float(Y), Yref, B, f"FFN-down M={M}")


@pytest.mark.parametrize("nbytes", [1024, 3 * (1 << 20) + 5 * 1024, 117440512])
def test_read_probe_reads_every_byte_once(nbytes):
    """The read-bandwidth probe behind the benchmark's ceiling: XOR of its
    per-thread outputs equals the XOR of the buffer's 16-byte words."""
    w4 = lib()
    rng = np.random.default_rng(nbytes % 1000)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    say(f"read probe over {nbytes} bytes")
    out = w4.w4a16_read_probe(buf, nbytes)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    want = np.bitwise_xor.reduce(host.reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)


PREFILL = [n for n in synth.WORKLOADS if n.startswith("prefill_")]


@pytest.mark.parametrize("name", PREFILL)
def test_prefill_dense_samples(name):
    """Prefill at full size in the benchmark's launch configuration, against the
    oracle element by element: 64 random rows over every output column, and
    every row over 256 columns (the first 64, the last 64 and 128 random
    ones)."""
    p = full_problem(name)
    say(f"prefill dense samples {name}: M={p.M} K={p.K} N={p.N}")
    d = OnDevice(p)
    Y = d.gemm()
    Yb = d.w4.bits_of(Y)
    del Y
    rng = np.random.default_rng(7)
    rows = np.sort(rng.choice(p.M, 64, replace=False))
    Xr = np.ascontiguousarray(p.X[rows])
    Yref, B = oracle.gemm(Xr, p.qweight, p.scales, p.zeros, 64, p.N, p.K, p.G, p.dtype, p.sym)
    sub = synth.Problem(64, p.K, p.N, p.G, p.dtype, p.sym, Xr, p.qweight, p.scales, p.zeros)
    assert_gemm_close(sub, oracle.bits_to_float(Yb[rows], p.dtype), Yref, B, f"{name} rows")
    inner = rng.choice(np.arange(64, p.N - 64), 128, replace=False)
    cols = np.sort(np.concatenate([np.arange(64), np.arange(p.N - 64, p.N), inner]))
    sl = column_slice(p, cols)
    Yref, B = oracle.gemm(sl.X, sl.qweight, sl.scales, sl.zeros, p.M, sl.N, p.K, p.G, p.dtype,
                          p.sym)
    assert_gemm_close(sl, oracle.bits_to_float(Yb[:, cols], p.dtype), Yref, B, f"{name} cols")
