"""Pins for the CPU oracle: checks it against facts fixed by the pages and by
mathematics, independently of its own code.

Each test names what it pins.  None of these needs a GPU.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden
import w4a16_synth as synth


# --------------------------------------------------------------------------
# independent helpers (written here, not taken from the oracle)
# --------------------------------------------------------------------------

def hex_nibbles(word: int):
    """Nibbles of a 32-bit word in k order: its hex digits read right to left."""
    return [int(c, 16) for c in reversed(f"{word:08x}")]


def frac_of_bits(bits: int, dtype: str) -> Fraction:
    """Exact value of an fp16/bf16 bit pattern, decoded by numpy."""
    if dtype == "fp16":
        return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))
    return Fraction(float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]))


def frac_rne(x: Fraction, dtype: str) -> Fraction:
    """Round a rational to the nearest fp16/bf16 value, ties to even (finite range only)."""
    mbits, emin = (10, -14) if dtype == "fp16" else (7, -126)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mbits)
    t = a / ulp
    fl = t.numerator // t.denominator
    rem = t - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def to_bits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Library RNE: numpy for fp16, torch (float32 -> bfloat16) for bf16."""
    if dtype == "fp16":
        return np.asarray(values, dtype=np.float64).astype(np.float16).view(np.uint16)
    f32 = torch.from_numpy(np.asarray(values, dtype=np.float64).astype(np.float32))
    return f32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def nonneg_finite_patterns(dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return np.arange(0, 0x7C00, dtype=np.uint16)          # +0 .. largest finite
    return np.arange(0, 0x7F80, dtype=np.uint16)


# --------------------------------------------------------------------------
# unpacking
# --------------------------------------------------------------------------

def test_unpack_golden_words(oracle_mod):
    """Hand-worked words: 8 nibbles per word, least significant first."""
    rows = read_golden("unpack_words.txt")
    words = np.array([int(r[0], 16) for r in rows], dtype=np.uint32)
    expect = np.array([[int(v) for v in r[1:]] for r in rows], dtype=np.uint8)   # [N][8]
    q = oracle_mod.unpack(words.reshape(1, -1), 8, len(words))                   # [8][N]
    np.testing.assert_array_equal(q.T, expect)


def test_unpack_matches_hex_decoder_and_layout(oracle_mod):
    """Random [K/8][N] words: q[k][n] is nibble k%8 of word [k/8][n] (hex-digit decoder)."""
    rng = np.random.default_rng(1)
    K, N = 24, 5
    qw = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32)
    q = oracle_mod.unpack(qw, K, N)
    for k in range(K):
        for n in range(N):
            assert q[k, n] == hex_nibbles(int(qw[k // 8, n]))[k % 8]


def test_pack_then_unpack_roundtrip(oracle_mod):
    """The generator's packing and the oracle's unpacking agree on every nibble."""
    p = synth.make_problem(3, 64, 48, G=32, keep_q=True, seed=5)
    np.testing.assert_array_equal(oracle_mod.unpack(p.qweight, 64, 48), p.q)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def test_decoders_match_numpy(oracle_mod):
    """Every fp16 and bf16 pattern decodes to the value numpy gives it."""
    lib = oracle_mod._load()
    allp = np.arange(65536, dtype=np.uint32)
    f16 = allp.astype(np.uint16).view(np.float16).astype(np.float64)
    bf16 = (allp << 16).view(np.float32).astype(np.float64)
    for b in range(0, 65536, 7):          # a spread covering all exponents
        a = lib.oracle_f16_to_double(b)
        c = lib.oracle_bf16_to_double(b)
        assert (a == f16[b]) or (np.isnan(a) and np.isnan(f16[b]))
        assert (c == bf16[b]) or (np.isnan(c) and np.isnan(bf16[b]))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_round_matches_library_on_values_and_ties(oracle_mod, dtype):
    """RNE to fp16/bf16 equals the library conversion on every representable value,
    every exact midpoint (ties) between neighbours, and random doubles."""
    pats = nonneg_finite_patterns(dtype)
    if dtype == "fp16":
        vals = pats.view(np.float16).astype(np.float64)
    else:
        vals = (pats.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2            # exact in float64
    rng = np.random.default_rng(2)
    rnd = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 12, 20000))
    xs = np.concatenate([vals, mids, -mids[::97], rnd])
    if dtype == "bf16":
        xs = xs[np.abs(xs) < 3e38]
        xs = xs.astype(np.float32).astype(np.float64)   # torch's path is from float32
    got = np.array([(oracle_mod.round_f16 if dtype == "fp16" else oracle_mod.round_bf16)(x)
                    for x in xs], dtype=np.uint16)
    np.testing.assert_array_equal(got, to_bits(xs, dtype))


def test_round_overflow_and_zero(oracle_mod):
    assert oracle_mod.round_f16(65504.0) == 0x7BFF
    assert oracle_mod.round_f16(65519.99) == 0x7BFF
    assert oracle_mod.round_f16(65520.0) == 0x7C00       # tie rounds to even = overflow
    assert oracle_mod.round_f16(-0.0) == 0x8000
    assert oracle_mod.round_f16(2.0 ** -25) == 0x0000    # tie between 0 and 2^-24 -> even 0
    assert oracle_mod.round_f16(3 * 2.0 ** -25) == 0x0002
    assert oracle_mod.round_bf16(1.0 + 2.0 ** -8) == 0x3F80   # tie -> even
    assert oracle_mod.round_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82


# --------------------------------------------------------------------------
# dequantization
# --------------------------------------------------------------------------

def test_dequant_golden_values(oracle_mod):
    """Hand-worked (q, z, s) -> deq bit patterns."""
    for dtype, q, z, s, expect in read_golden("dequant_values.txt"):
        got = oracle_mod.dequant_values(np.array([int(q)]), np.array([int(z)]),
                                        np.array([int(s, 16)]), dtype)[0]
        assert got == int(expect, 16), (dtype, q, z, s, hex(got), expect)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_dequant_exhaustive(oracle_mod, dtype):
    """All (q, z) in 16x16 times every non-negative finite scale pattern: the oracle
    equals the library's single RNE of the exact product (exact in float64)."""
    s = nonneg_finite_patterns(dtype)
    qz = np.arange(256)
    q = np.repeat((qz // 16).astype(np.uint8), s.size)
    z = np.repeat((qz % 16).astype(np.uint8), s.size)
    sb = np.tile(s, 256)
    got = oracle_mod.dequant_values(q, z, sb, dtype)
    sv = oracle_mod.bits_to_float(sb, dtype)
    exact = (q.astype(np.float64) - z.astype(np.float64)) * sv
    want = to_bits(exact, dtype)
    # a zero product may carry either sign; compare with -0 mapped to +0
    got = np.where(got == 0x8000, 0, got)
    want = np.where(want == 0x8000, 0, want)
    np.testing.assert_array_equal(got, want)


def test_exponent_bias_constants():
    """Closed forms behind the exponent-bias unpack: OR-ing a nibble into the
    fraction field of a float whose spacing is 1 gives that float plus the nibble.
    fp16: 0x6400|n = 1024 + n and 0x5400|(n<<4) = 64 + n; bf16: 0x4300|n = 128 + n."""
    n = np.arange(16, dtype=np.uint16)
    assert np.all((0x6400 | n).view(np.float16).astype(np.float64) == 1024 + n)
    assert np.all((0x5400 | (n << 4)).view(np.float16).astype(np.float64) == 64 + n)
    bf = ((0x4300 | n).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(bf == 128 + n)


def test_dequant_matrix_indexing(oracle_mod):
    """deq[k][n] uses nibble k%8 of word [k/8][n], scale and zero of group k//G
    (checked element by element with the hex decoder and Fraction rounding)."""
    for dtype, sym in (("fp16", False), ("bf16", False), ("fp16", True)):
        K, N, G = 32, 3, 8
        p = synth.make_problem(1, K, N, G=G, dtype=dtype, sym=sym, seed=11)
        deq = oracle_mod.dequant(p.qweight, p.scales, p.zeros, K, N, G, dtype, sym)
        for k in range(K):
            for n in range(N):
                q = hex_nibbles(int(p.qweight[k // 8, n]))[k % 8]
                z = 8 if sym else int(p.zeros[k // G, n])
                s = frac_of_bits(int(p.scales[k // G, n]), dtype)
                want = frac_rne((q - z) * s, dtype)
                assert frac_of_bits(int(deq[k, n]), dtype) == want


def test_scale_applied_per_group_before_sum(oracle_mod):
    """Two groups with different scales: Y must use each group's own scale inside the
    sum (a scale hoisted out of the sum over k gives another number)."""
    K, N, G = 16, 1, 8
    q = np.full((K, N), 9, dtype=np.uint8)                 # q - z = 1 everywhere
    qw = synth.pack_nibbles(q)
    zeros = np.full((2, 1), 8, dtype=np.uint8)
    scales = np.array([[0x3C00], [0x4000]], dtype=np.uint16)   # 1.0 and 2.0
    X = np.full((1, K), 0x3C00, dtype=np.uint16)               # ones
    Y, B = oracle_mod.gemm(X, qw, scales, zeros, 1, N, K, G, "fp16", False)
    assert Y[0, 0] == 8 * 1.0 + 8 * 2.0
    assert Y[0, 0] != 16 * 1.0 and Y[0, 0] != 16 * 2.0
    assert B[0, 0] == 24.0


# --------------------------------------------------------------------------
# the product
# --------------------------------------------------------------------------

def brute_force(p):
    """Exact rational Y and B from the definition, independent of the oracle."""
    Y = [[Fraction(0)] * p.N for _ in range(p.M)]
    Bd = [[Fraction(0)] * p.N for _ in range(p.M)]
    for n in range(p.N):
        col = []
        for k in range(p.K):
            q = hex_nibbles(int(p.qweight[k // 8, n]))[k % 8]
            z = 8 if p.sym else int(p.zeros[k // p.G, n])
            s = frac_of_bits(int(p.scales[k // p.G, n]), p.dtype)
            col.append(frac_rne((q - z) * s, p.dtype))
        for m in range(p.M):
            for k in range(p.K):
                x = frac_of_bits(int(p.X[m, k]), p.dtype)
                Y[m][n] += x * col[k]
                Bd[m][n] += abs(x) * abs(col[k])
    return Y, Bd


@pytest.mark.parametrize("M,K,N,G,dtype,sym", [
    (1, 16, 1, 8, "fp16", False),
    (2, 16, 3, 16, "fp16", False),
    (3, 32, 5, 8, "fp16", True),
    (3, 32, 4, 16, "bf16", False),
    (2, 16, 5, 8, "bf16", True),
])
def test_gemm_brute_force_fraction(oracle_mod, M, K, N, G, dtype, sym):
    """Tiny products against exact rational sums: |Y - exact| <= K * 2^-53 * B,
    and B equals its exact value to fp64 precision.  M, K, N all differ, so a
    transposed operand or a swapped index cannot pass."""
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=M * 100 + N)
    Y, B = oracle_mod.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, sym)
    Ye, Be = brute_force(p)
    for m in range(M):
        for n in range(N):
            bound = float(Be[m][n]) * K * 2.0 ** -53
            assert abs(Fraction(Y[m, n]) - Ye[m][n]) <= Fraction(bound) + Fraction(1, 2**1000)
            assert abs(B[m, n] - float(Be[m][n])) <= float(Be[m][n]) * K * 2.0 ** -53


def test_gemm_identity_dequantize_then_matmul(oracle_mod):
    """The fused per-element definition equals 'dequantize to an fp32 matrix, then a
    float64 matmul' (numpy) to within 1e-12 of the bound."""
    for dtype, sym, G in (("fp16", False, 128), ("bf16", True, 64), ("bf16", False, 32)):
        M, K, N = 7, 512, 96
        p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=sym, seed=3, outlier_frac=0.01)
        Y, B = oracle_mod.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, sym)
        W32 = oracle_mod.bits_to_float(
            oracle_mod.dequant(p.qweight, p.scales, p.zeros, K, N, G, dtype, sym),
            dtype).astype(np.float32)
        X64 = oracle_mod.bits_to_float(p.X, dtype)
        Ynp = X64 @ W32.astype(np.float64)
        assert np.max(np.abs(Y - Ynp) / B) <= 1e-12


def test_q_equal_z_contributes_nothing(oracle_mod):
    """q == z everywhere gives Y == 0; q == z in one group makes Y blind to X on
    that group's k-range (bitwise)."""
    M, K, N, G = 3, 256, 16, 64
    p = synth.make_problem(M, K, N, G=G, keep_q=True, seed=7)
    q_all = np.repeat(p.zeros, G, axis=0)                      # q[k][n] = z[k//G][n]
    Y0, B0 = oracle_mod.gemm(p.X, synth.pack_nibbles(q_all), p.scales, p.zeros,
                             M, N, K, G, "fp16", False)
    assert np.all(Y0 == 0.0) and np.all(B0 == 0.0)
    q = p.q.copy()
    q[G:2 * G, :] = q_all[G:2 * G, :]                          # group 1 only
    qw = synth.pack_nibbles(q)
    Ya, _ = oracle_mod.gemm(p.X, qw, p.scales, p.zeros, M, N, K, G, "fp16", False)
    X2 = p.X.copy()
    X2[:, G:2 * G] = synth.to_dtype_bits(np.random.default_rng(9).standard_normal((M, G)) * 50,
                                         "fp16")
    Yb, _ = oracle_mod.gemm(X2, qw, p.scales, p.zeros, M, N, K, G, "fp16", False)
    np.testing.assert_array_equal(Ya, Yb)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_sym_equals_asym_with_zero_eight(oracle_mod, dtype):
    M, K, N, G = 2, 256, 32, 128
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, sym=True, seed=4)
    z8 = np.full((K // G, N), 8, dtype=np.uint8)
    Ys, Bs = oracle_mod.gemm(p.X, p.qweight, p.scales, None, M, N, K, G, dtype, True)
    Ya, Ba = oracle_mod.gemm(p.X, p.qweight, p.scales, z8, M, N, K, G, dtype, False)
    np.testing.assert_array_equal(Ys, Ya)
    np.testing.assert_array_equal(Bs, Ba)


def test_integer_special_case_is_int64_matmul(oracle_mod):
    """G = K, s = 1, z = 0 and small-integer X: Y is the integer product X @ Q."""
    M, K, N = 4, 64, 8
    rng = np.random.default_rng(8)
    Xi = rng.integers(-20, 21, size=(M, K))
    Q = rng.integers(0, 16, size=(K, N))
    X = synth.to_dtype_bits(Xi.astype(np.float64), "fp16")
    scales = np.full((1, N), 0x3C00, dtype=np.uint16)
    zeros = np.zeros((1, N), dtype=np.uint8)
    Y, _ = oracle_mod.gemm(X, synth.pack_nibbles(Q), scales, zeros, M, N, K, K, "fp16", False)
    np.testing.assert_array_equal(Y, (Xi.astype(np.int64) @ Q.astype(np.int64)).astype(np.float64))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_doubling_scales_doubles_y(oracle_mod, dtype):
    M, K, N, G = 3, 256, 24, 32
    p = synth.make_problem(M, K, N, G=G, dtype=dtype, seed=6)
    s2 = synth.to_dtype_bits(oracle_mod.bits_to_float(p.scales, dtype) * 2.0, dtype)
    Y1, _ = oracle_mod.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, dtype, False)
    Y2, _ = oracle_mod.gemm(p.X, p.qweight, s2, p.zeros, M, N, K, G, dtype, False)
    np.testing.assert_array_equal(Y2, 2.0 * Y1)


def test_gemm_at_equals_full(oracle_mod):
    """The sampled form computes the same numbers as the full form, bitwise."""
    M, K, N, G = 5, 384, 40, 128
    p = synth.make_problem(M, K, N, G=G, seed=12, outlier_frac=0.01)
    Y, B = oracle_mod.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, "fp16", False)
    rng = np.random.default_rng(0)
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    Ys, Bs = oracle_mod.gemm_at(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, "fp16", False,
                                ms, ns)
    np.testing.assert_array_equal(Ys, Y[ms, ns])
    np.testing.assert_array_equal(Bs, B[ms, ns])


def test_dequant_rounding_share_is_small(oracle_mod):
    """Diagnostic relation: |Y - Y_unrounded| <= 2^-11 * B for fp16 (each weight moves
    by at most half an fp16 spacing)."""
    M, K, N, G = 4, 512, 32, 128
    p = synth.make_problem(M, K, N, G=G, seed=13)
    Y, B, Yx = oracle_mod.gemm(p.X, p.qweight, p.scales, p.zeros, M, N, K, G, "fp16", False,
                               with_exact=True)
    assert np.all(np.abs(Y - Yx) <= 2.0 ** -11 * B * (1 + 1e-9) + 1e-300)


def test_oracle_rejects_bad_shapes(oracle_mod):
    qw = np.zeros((1, 4), dtype=np.uint32)
    with pytest.raises(ValueError):
        oracle_mod.unpack(qw, 12, 4)           # K not a multiple of 8
    with pytest.raises(ValueError):
        oracle_mod.gemm(np.zeros((1, 8), np.uint16), qw, np.zeros((1, 4), np.uint16),
                        np.zeros((1, 4), np.uint8), 1, 4, 8, 3, "fp16", False)   # K % G
