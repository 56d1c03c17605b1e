"""Pins of the W4A8 oracle (oracle/w4a8.py) to facts outside itself: the
hand-worked congruence table, the plain-integer reading of the congruence,
the W4A16 oracle's already pinned nibble order and rounding, numpy's float16
conversion, brute-force sums and closed forms.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import w4a8 as o8
import w4a16_synth as synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows():
    rows = []
    with open(os.path.join(GOLDEN, "w4a8_congruence.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            q, s, a, pre, post, v = line.split()
            rows.append((int(q), int(s), int(a), int(pre, 16), int(post, 16), int(v)))
    return rows


def _one_group(q, s, a):
    """A 1-column, 8-row problem whose group holds the code q everywhere."""
    qw = synth.pack_nibbles(np.full((8, 1), q, dtype=np.uint8))
    return qw, np.array([[s]], np.uint8), np.array([[a]], np.uint8)


def test_congruence_golden_table():
    rows = _golden_rows()
    assert len(rows) >= 10
    for q, s, a, pre, post, v in rows:
        assert (q * s + a) % 256 == pre          # the table's own arithmetic
        assert pre ^ 0x80 == post
        qw, s8, a8 = _one_group(q, s, a)
        w8 = o8.weight_int8(qw, s8, a8, 8, 1, 8)
        assert np.all(w8 == v), (q, s, a, w8[0, 0], v)


def test_congruence_is_offset_subtraction_inside_the_format():
    # Every (q, s8, a) of the format: the XOR reading equals q*s8 + a - 128.
    qs, ss, aa = [], [], []
    for s in range(0, 17):
        for a in range(0, 256 - 15 * s):
            for q in range(16):
                qs.append(q); ss.append(s); aa.append(a)
    n = len(qs)
    # one group of G = 8 per case: case j's code at row 8j, code 0 on the rest
    K2 = 8 * n
    q = np.zeros((K2, 1), np.uint8)
    q[0::8, 0] = qs
    s8 = np.array(ss, np.uint8).reshape(n, 1)
    a8 = np.array(aa, np.uint8).reshape(n, 1)
    w8 = o8.weight_int8(synth.pack_nibbles(q), s8, a8, K2, 1, 8).astype(np.int64)
    expect = np.array(qs) * np.array(ss) + np.array(aa) - 128
    assert np.array_equal(w8[0::8, 0], expect)
    assert np.array_equal(w8[1::8, 0], np.array(aa) - 128)
    assert not np.any(o8.overflow_groups(s8, a8))


def test_congruence_wraps_outside_the_format():
    rng = np.random.default_rng(5)
    n = 512
    q = rng.integers(0, 16, n)
    s = rng.integers(0, 256, n)
    a = rng.integers(0, 256, n)
    K2 = 8 * n
    qq = np.zeros((K2, 1), np.uint8)
    qq[0::8, 0] = q
    w8 = o8.weight_int8(synth.pack_nibbles(qq), s.astype(np.uint8).reshape(n, 1),
                        a.astype(np.uint8).reshape(n, 1), K2, 1, 8).astype(np.int64)
    # congruent to q*s + a - 128 modulo 256, and an int8
    assert np.all((w8[0::8, 0] - (q * s + a - 128)) % 256 == 0)
    assert w8.min() >= -128 and w8.max() <= 127
    bad = o8.overflow_groups(s.reshape(n, 1), a.reshape(n, 1))[:, 0]
    assert np.array_equal(bad, (s > 16) | (a + 15 * s > 255))


def test_unpack_matches_pinned_w4a16_oracle():
    rng = np.random.default_rng(1)
    K, N = 64, 24
    qw = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(o8.unpack(qw, K, N), oracle.unpack(qw, K, N))


def test_group_index_is_k_over_g():
    K, N, G = 256, 3, 64
    qw, s8, a, sw = synth.make_w4a8_weights(K, N, G, seed=2)
    base = o8.weight_int8(qw, s8, a, K, N, G)
    for g in range(K // G):
        a2 = a.copy()
        a2[g, 1] = (int(a2[g, 1]) + 1) % 256 if a2[g, 1] + 15 * s8[g, 1] < 255 else a2[g, 1] - 1
        w2 = o8.weight_int8(qw, s8, a2, K, N, G)
        diff = np.nonzero(np.any(w2 != base, axis=1))[0]
        assert diff.min() == g * G and diff.max() == g * G + G - 1
        assert np.array_equal(np.nonzero(np.any(w2 != base, axis=0))[0], [1])


def test_accumulate_brute_force():
    M, K, N, G = 3, 16, 5, 8
    p = synth.make_w4a8_problem(M, K, N, G, seed=3)
    w8 = o8.weight_int8(p.qweight, p.s8, p.a, K, N, G)
    acc = o8.accumulate(p.xq, w8)
    q = oracle.unpack(p.qweight, K, N)
    for m in range(M):
        for n in range(N):
            total = 0
            for k in range(K):
                g = k // G
                wv = int(q[k, n]) * int(p.s8[g, n]) + int(p.a[g, n]) - 128   # in-format reading
                total += int(p.xq[m, k]) * wv
            assert acc[m, n] == total


def test_accumulate_extremes_exact():
    # |xq| = 127 and w8 = -128 everywhere: the largest sum a K of 8192 can reach
    K, N = 8192, 2
    xq = np.full((1, K), -127, np.int8)
    w8 = np.full((K, N), -128, np.int8)
    assert np.all(o8.accumulate(xq, w8) == 127 * 128 * K)


def test_round_to_bits_fp16_matches_numpy():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                        [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 2.0 ** -25, 2.0 ** -24 * 1.5,
                         2.0 ** -24 * 2.5, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1e300]])
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(o8.round_to_bits(v, "fp16"), want)


def test_round_to_bits_bf16_matches_pinned_c_oracle():
    rng = np.random.default_rng(6)
    v = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 39, 3000))
    v += [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -133,
          2.0 ** -134, 3 * 2.0 ** -134, 3.3895313892515355e38, 3.39e38, 3.4e38, 1e300]
    v = np.array(v)
    got = o8.round_to_bits(v, "bf16")
    want = np.array([oracle.round_bf16(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_scale_output_exact_rational():
    # acc * sx * sw rounded once: compare with exact rationals rounded by hand
    rng = np.random.default_rng(7)
    acc = rng.integers(-2**28, 2**28, size=(4, 6))   # |Y| stays below the fp16 maximum
    sx = rng.uniform(1e-3, 2e-2, 4).astype(np.float32)
    sw = rng.uniform(5e-4, 5e-3, 6).astype(np.float32)
    y = o8.scale_output(acc, sx, sw, "fp16")
    for m in range(4):
        for n in range(6):
            exact = Fraction(int(acc[m, n])) * Fraction(float(sx[m])) * Fraction(float(sw[n]))
            got = Fraction(float(np.uint16(y[m, n]).view(np.float16)))
            # the nearest fp16 to the exact value (fp64 product error is far below half an ulp)
            u = Fraction(float(o8.ulp(np.array([float(exact)]), "fp16")[0]))
            assert abs(got - exact) <= u / 2 * (1 + Fraction(1, 2**20))


def test_gemm_at_equals_gemm_and_sign_symmetry():
    M, K, N, G = 5, 512, 64, 128
    p = synth.make_w4a8_problem(M, K, N, G, seed=8)
    for dt in ("fp16", "bf16", "i32"):
        Y, acc = o8.gemm(p.xq, p.sx, p.qweight, p.s8, p.a, p.sw, M, N, K, G, dt)
        ms = np.repeat(np.arange(M), N)
        ns = np.tile(np.arange(N), M)
        Ys, accs = o8.gemm_at(p.xq, p.sx, p.qweight, p.s8, p.a, p.sw, M, N, K, G, ms, ns, dt)
        assert np.array_equal(accs, acc.reshape(-1))
        if Y is not None:
            assert np.array_equal(Ys, Y.reshape(-1))
            # negating xq (|xq| <= 127, so exact) negates Y bit for bit (RNE is odd)
            Yn, _ = o8.gemm(-p.xq, p.sx, p.qweight, p.s8, p.a, p.sw, M, N, K, G, dt)
            nz = acc != 0
            assert np.array_equal(Yn[nz], Y[nz] ^ np.uint16(0x8000))


def test_gemm_zero_scale_closed_form():
    # s8 = 0: every weight of a group is a - 128, so the sum factors per group
    M, K, N, G = 2, 256, 32, 64
    p = synth.make_w4a8_problem(M, K, N, G, seed=9)
    s8 = np.zeros_like(p.s8)
    _, acc = o8.gemm(p.xq, p.sx, p.qweight, s8, p.a, p.sw, M, N, K, G, "i32")
    xs = p.xq.astype(np.int64).reshape(M, K // G, G).sum(axis=2)
    want = xs @ (p.a.astype(np.int64) - 128)
    assert np.array_equal(acc, want)


def test_quantize_rows_hand_worked():
    # amax 127 gives sx = 1 exactly, so xq is x rounded half to even
    x = np.array([[127.0, -2.5, 3.5, 0.49, -126.5, 0.5, -0.5, 1.5]])
    xq, sx = o8.quantize_rows(x)
    assert sx[0] == np.float32(1.0)
    assert xq.tolist() == [[127, -2, 4, 0, -126, 0, 0, 2]]
    z, sz = o8.quantize_rows(np.zeros((2, 16)))
    assert np.all(z == 0) and np.all(sz == 0)


def test_quantize_rows_invariants():
    bits = synth.make_activations(6, 1024, "fp16", seed=10, outlier_frac=0.01)
    x = oracle.bits_to_float(bits, "fp16")
    xq, sx = o8.quantize_rows(x)
    assert np.all(np.abs(xq.astype(int)) <= 127)
    assert np.all(np.max(np.abs(xq.astype(int)), axis=1) == 127)
    err = np.abs(x - xq.astype(np.float64) * sx.astype(np.float64)[:, None])
    assert np.all(err <= sx.astype(np.float64)[:, None] * (0.5 + 1e-5))
    # a constant multiple of a row scales sx and leaves xq unchanged (power of two)
    xq2, sx2 = o8.quantize_rows(x * 4.0)
    assert np.array_equal(xq2, xq) and np.array_equal(sx2, sx * np.float32(4.0))


def test_two_level_quantizer_stays_in_format():
    rng = np.random.default_rng(11)
    K, N, G = 512, 40, 128
    w = rng.standard_normal((K, N)) * 0.02
    w[:, 3] *= 50.0                        # a column of large weights
    w[::G, 7] = 0.5                        # groups with a far outlier
    qw, s8, a, sw, wi8 = o8.quantize_weights_two_level(w, G)
    assert s8.max() <= 16 and not np.any(o8.overflow_groups(s8, a))
    w8 = o8.weight_int8(qw, s8, a, K, N, G).astype(np.int64)
    s_rows = np.repeat(s8.astype(np.int64), G, axis=0)
    assert np.all(np.abs(w8 - wi8.astype(np.int64)) <= (s_rows + 1) // 2)
    # level 1 rounds by at most half a step of sw, level 2 by at most half of s8
    bound = ((s_rows + 1) // 2 + 0.5) * sw.astype(np.float64)[None, :] * (1 + 1e-6)
    assert np.all(np.abs(w8 * sw.astype(np.float64) - w) <= bound)
