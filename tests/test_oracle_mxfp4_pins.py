"""Pins of the MXFP4 oracle (oracle/mxfp4.py): the hand-worked format table,
brute-force nearest-value rounding, closed forms and brute-force sums.  CPU only."""
import math
import os
from fractions import Fraction

import numpy as np

from oracle import mxfp4 as mx
import w4a16_synth as synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_formats.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_formats_against_hand_worked_table():
    n = {"e2m1": 0, "e4m3": 0, "e8m0": 0, "mxq": 0}
    for row in _golden():
        kind = row[0]
        n[kind] += 1
        if kind == "e2m1":
            assert mx.e2m1_value(int(row[1])) == float(row[2])
        elif kind == "e4m3":
            v = mx.e4m3_value(int(row[1], 16))
            assert (math.isnan(v) and row[2] == "nan") or v == float(row[2]), row
        elif kind == "e8m0":
            assert math.ldexp(1.0, int(row[1]) - 127) == float(row[2])
            w = mx.weights(synth.pack_nibbles(np.full((32, 1), 2, np.uint8)),
                           np.array([[int(row[1])]], np.uint8), 32, 1)
            assert np.all(w == float(row[2]))            # code 2 is 1.0
        else:
            x = np.zeros((1, 32))
            x[0, 7] = float(row[1])
            q, s = mx.quantize_rows(x)
            assert s[0, 0] == int(row[2]) and q[0, 7] == int(row[3], 16), row
            assert np.all(np.delete(q[0], 7) == 0)
    assert all(v >= 3 for v in n.values())


def test_e4m3_table_shape():
    t = mx.E4M3_TABLE
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.count_nonzero(np.isfinite(t)) == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                  # codes 0..126 increase
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])   # sign bit
    assert pos.max() == 448.0 and pos[1] == 2.0 ** -9


def test_nearest_e4m3_brute_force():
    rng = np.random.default_rng(0)
    fin = np.array([b for b in range(256) if b not in (0x7F, 0xFF)])
    vals = mx.E4M3_TABLE[fin]
    v = np.concatenate([rng.standard_normal(3000) * 10.0 ** rng.integers(-4, 3, 3000),
                        # exact midpoints between neighbours (ties)
                        (np.sort(vals[vals > 0])[1:] + np.sort(vals[vals > 0])[:-1]) / 2,
                        [0.0, -0.0, 448.0, 460.0, 464.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -11]])
    got = mx.nearest_e4m3_array(v)
    for x, g in zip(v, got):
        assert mx.nearest_e4m3(float(x)) == g
        a = min(abs(x), 448.0)
        d = np.abs(np.abs(vals) - a)
        cand = fin[(d == d.min()) & ((fin & 0x80) == 0)]
        if len(cand) == 2:                           # a tie: the even code
            cand = cand[cand % 2 == 0]
        assert (g & 0x7F) == cand[0], (x, hex(g), cand)
        assert (g >> 7) == (1 if math.copysign(1.0, x) < 0 else 0)


def test_quantize_rows_invariants():
    bits = synth.make_activations(5, 512, "fp16", seed=3, outlier_frac=0.01)
    x = bits.view(np.float16).astype(np.float64)
    x[1, 32:64] = 0.0
    xq, xs = mx.quantize_rows(x)
    assert xs[1, 1] == 0 and np.all(xq[1, 32:64] == 0)
    xa = mx.activations(xq, xs, 5, 512)
    blk_max = np.repeat(np.max(np.abs(x.reshape(5, 16, 32)), axis=2), 32, axis=1)
    # every element within half an E4M3 step of its own binade (3 mantissa bits: 2^-4
    # relative), or at the saturated top of the block
    err = np.abs(xa - x)
    assert np.all((err <= np.abs(x) * 2.0 ** -4 + 2.0 ** -9 * np.repeat(
        np.ldexp(1.0, xs.astype(np.int64) - 127), 32, axis=1)) | (np.abs(xa) == 448 * np.repeat(
            np.ldexp(1.0, xs.astype(np.int64) - 127), 32, axis=1)))
    # the block maximum lands in [256, 448] after scaling
    sc = np.abs(xa[np.abs(x) == blk_max]) / np.repeat(np.ldexp(1.0, xs.astype(np.int64) - 127),
                                                       32, axis=1)[np.abs(x) == blk_max]
    assert np.all((sc[sc > 0] >= 256) & (sc[sc > 0] <= 448))
    # a power-of-two multiple of the input moves only the scales
    xq2, xs2 = mx.quantize_rows(x * 8.0)
    assert np.array_equal(xq2, xq)
    nz = np.max(np.abs(x.reshape(5, 16, 32)), axis=2) > 0
    assert np.array_equal(xs2[nz].astype(int), xs[nz].astype(int) + 3)


def test_gemm_brute_force_fractions():
    M, K, N = 3, 64, 5
    p = synth.make_mxfp4_problem(M, K, N, seed=4)
    Yb, y, B = mx.gemm(p.xq, p.xs, p.qweight, p.ws, M, N, K, "fp16")
    q = np.zeros((K, N), np.int64)
    for k in range(K):
        q[k] = (p.qweight[k // 8] >> np.uint32(4 * (k % 8))) & 0xF
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            babs = Fraction(0)
            for k in range(K):
                xa = Fraction(mx.e4m3_value(int(p.xq[m, k]))) * Fraction(2) ** (int(p.xs[m, k // 32]) - 127)
                wv = Fraction(mx.e2m1_value(int(q[k, n]))) * Fraction(2) ** (int(p.ws[k // 32, n]) - 127)
                tot += xa * wv
                babs += abs(xa * wv)
            assert abs(Fraction(y[m, n]) - tot) <= babs * Fraction(K, 2 ** 52)
            assert Fraction(B[m, n]) >= abs(tot)


def test_gemm_rows_cols_matches_gemm():
    M, K, N = 6, 256, 64
    p = synth.make_mxfp4_problem(M, K, N, seed=5)
    Yb, y, B = mx.gemm(p.xq, p.xs, p.qweight, p.ws, M, N, K, "bf16")
    rows, cols = [0, 3, 5], [1, 2, 40, 63]
    Yr, yr, Br = mx.gemm_rows_cols(p.xq, p.xs, p.qweight, p.ws, M, N, K, rows, cols, "bf16")
    assert np.allclose(yr, y[np.ix_(rows, cols)], rtol=0, atol=1e-12 * np.abs(B).max())
    # a block scale that doubles every weight of block 1 of column 2 changes only column 2
    ws2 = p.ws.copy()
    ws2[1, 2] += 1
    _, y2, _ = mx.gemm(p.xq, p.xs, p.qweight, ws2, M, N, K, "bf16")
    assert np.array_equal(np.delete(y2, 2, axis=1), np.delete(y, 2, axis=1))
    xa = mx.activations(p.xq, p.xs, M, K)
    w = mx.weights(p.qweight, p.ws, K, N)
    assert np.allclose(y2[:, 2] - y[:, 2], xa[:, 32:64] @ w[32:64, 2], rtol=1e-12, atol=0)
