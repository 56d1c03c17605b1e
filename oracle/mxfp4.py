"""CPU oracle for the MXFP4 route: block-scaled 4-bit weights (E2M1 with an
E8M0 scale per 32 reduction indices), block-scaled 8-bit activations (E4M3
with an E8M0 scale per 32), the product taken by the matrix unit itself.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and ``bench.py``'s CPU-baseline leg may import this module.  The GPU library
never calls it and it imports nothing from the GPU package.  Plain Python and
numpy, written as the definition.

What it computes
----------------
Page "量化开销对比：各家方案的矩阵乘账本与省账手段" (laojiahuo2003.github.io),
section 3, closing paragraph: MXFP4 puts the in-block scale into the
hardware -- blocks of 32 with an E8M0 (power-of-two) scale -- so a 4-bit
weight format can take route A again (section 1: the matrix unit consumes the
low-precision operands directly; no dequantisation to fp16 in between).  The
pages fix the block size and the scale type; the element formats and the
activation side are this module's reading (the plainest one the hardware
supports): weights are E2M1, activations are E4M3 with their own E8M0 block
scales, quantised per row at run time like the dynamic route of section 4.

  E2M1 code c (4 bits): sign c>>3, exponent e = (c>>1)&3, mantissa m = c&1;
      value = (-1)^s * (m/2 if e == 0 else (1 + m/2) * 2^(e-1)),
      i.e. the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
  E4M3 byte b (the variant with no infinities): sign b>>7, exponent
      e = (b>>3)&15, mantissa m = b&7; value = (-1)^s * (m/8 * 2^-6 if e == 0
      else (1 + m/8) * 2^(e-7)); the two bytes with e = 15, m = 7 are NaN;
      the largest finite magnitude is 448.
  E8M0 byte u: the scale 2^(u-127) (u = 255 is NaN; never produced here).

  Weights: w[k][n] = e2m1(q[k][n]) * 2^(ws[k/32][n] - 127), q packed 8 per
      uint32 like the other routes (nibble i of word [r][n] is k = 8r+i).
  Activations (quantise_rows): per row and block of 32 along k, amax = the
      largest |x|; the shared exponent is E = floor(log2 amax) - 8 (8 being
      E4M3's largest exponent), at least -127 (E = -127 for a block of
      zeros); xs = E + 127; each element is x * 2^-E rounded to the nearest
      E4M3 value, ties to the even code, magnitudes above 448 saturating to
      448.
  Product: Y[m][n] = RNE_dtype( sum over k of xa[m][k] * w[k][n] ), with
      xa = e4m3(xq) * 2^(xs - 127); every product is exact in fp64 (4 + 2
      significant bits) and the sum is a float64 library matmul, within
      about K * 2^-53 * B of the exact sum whatever its order.
      B[m][n] = sum of |xa| * |w|, the denominator of the error bound.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["e2m1_value", "e4m3_value", "E2M1_TABLE", "E4M3_TABLE", "nearest_e4m3",
           "nearest_e4m3_array",
           "quantize_rows", "weights", "activations", "gemm", "gemm_rows_cols"]


def e2m1_value(c: int) -> float:
    s = -1.0 if c & 8 else 1.0
    e = (c >> 1) & 3
    m = c & 1
    return s * (m / 2 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))


def e4m3_value(b: int) -> float:
    s = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 15
    m = b & 7
    if e == 15 and m == 7:
        return math.nan
    return s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)])
E4M3_TABLE = np.array([e4m3_value(b) for b in range(256)])
# the finite non-negative E4M3 values in increasing order, with their codes
_POS_CODES = np.array([b for b in range(0x7F)])          # 0x00 .. 0x7E, increasing value
_POS_VALS = E4M3_TABLE[_POS_CODES]


def nearest_e4m3(v: float) -> int:
    """The E4M3 code nearest to v, ties to the even code, |v| > 448 -> 448."""
    s = 0x80 if (v < 0 or (v == 0 and math.copysign(1.0, v) < 0)) else 0
    a = abs(v)
    if a >= 448.0:
        return s | 0x7E
    i = int(np.searchsorted(_POS_VALS, a))      # _POS_VALS[i-1] < a <= _POS_VALS[i]
    if _POS_VALS[i] == a:
        return s | int(_POS_CODES[i])
    lo, hi = i - 1, i
    dlo, dhi = a - _POS_VALS[lo], _POS_VALS[hi] - a
    if dlo < dhi:
        c = lo
    elif dhi < dlo:
        c = hi
    else:
        c = lo if _POS_CODES[lo] % 2 == 0 else hi
    return s | int(_POS_CODES[c])


def nearest_e4m3_array(v: np.ndarray) -> np.ndarray:
    """nearest_e4m3 over an array (the same rule, vectorised)."""
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), 448.0)
    i = np.clip(np.searchsorted(_POS_VALS, a), 1, len(_POS_VALS) - 1)
    lo, hi = i - 1, i
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[lo] % 2 == 1))
    c = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    c = np.where(a == 0.0, 0, c)
    return (c | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows(x: np.ndarray):
    """x [M][K] (exact values of the activation dtype, K % 32 == 0) ->
    (xq uint8 [M][K] E4M3 codes, xs uint8 [M][K/32] E8M0 scales)."""
    x = np.asarray(x, dtype=np.float64)
    M, K = x.shape
    blk = x.reshape(M, K // 32, 32)
    amax = np.max(np.abs(blk), axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))        # amax = f * 2^ex, 0.5 <= f < 1
    E = np.where(amax > 0, np.maximum(ex.astype(np.int64) - 1 - 8, -127), -127)
    xs = (E + 127).astype(np.uint8)
    scaled = np.ldexp(blk, (-E)[:, :, None].astype(np.int32))
    xq = nearest_e4m3_array(scaled).reshape(M, K)
    return xq, xs


def weights(qweight, ws, K: int, N: int) -> np.ndarray:
    """w [K][N] float64 from the E2M1 codes and the E8M0 block scales."""
    w = np.asarray(qweight, dtype=np.uint32).reshape(K // 8, N)
    q = np.empty((K, N), dtype=np.uint8)
    for i in range(8):
        q[i::8, :] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    scale = np.ldexp(1.0, np.asarray(ws, dtype=np.int64).reshape(K // 32, N) - 127)
    return E2M1_TABLE[q] * np.repeat(scale, 32, axis=0)


def activations(xq, xs, M: int, K: int) -> np.ndarray:
    scale = np.ldexp(1.0, np.asarray(xs, dtype=np.int64).reshape(M, K // 32) - 127)
    return E4M3_TABLE[np.asarray(xq, dtype=np.uint8).reshape(M, K)] * np.repeat(scale, 32, axis=1)


def _round_bits(y: np.ndarray, dtype: str) -> np.ndarray:
    from oracle import w4a8 as _w8     # the pinned round-to-nearest-even of the W4A8 oracle
    return _w8.round_to_bits(y, dtype)


def gemm(xq, xs, qweight, ws, M: int, N: int, K: int, dtype: str = "fp16"):
    """(Y bits uint16 [M][N], Y exact float64, B float64)."""
    xa = activations(xq, xs, M, K)
    w = weights(qweight, ws, K, N)
    y = xa @ w
    b = np.abs(xa) @ np.abs(w)
    return _round_bits(y, dtype), y, b


def gemm_rows_cols(xq, xs, qweight, ws, M: int, N: int, K: int, rows, cols, dtype="fp16"):
    """The product restricted to the given rows and columns."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    xa = activations(np.asarray(xq).reshape(M, K)[rows], np.asarray(xs).reshape(M, K // 32)[rows],
                     len(rows), K)
    w = weights(np.asarray(qweight).reshape(K // 8, N)[:, cols],
                np.asarray(ws).reshape(K // 32, N)[:, cols], K, len(cols))
    y = xa @ w
    return _round_bits(y, dtype), y, np.abs(xa) @ np.abs(w)
