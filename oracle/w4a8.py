"""CPU oracle for the W4A8 route: 4-bit weights, int8 activations, int8 MFMA.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and ``bench.py``'s CPU-baseline leg may import this module.  The GPU library
never calls it and it imports nothing from the GPU package.  Plain numpy,
written as the definition, with no blocking or reordering.

What it computes
----------------
Weights (page "W4A8量化计算优化：提升LLM推理效率的关键技术", section 2.1
"LiquidQuant的数学魔术").  A weight is a 4-bit code q (0..15); each group of
G consecutive reduction indices of one output column has a u8 scale s8 and a
u8 offset a.  The int8 weight is the byte congruent to q*s8 + a, with its
most significant bit flipped, read as two's complement:

    w8[k][n] = int8( ((q[k][n] * s8[g][n] + a[g][n]) mod 256) XOR 0x80 ),
    g = floor(k / G).

The page fixes a = 128 + (the group's smallest int8 weight) and s8 <= 16 so
that the product plus offset never passes 255; then the XOR is a subtraction
of 128 and w8 = q*s8 + a - 128 exactly (the tests pin both readings against
each other).  A group whose a + 15*s8 passes 255 is outside the format.

Activations (page "量化开销对比" (laojiahuo2003.github.io), section 4,
dynamic route): each row (token) gets its own scale from its largest
magnitude, taken at run time.  Symmetric int8 (section 2: with zero points
at 0 the integer product is the only term): sx[m] = max_k |x[m][k]| / 127 in
fp32, xq[m][k] = round-half-even(x[m][k] / sx[m]) in fp32, clamped to
[-127, 127]; a row of zeros gets sx = 0 and xq = 0.  The integer these
decide is decided in fp32, the precision the kernel uses.

Product (page "量化开销对比", section 1, route A: int8 times int8, int32
accumulation, then the scales; section 2: per-row and per-column scales
multiply outside the sum; page "W4A8量化计算优化", section 2.1: the group
level of the weight quantisation is integer, so nothing inside the sum is
floating point):

    acc[m][n] = sum_k xq[m][k] * w8[k][n]          (exact integer)
    Y[m][n]   = RNE_dtype( acc[m][n] * sx[m] * sw[n] )

with sw[n] the fp32 per-output-channel weight scale.  |xq| <= 127 and
|w8| <= 128, so |acc| < 2^14 * K < 2^31 for K < 2^17: the sum fits int32,
and a float64 matmul of the integer operands is exact (every partial sum is
an integer below 2^53), which is why a library matmul may stand in for the
plain sum here.  acc*sx*sw is taken in fp64 and rounded once to the output
dtype.

Layouts (the canonical tensors at the library boundary, row-major):
  xq       int8 [M][K];   sx  float32 [M]
  qweight  uint32 [K/8][N]; nibble i (bits 4i..4i+3) of word [r][n] is
           q[8r+i][n] -- the same order as the W4A16 route
  s8, a    uint8 [K/G][N]
  sw       float32 [N]
"""
from __future__ import annotations

import numpy as np

__all__ = ["unpack", "weight_int8", "overflow_groups", "quantize_rows", "accumulate",
           "scale_output", "gemm", "gemm_at", "round_to_bits", "bits_to_float", "ulp",
           "quantize_weights_two_level"]


def unpack(qweight: np.ndarray, K: int, N: int) -> np.ndarray:
    """qweight uint32 [K/8][N] -> q uint8 [K][N]; nibble i of word r is row 8r+i."""
    w = np.asarray(qweight, dtype=np.uint32).reshape(K // 8, N)
    q = np.empty((K, N), dtype=np.uint8)
    for i in range(8):
        q[i::8, :] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return q


def weight_int8(qweight, s8, a, K: int, N: int, G: int) -> np.ndarray:
    """The LiquidQuant congruence, element by element: int8 [K][N]."""
    q = unpack(qweight, K, N).astype(np.int64)
    g = np.arange(K) // G
    s = np.asarray(s8, dtype=np.int64).reshape(K // G, N)[g, :]
    off = np.asarray(a, dtype=np.int64).reshape(K // G, N)[g, :]
    byte = ((q * s + off) % 256) ^ 0x80
    return byte.astype(np.uint8).view(np.int8)


def overflow_groups(s8, a) -> np.ndarray:
    """Boolean mask of the groups outside the format: q*s8 + a can pass 255
    for some code q in 0..15 (page "W4A8量化计算优化", section 2.1: the scale
    is held to at most 16 so that the multiply-add cannot overflow)."""
    s = np.asarray(s8, dtype=np.int64)
    off = np.asarray(a, dtype=np.int64)
    return (s > 16) | (off + 15 * s > 255)


def quantize_rows(x: np.ndarray):
    """Dynamic per-row symmetric int8: x float [M][K] (values of the
    activation dtype) -> (xq int8 [M][K], sx float32 [M]).  fp32 arithmetic,
    IEEE division, round half to even."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=1) if x32.shape[1] else np.zeros(x32.shape[0], np.float32)
    sx = (amax / np.float32(127.0)).astype(np.float32)
    xq = np.zeros(x32.shape, dtype=np.int8)
    nz = sx > 0
    if np.any(nz):
        r = np.rint(x32[nz] / sx[nz, None]).astype(np.float32)   # fp32 division, then RNE
        xq[nz] = np.clip(r, -127, 127).astype(np.int8)
    return xq, sx


def accumulate(xq, w8) -> np.ndarray:
    """acc[m][n] = sum_k xq[m][k] * w8[k][n] as int64 (exact; see header)."""
    xf = np.asarray(xq, dtype=np.int8).astype(np.float64)
    wf = np.asarray(w8, dtype=np.int8).astype(np.float64)
    acc = xf @ wf
    return acc.astype(np.int64)


def _frexp_exponent(x: np.ndarray) -> np.ndarray:
    """floor(log2 |x|) for finite nonzero x, exactly (via frexp)."""
    _, e = np.frexp(x)
    return e.astype(np.int64) - 1


def round_to_bits(v: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> uint16 bit patterns of fp16 or bf16, round to nearest, ties
    to even, overflow to infinity, gradual underflow.  Done by scaling to the
    target's unit in the last place (a power of two, so exact) and rounding
    with numpy's half-to-even rint."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "fp16":
        man, emin, emax_val = 10, -14, 65504.0
    elif dtype == "bf16":
        man, emin, emax_val = 7, -126, float(np.float32(3.3895313892515355e38))
    else:
        raise ValueError(dtype)
    out = np.zeros(v.shape, dtype=np.float64)
    fin = np.isfinite(v) & (v != 0)
    e = np.maximum(_frexp_exponent(np.where(fin, v, 1.0)), emin)
    ulp_ = np.ldexp(1.0, (e - man).astype(np.int32))
    r = np.rint(np.where(fin, v, 0.0) / ulp_) * ulp_
    out = np.where(fin, r, v)
    # values that round past the largest finite value become infinity
    top = emax_val + np.ldexp(1.0, int(np.floor(np.log2(emax_val))) - man - 1)
    over = fin & (np.abs(v) >= top)
    out = np.where(over, np.copysign(np.inf, v), out)
    if dtype == "fp16":
        return out.astype(np.float16).view(np.uint16)   # exact: out is representable
    b = out.astype(np.float32).view(np.uint32)          # exact: out is representable in fp32
    return (b >> np.uint32(16)).astype(np.uint16)


def bits_to_float(bits: np.ndarray, dtype: str) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the output dtype's representable values at |v| (its unit in
    the last place; the smallest subnormal spacing near zero)."""
    man, emin = (10, -14) if dtype == "fp16" else (7, -126)
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.maximum(_frexp_exponent(np.where(a > 0, a, 1.0)), emin)
    e = np.where(a > 0, e, emin)
    return np.ldexp(1.0, (e - man).astype(np.int32))


def scale_output(acc, sx, sw, dtype: str) -> np.ndarray:
    """Y bits = RNE_dtype(acc * sx[m] * sw[n]), the product taken in fp64."""
    y = (np.asarray(acc, dtype=np.float64) * np.asarray(sx, np.float32).astype(np.float64)[:, None]
         * np.asarray(sw, np.float32).astype(np.float64)[None, :])
    return round_to_bits(y, dtype)


def gemm(xq, sx, qweight, s8, a, sw, M, N, K, G, dtype="fp16"):
    """Full W4A8 product.  Returns (Y bits uint16 [M][N] or None for
    dtype == "i32", acc int64 [M][N])."""
    w8 = weight_int8(qweight, s8, a, K, N, G)
    acc = accumulate(np.asarray(xq).reshape(M, K), w8)
    if dtype == "i32":
        return None, acc
    return scale_output(acc, sx, sw, dtype), acc


def gemm_at(xq, sx, qweight, s8, a, sw, M, N, K, G, ms, ns, dtype="fp16"):
    """Y and acc at the outputs (ms[i], ns[i]) only, each by its own dot
    product, for shapes whose full product is too large for the CPU."""
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    cols = np.unique(ns)
    q = np.asarray(qweight, dtype=np.uint32).reshape(K // 8, N)[:, cols]
    s = np.asarray(s8).reshape(K // G, N)[:, cols]
    o = np.asarray(a).reshape(K // G, N)[:, cols]
    w8 = weight_int8(q, s, o, K, len(cols), G).astype(np.int64)
    where = {int(c): i for i, c in enumerate(cols)}
    x = np.asarray(xq, dtype=np.int8).reshape(M, K).astype(np.int64)
    acc = np.array([int(np.dot(x[m], w8[:, where[int(n)]])) for m, n in zip(ms, ns)],
                   dtype=np.int64)
    if dtype == "i32":
        return None, acc
    y = (acc.astype(np.float64) * np.asarray(sx, np.float32).astype(np.float64)[ms]
         * np.asarray(sw, np.float32).astype(np.float64)[ns])
    return round_to_bits(y, dtype), acc


def quantize_weights_two_level(w: np.ndarray, G: int):
    """Two-level weight quantisation that produces inputs in this format from
    real weights (used to check the format's reach, not on the product path).

    Level 1, per output column: sw = max|w| / 120 and w_i8 = round(w / sw),
    so every int8 weight lies in [-120, 120] and a group spans at most 240.
    Level 2, per group of G along k (page "W4A8量化计算优化", section 2.1):
    s8 = ceil((max - min) / 15) <= 16, codes q = round((w_i8 - min') / s8) in
    0..15 and a = 128 + min', where min' = min(group min, 127 - 15*s8) keeps
    a + 15*s8 <= 255 (no code can overflow) while 15 codes still cover
    [min, max].  Returns (qweight, s8, a, sw, w_i8)."""
    w = np.asarray(w, dtype=np.float64)
    K, N = w.shape
    amax = np.max(np.abs(w), axis=0)
    sw = np.where(amax > 0, amax / 120.0, 1.0).astype(np.float32)
    wi8 = np.clip(np.rint(w / sw.astype(np.float64)[None, :]), -120, 120).astype(np.int64)
    g = wi8.reshape(K // G, G, N)
    lo = g.min(axis=1)
    hi = g.max(axis=1)
    s8 = np.maximum(1, -((lo - hi) // 15))           # ceil((hi - lo) / 15), at least 1
    lo2 = np.minimum(lo, 127 - 15 * s8)
    q = np.clip(np.rint((g - lo2[:, None, :]) / s8[:, None, :]), 0, 15).astype(np.uint32)
    q = q.reshape(K, N)
    qweight = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        qweight |= q[i::8, :] << np.uint32(4 * i)
    return qweight, s8.astype(np.uint8), (128 + lo2).astype(np.uint8), sw, wi8.astype(np.int8)
