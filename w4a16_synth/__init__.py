"""Seeded synthetic inputs for the W4A16 dequantize-GEMM.

This module only draws random numbers and lays them out in the canonical
input format; it holds none of the method's arithmetic (no dequantization,
no product).  Both the GPU tests/benchmark and the CPU oracle take their
inputs from here, and from nowhere else.

Canonical format:
  X        uint16 bit patterns [M][K] of fp16 or bf16, row-major
  qweight  uint32 [K/8][N]; nibble i (bits 4i..4i+3) of word [r][n] is the
           4-bit weight at k = 8r + i, column n
  scales   uint16 bit patterns [K/G][N], same dtype as X
  zeros    uint8 [K/G][N], values 0..15 (None for the symmetric format,
           whose zero point is fixed at 8)

Recipe (the workloads of the pages: decode of a 70B-class model, whose
hidden size is 8192 and FFN size 28672):
  * numpy Generator(PCG64); SeedSequence(seed).spawn(5) gives independent
    streams for [X, q, scales, zeros, outlier columns].
  * X ~ N(0, 1) drawn in float64, optionally with round(frac*K) distinct
    "outlier" columns of K (chosen without replacement) multiplied by 20,
    then rounded to the dtype (fp16: float64 -> float16 RNE; bf16:
    float64 -> float32 -> bfloat16, both RNE).
  * q ~ uniform integers 0..15.
  * scale ~ U(0.002, 0.02) drawn in float64, rounded to the dtype like X.
  * zero ~ uniform integers 0..15 (asymmetric) or none (symmetric).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = ["Problem", "make_problem", "make_weights", "make_activations", "with_activations",
           "pack_nibbles", "to_dtype_bits", "WORKLOADS", "workload", "ProblemW8",
           "make_w4a8_weights", "make_w4a8_activations", "make_w4a8_problem", "W4A8_WORKLOADS",
           "ProblemMX", "make_mxfp4_weights", "make_mx_activations", "make_mxfp4_problem",
           "MXFP4_WORKLOADS"]


def to_dtype_bits(x64: np.ndarray, dtype: str) -> np.ndarray:
    """float64 array -> uint16 bit patterns of fp16 or bf16 (round to nearest even)."""
    if dtype == "fp16":
        return np.asarray(x64, dtype=np.float64).astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        f32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
        u = f32.view(np.uint32).astype(np.uint64)
        # round-to-nearest-even on the low 16 bits (inputs here are finite)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return u.astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """q[K][N] (values 0..15) -> qweight[K/8][N] uint32, nibble i = row 8r+i."""
    K, N = q.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    q8 = np.asarray(q, dtype=np.uint32).reshape(K // 8, 8, N)
    out = np.zeros((K // 8, N), dtype=np.uint32)
    for i in range(8):
        out |= q8[:, i, :] << np.uint32(4 * i)
    return out


@dataclass
class Problem:
    M: int
    K: int
    N: int
    G: int
    dtype: str
    sym: bool
    X: np.ndarray                 # uint16 [M][K]
    qweight: np.ndarray           # uint32 [K/8][N]
    scales: np.ndarray            # uint16 [K/G][N]
    zeros: Optional[np.ndarray]   # uint8 [K/G][N] or None
    q: Optional[np.ndarray] = field(default=None, repr=False)   # uint8 [K][N] if kept


def _streams(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(5)]


def make_activations(M: int, K: int, dtype: str = "fp16", seed: int = 0,
                     outlier_frac: float = 0.0, outlier_mult: float = 20.0) -> np.ndarray:
    """X bit patterns [M][K] (streams 0 and 4 of the seed)."""
    st = _streams(seed)
    x64 = st[0].standard_normal((M, K))
    if outlier_frac > 0:
        n_out = int(round(outlier_frac * K))
        if n_out > 0:
            cols = st[4].choice(K, size=n_out, replace=False)
            x64[:, cols] *= outlier_mult
    return to_dtype_bits(x64, dtype)


def make_weights(K: int, N: int, G: int = 128, dtype: str = "fp16", sym: bool = False,
                 seed: int = 0, keep_q: bool = False, scale_range=(0.002, 0.02)):
    """(qweight, scales, zeros, q or None) (streams 1, 2 and 3 of the seed)."""
    if K % 8 or K % G:
        raise ValueError("K must be a multiple of 8 and of G")
    st = _streams(seed)
    q = st[1].integers(0, 16, size=(K, N), dtype=np.uint8)
    qweight = pack_nibbles(q)
    s64 = st[2].uniform(scale_range[0], scale_range[1], size=(K // G, N))
    scales = to_dtype_bits(s64, dtype)
    zeros = None if sym else st[3].integers(0, 16, size=(K // G, N), dtype=np.uint8)
    return qweight, scales, zeros, (q if keep_q else None)


def make_problem(M: int, K: int, N: int, G: int = 128, dtype: str = "fp16",
                 sym: bool = False, seed: int = 0, outlier_frac: float = 0.0,
                 outlier_mult: float = 20.0, keep_q: bool = False,
                 scale_range=(0.002, 0.02)) -> Problem:
    qweight, scales, zeros, q = make_weights(K, N, G, dtype, sym, seed, keep_q, scale_range)
    X = make_activations(M, K, dtype, seed, outlier_frac, outlier_mult)
    return Problem(M, K, N, G, dtype, bool(sym), X, qweight, scales, zeros, q)


def with_activations(p: Problem, M: int, seed: int = 0, outlier_frac: float = 0.0) -> Problem:
    """The same weights as p with a fresh X of M rows."""
    X = make_activations(M, p.K, p.dtype, seed, outlier_frac)
    return Problem(M, p.K, p.N, p.G, p.dtype, p.sym, X, p.qweight, p.scales, p.zeros, p.q)


# Named workloads (shapes of a 70B-class decoder layer; "outliers" marks the
# 0.1%-of-K-columns x20 activation pattern).
WORKLOADS = {
    "decode_m1_k4096_n4096_fp16_asym_g128":
        dict(M=1, K=4096, N=4096, G=128, dtype="fp16", sym=False),
    **{f"decode_m{m}_k8192_n28672_fp16_asym_g128_outliers":
       dict(M=m, K=8192, N=28672, G=128, dtype="fp16", sym=False, outlier_frac=0.001)
       for m in (1, 4, 8)},
    **{f"decode_m{m}_k8192_n8192_fp16_asym_g128_outliers":
       dict(M=m, K=8192, N=8192, G=128, dtype="fp16", sym=False, outlier_frac=0.001)
       for m in (1, 4, 8)},
    **{f"transition_m{m}_k8192_n28672_bf16_sym_g128":
       dict(M=m, K=8192, N=28672, G=128, dtype="bf16", sym=True) for m in (16, 32)},
    **{f"transition_m{m}_k28672_n8192_bf16_sym_g128":
       dict(M=m, K=28672, N=8192, G=128, dtype="bf16", sym=True) for m in (16, 32)},
    **{f"batch_m{m}_k8192_n28672_fp16_asym_g{g}":
       dict(M=m, K=8192, N=28672, G=g, dtype="fp16", sym=False)
       for m in (64, 128) for g in (64, 32)},
    **{f"prefill_m{m}_k8192_n{n}_bf16_asym_g128":
       dict(M=m, K=8192, N=n, G=128, dtype="bf16", sym=False)
       for m in (4096, 8192) for n in (8192, 28672)},
}


def workload(name: str, seed: int = 0, keep_q: bool = False) -> Problem:
    return make_problem(seed=seed, keep_q=keep_q, **WORKLOADS[name])


# ---------------------------------------------------------------------------
# W4A8 route inputs.  Random draws only, inside the format's valid ranges:
#   xq   int8 [M][K], uniform integers in [-127, 127]   (stream 0)
#   sx   float32 [M], U(0.001, 0.02)                     (stream 4)
#   q    uint8 [K][N], uniform integers 0..15, packed like qweight above (stream 1)
#   s8   uint8 [K/G][N], uniform integers in [s_lo, 16]  (stream 2)
#   a    uint8 [K/G][N], uniform integers in [0, 255 - 15*s8] (stream 3), the
#        offsets for which no code can pass 255
#   sw   float32 [N], U(0.0005, 0.005)                   (stream 2, after s8)
# ---------------------------------------------------------------------------

@dataclass
class ProblemW8:
    M: int
    K: int
    N: int
    G: int
    xq: np.ndarray        # int8 [M][K]
    sx: np.ndarray        # float32 [M]
    qweight: np.ndarray   # uint32 [K/8][N]
    s8: np.ndarray        # uint8 [K/G][N]
    a: np.ndarray         # uint8 [K/G][N]
    sw: np.ndarray        # float32 [N]


def make_w4a8_weights(K: int, N: int, G: int = 128, seed: int = 0, s_lo: int = 1):
    """(qweight, s8, a, sw) for the W4A8 route."""
    if K % 8 or K % G:
        raise ValueError("K must be a multiple of 8 and of G")
    st = _streams(seed)
    q = st[1].integers(0, 16, size=(K, N), dtype=np.uint8)
    s8 = st[2].integers(s_lo, 17, size=(K // G, N), dtype=np.int64)
    a = np.floor(st[3].random((K // G, N)) * (256 - 15 * s8)).astype(np.int64)
    sw = st[2].uniform(0.0005, 0.005, size=N).astype(np.float32)
    return pack_nibbles(q), s8.astype(np.uint8), a.astype(np.uint8), sw


def make_w4a8_activations(M: int, K: int, seed: int = 0):
    """(xq int8 [M][K], sx float32 [M])."""
    st = _streams(seed)
    xq = st[0].integers(-127, 128, size=(M, K), dtype=np.int64).astype(np.int8)
    sx = st[4].uniform(0.001, 0.02, size=M).astype(np.float32)
    return xq, sx


def make_w4a8_problem(M: int, K: int, N: int, G: int = 128, seed: int = 0) -> ProblemW8:
    qweight, s8, a, sw = make_w4a8_weights(K, N, G, seed)
    xq, sx = make_w4a8_activations(M, K, seed)
    return ProblemW8(M, K, N, G, xq, sx, qweight, s8, a, sw)


# The W4A8 workloads: the same 70B-class layer; batch 128 is where the pages
# switch to the compute-bound mode, 4096 rows a prefill.
W4A8_WORKLOADS = {
    "w4a8_decode_m1_k8192_n28672_g128": dict(M=1, K=8192, N=28672, G=128),
    "w4a8_batch_m128_k8192_n28672_g128": dict(M=128, K=8192, N=28672, G=128),
    "w4a8_prefill_m4096_k8192_n28672_g128": dict(M=4096, K=8192, N=28672, G=128),
}


# ---------------------------------------------------------------------------
# MXFP4 route inputs.  Random draws only:
#   q    uint8 [K][N] E2M1 codes, uniform 0..15, packed like qweight (stream 1)
#   ws   uint8 [K/32][N] E8M0 weight block scales, uniform in [118, 124] (stream 2)
#   xq   uint8 [M][K] E4M3 codes, uniform over the 254 finite codes (stream 0)
#   xs   uint8 [M][K/32] E8M0 activation block scales, uniform in [116, 122] (stream 4)
# (activations taken from real values go through the quantiser instead)
# ---------------------------------------------------------------------------

@dataclass
class ProblemMX:
    M: int
    K: int
    N: int
    xq: np.ndarray       # uint8 [M][K]
    xs: np.ndarray       # uint8 [M][K/32]
    qweight: np.ndarray  # uint32 [K/8][N]
    ws: np.ndarray       # uint8 [K/32][N]


def make_mxfp4_weights(K: int, N: int, seed: int = 0):
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    st = _streams(seed)
    q = st[1].integers(0, 16, size=(K, N), dtype=np.uint8)
    ws = st[2].integers(118, 125, size=(K // 32, N), dtype=np.int64).astype(np.uint8)
    return pack_nibbles(q), ws


def make_mx_activations(M: int, K: int, seed: int = 0):
    st = _streams(seed)
    c = st[0].integers(0, 254, size=(M, K), dtype=np.int64)
    xq = np.where(c >= 127, c + 1, c).astype(np.uint8)      # skip 0x7F (NaN); 0xFF is never drawn
    xs = st[4].integers(116, 123, size=(M, K // 32), dtype=np.int64).astype(np.uint8)
    return xq, xs


def make_mxfp4_problem(M: int, K: int, N: int, seed: int = 0) -> ProblemMX:
    qweight, ws = make_mxfp4_weights(K, N, seed)
    xq, xs = make_mx_activations(M, K, seed)
    return ProblemMX(M, K, N, xq, xs, qweight, ws)


MXFP4_WORKLOADS = {
    "mxfp4_decode_m1_k8192_n28672": dict(M=1, K=8192, N=28672),
    "mxfp4_batch_m128_k8192_n28672": dict(M=128, K=8192, N=28672),
    "mxfp4_prefill_m4096_k8192_n28672": dict(M=4096, K=8192, N=28672),
}
