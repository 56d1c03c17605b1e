"""CPU oracle for the fused W4A16 dequantize-GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library never calls it, and it imports nothing from the GPU package.

The arithmetic lives in ``w4a16_oracle.c`` (plain C, fp64 accumulation); this
module compiles it with gcc when the shared object is missing and wraps it
with numpy arrays.  See the C file's header for the definition it follows and
the passages of the pages each step comes from.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a16_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F16 = 0
BF16 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-D_DEFAULT_SOURCE", "-shared", "-fPIC",
               "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    ci = ctypes.c_int
    lib.oracle_version.restype = ci
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_round_f16.argtypes = [ctypes.c_double]
    lib.oracle_round_f16.restype = ctypes.c_uint16
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_round_bf16.restype = ctypes.c_uint16
    lib.oracle_unpack.argtypes = [p, i64, i64, p]
    lib.oracle_unpack.restype = ci
    lib.oracle_dequant.argtypes = [p, p, p, i64, i64, i64, ci, ci, p, p]
    lib.oracle_dequant.restype = ci
    lib.oracle_dequant_values.argtypes = [p, p, p, i64, ci, p]
    lib.oracle_dequant_values.restype = ci
    lib.oracle_gemm.argtypes = [p, p, p, p, i64, i64, i64, i64, ci, ci, p, p, p, ci]
    lib.oracle_gemm.restype = ci
    lib.oracle_gemm_at.argtypes = [p, p, p, p, i64, i64, i64, i64, ci, ci, p, p, i64, p, p, ci]
    lib.oracle_gemm_at.restype = ci
    lib.oracle_epilogue.argtypes = [p, p, p, p, i64, i64, i64, p, p, p, ci, ci, ci, p, p]
    lib.oracle_epilogue.restype = ci
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def dtype_code(name: str) -> int:
    return {"fp16": F16, "f16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}[name]


def f16_to_double(bits: int) -> float:
    return _load().oracle_f16_to_double(int(bits))


def bf16_to_double(bits: int) -> float:
    return _load().oracle_bf16_to_double(int(bits))


def round_f16(v: float) -> int:
    return int(_load().oracle_round_f16(float(v)))


def round_bf16(v: float) -> int:
    return int(_load().oracle_round_bf16(float(v)))


def unpack(qweight: np.ndarray, K: int, N: int) -> np.ndarray:
    """q[K][N] (uint8) from qweight[K/8][N]."""
    qw = _c(qweight, np.uint32)
    q = np.empty((K, N), dtype=np.uint8)
    rc = _load().oracle_unpack(_ptr(qw), K, N, _ptr(q))
    if rc:
        raise ValueError(f"oracle_unpack: bad shape K={K} N={N}")
    return q


def dequant(qweight, scales, zeros, K, N, G, dtype, sym, exact=False):
    """deq bit patterns [K][N] (uint16) and optionally the exact fp64 values."""
    qw = _c(qweight, np.uint32)
    sc = _c(scales, np.uint16)
    zr = None if sym else _c(zeros, np.uint8)
    out = np.empty((K, N), dtype=np.uint16)
    ex = np.empty((K, N), dtype=np.float64) if exact else None
    rc = _load().oracle_dequant(_ptr(qw), _ptr(sc), _ptr(zr), K, N, G, dtype_code(dtype)
                                if isinstance(dtype, str) else dtype, int(bool(sym)),
                                _ptr(out), _ptr(ex))
    if rc:
        raise ValueError("oracle_dequant: bad arguments")
    return (out, ex) if exact else out


def dequant_values(q, z, s_bits, dtype):
    """RNE((q - z) * s) bit patterns for flat arrays q, z (uint8) and s_bits (uint16)."""
    q = _c(q, np.uint8).ravel()
    z = _c(z, np.uint8).ravel()
    s = _c(s_bits, np.uint16).ravel()
    assert q.size == z.size == s.size
    out = np.empty(q.size, dtype=np.uint16)
    code = dtype_code(dtype) if isinstance(dtype, str) else dtype
    rc = _load().oracle_dequant_values(_ptr(q), _ptr(z), _ptr(s), q.size, code, _ptr(out))
    if rc:
        raise ValueError("oracle_dequant_values: bad dtype")
    return out


def _threads(n):
    """Worker threads: n if given, else this process's CPU share, at most 16."""
    if n and n > 0:
        return int(n)
    try:
        share = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        share = os.cpu_count() or 1
    return max(1, min(16, share))


def gemm(X, qweight, scales, zeros, M, N, K, G, dtype, sym, with_exact=False, nthreads=0):
    """(Y, B) or (Y, B, Yx): fp64 [M][N] product, error-bound denominator, unrounded-deq product."""
    x = _c(X, np.uint16)
    qw = _c(qweight, np.uint32)
    sc = _c(scales, np.uint16)
    zr = None if sym else _c(zeros, np.uint8)
    Y = np.empty((M, N), dtype=np.float64)
    B = np.empty((M, N), dtype=np.float64)
    Yx = np.empty((M, N), dtype=np.float64) if with_exact else None
    code = dtype_code(dtype) if isinstance(dtype, str) else dtype
    rc = _load().oracle_gemm(_ptr(x), _ptr(qw), _ptr(sc), _ptr(zr), M, N, K, G, code,
                             int(bool(sym)), _ptr(Y), _ptr(B), _ptr(Yx), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_gemm failed with status {rc}")
    return (Y, B, Yx) if with_exact else (Y, B)


def gemm_at(X, qweight, scales, zeros, M, N, K, G, dtype, sym, ms, ns, nthreads=0):
    """(Y, B) for the sampled output elements (ms[i], ns[i])."""
    x = _c(X, np.uint16)
    qw = _c(qweight, np.uint32)
    sc = _c(scales, np.uint16)
    zr = None if sym else _c(zeros, np.uint8)
    ms = _c(ms, np.int64).ravel()
    ns = _c(ns, np.int64).ravel()
    assert ms.size == ns.size
    Y = np.empty(ms.size, dtype=np.float64)
    B = np.empty(ms.size, dtype=np.float64)
    code = dtype_code(dtype) if isinstance(dtype, str) else dtype
    rc = _load().oracle_gemm_at(_ptr(x), _ptr(qw), _ptr(sc), _ptr(zr), M, N, K, G, code,
                                int(bool(sym)), _ptr(ms), _ptr(ns), ms.size, _ptr(Y),
                                _ptr(B), _threads(nthreads))
    if rc:
        raise ValueError(f"oracle_gemm_at failed with status {rc}")
    return Y, B


ACTIVATIONS = {"none": 0, "relu": 1, "silu": 2}
AUX_OPS = {"add": 0, "mul": 1}


def epilogue(Y, B, M, N, dtype, col_scale=None, bias=None, aux=None, activation="none",
             aux_op="add", ms=None, ns=None):
    """(Yo, Bo): the epilogue y = aux_op(act(Y*c + b), a) and its error-bound
    denominator, in fp64.  Y, B are [M][N] (full output) or, with ms/ns, the
    sampled elements (ms[i], ns[i]).  col_scale: float values [N]; bias: bit
    patterns [N]; aux: bit patterns [M][N]; each optional."""
    Yf = np.ascontiguousarray(np.asarray(Y, dtype=np.float64).ravel())
    Bf = np.ascontiguousarray(np.asarray(B, dtype=np.float64).ravel())
    if ms is None:
        mm, nn = np.meshgrid(np.arange(M, dtype=np.int64), np.arange(N, dtype=np.int64),
                             indexing="ij")
        ms, ns = mm.ravel(), nn.ravel()
    ms = _c(ms, np.int64).ravel()
    ns = _c(ns, np.int64).ravel()
    assert ms.size == ns.size == Yf.size == Bf.size
    cs = None if col_scale is None else _c(np.asarray(col_scale, dtype=np.float64).ravel(), np.float64)
    bs = None if bias is None else _c(bias, np.uint16)
    ax = None if aux is None else _c(aux, np.uint16)
    Yo = np.empty_like(Yf)
    Bo = np.empty_like(Bf)
    code = dtype_code(dtype) if isinstance(dtype, str) else dtype
    rc = _load().oracle_epilogue(_ptr(Yf), _ptr(Bf), _ptr(ms), _ptr(ns), ms.size, M, N,
                                 _ptr(cs), _ptr(bs), _ptr(ax), code, ACTIVATIONS[activation],
                                 AUX_OPS[aux_op], _ptr(Yo), _ptr(Bo))
    if rc:
        raise ValueError(f"oracle_epilogue failed with status {rc}")
    shape = np.shape(Y)
    return Yo.reshape(shape), Bo.reshape(shape)


def bits_to_float(bits: np.ndarray, dtype) -> np.ndarray:
    """Decode uint16 bit patterns of fp16/bf16 to float64 (vectorised field decode)."""
    b = np.asarray(bits, dtype=np.uint16)
    code = dtype_code(dtype) if isinstance(dtype, str) else dtype
    if code == F16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def max_rel_error(Y_gpu: np.ndarray, Y_ref: np.ndarray, B: np.ndarray):
    """max |Y_gpu - Y_ref| / B over elements with B > 0, and whether every B == 0 entry is 0."""
    Yg = np.asarray(Y_gpu, dtype=np.float64)
    err = np.abs(Yg - Y_ref)
    pos = B > 0
    rel = float(np.max(err[pos] / B[pos])) if np.any(pos) else 0.0
    zero_ok = bool(np.all(Yg[~pos] == 0.0))
    return rel, zero_ok
