"""Python binding of the MXFP4 entry points (include/mxfp4.h) of libw4a16.so.

Argument marshalling only: the repack, the MX quantisation of activations and
the GEMM run in the library's HIP kernels.  PyTorch provides device memory and
the current stream.  There is no fallback.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import (W4A16Error, W4A16_ERR_INVALID_ARG, W4A16_ERR_UNSUPPORTED, W4A16_PLAN_PARAM_SHIFT,
               _bad, _check, _ptr, _require, _stream, load_library)

MXFP4_LAYOUT_VERSION = 1
MXFP4_PLAN = {"stream": 0x10, "tiled": 0x20}
C_FUNCTIONS_MXFP4 = ("mxfp4_packed_bytes", "mxfp4_repack", "mxfp4_quantize_rows", "mxfp4_gemm")
_DT = {"fp16": (0x0, torch.float16), "bf16": (0x1, torch.bfloat16)}

_declared = False


def _lib():
    global _declared
    lib = load_library()
    if not _declared:
        p, i64, u32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
        lib.mxfp4_packed_bytes.argtypes = [i64, i64]
        lib.mxfp4_packed_bytes.restype = sz
        lib.mxfp4_repack.argtypes = [p, p, i64, i64, p, sz, p]
        lib.mxfp4_repack.restype = ctypes.c_int
        lib.mxfp4_quantize_rows.argtypes = [p, p, p, i64, i64, u32, p]
        lib.mxfp4_quantize_rows.restype = ctypes.c_int
        lib.mxfp4_gemm.argtypes = [p, p, p, sz, p, i64, i64, i64, u32, p]
        lib.mxfp4_gemm.restype = ctypes.c_int
        _declared = True
    return lib


def plan_flags_mx(plan) -> int:
    """None, "stream", "tiled", or (name, parameter)."""
    if plan is None:
        return 0
    name, param = (plan, 0) if isinstance(plan, str) else plan
    if name not in MXFP4_PLAN or not 0 <= int(param) <= 255:
        raise ValueError(f"bad plan hint {plan!r}")
    return MXFP4_PLAN[name] | (int(param) << W4A16_PLAN_PARAM_SHIFT)


@dataclass
class PackedMX:
    data: torch.Tensor   # uint8 device tensor
    K: int
    N: int


def mxfp4_packed_bytes(K: int, N: int) -> int:
    return int(_lib().mxfp4_packed_bytes(K, N))


def mxfp4_repack(qweight: torch.Tensor, ws: torch.Tensor, K: int, N: int, stream=None) -> PackedMX:
    """qweight int32 [K/8][N] (E2M1 codes), ws uint8 [K/32][N] (E8M0) -> PackedMX."""
    nbytes = mxfp4_packed_bytes(K, N)
    if nbytes == 0:
        raise W4A16Error(W4A16_ERR_UNSUPPORTED if (N % 128 or K % 256) else
                         W4A16_ERR_INVALID_ARG, "mxfp4_packed_bytes")
    dev = qweight.device
    if qweight.dtype not in (torch.int32, torch.uint32) or qweight.numel() != (K // 8) * N \
            or not qweight.is_contiguous() or not qweight.is_cuda:
        _bad("mxfp4_repack: qweight must be a contiguous int32 device tensor of K/8*N elements")
    _require(ws, "mxfp4_repack: ws", torch.uint8, (K // 32) * N, dev)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(_lib().mxfp4_repack(_ptr(qweight), _ptr(ws), K, N, _ptr(packed), nbytes,
                               _stream(stream)), "mxfp4_repack")
    return PackedMX(packed, K, N)


def mxfp4_quantize_rows(X: torch.Tensor, stream=None):
    """X fp16/bf16 [M][K] -> (xq uint8 [M][K] E4M3, xs uint8 [M][K/32] E8M0)."""
    if X.dim() != 2 or X.dtype not in (torch.float16, torch.bfloat16) or not X.is_cuda \
            or not X.is_contiguous():
        _bad("mxfp4_quantize_rows: X must be a contiguous fp16/bf16 [M][K] device tensor")
    M, K = X.shape
    if K % 32:
        _bad("mxfp4_quantize_rows: K must be a multiple of 32")
    xq = torch.empty((M, K), dtype=torch.uint8, device=X.device)
    xs = torch.empty((M, K // 32), dtype=torch.uint8, device=X.device)
    flags = 0x1 if X.dtype == torch.bfloat16 else 0x0
    _check(_lib().mxfp4_quantize_rows(_ptr(X), _ptr(xq), _ptr(xs), M, K, flags, _stream(stream)),
           "mxfp4_quantize_rows")
    return xq, xs


def mxfp4_gemm(xq: torch.Tensor, xs: torch.Tensor, packed: PackedMX, out: str = "fp16",
               Y: Optional[torch.Tensor] = None, plan=None, stream=None) -> torch.Tensor:
    if xq.dim() != 2 or xq.dtype != torch.uint8 or not xq.is_cuda or not xq.is_contiguous():
        _bad("mxfp4_gemm: xq must be a contiguous uint8 [M][K] device tensor")
    M, K = xq.shape
    if K != packed.K:
        _bad(f"mxfp4_gemm: xq has K = {K}, the blob {packed.K}")
    if out not in _DT:
        raise ValueError(f"bad output dtype {out!r}")
    flag, tdt = _DT[out]
    N = packed.N
    _require(xs, "mxfp4_gemm: xs", torch.uint8, M * (K // 32), xq.device)
    if Y is None:
        Y = torch.empty((M, N), dtype=tdt, device=xq.device)
    _require(Y, "mxfp4_gemm: Y", tdt, M * N, xq.device)
    if packed.data.device != xq.device:
        _bad("mxfp4_gemm: the blob is on another device")
    _check(_lib().mxfp4_gemm(_ptr(xq), _ptr(xs), _ptr(packed.data), packed.data.numel(), _ptr(Y),
                             M, N, K, flag | plan_flags_mx(plan), _stream(stream)), "mxfp4_gemm")
    return Y
