"""Python binding of the W4A8 entry points (include/w4a8.h) of libw4a16.so.

Argument marshalling only: the repack, the activation quantisation and the
GEMM run in the library's HIP kernels.  PyTorch provides device memory and
the current stream.  There is no fallback.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import (W4A16Error, W4A16_ERR_INVALID_ARG, W4A16_ERR_UNSUPPORTED, W4A16_PLAN_PARAM_SHIFT,
               _bad, _check, _ptr, _require, _stream, load_library)

W4A8_LAYOUT_VERSION = 1
W4A8_OUT = {"fp16": 0x0, "bf16": 0x1, "i32": 0x2}
W4A8_PLAN = {"stream": 0x10, "tiled": 0x20}
W4A8_X = {"fp16": 0x0, "bf16": 0x1}
W4A8_TRAILER_OVERFLOW = 0x1
C_FUNCTIONS_W4A8 = ("w4a8_packed_bytes", "w4a8_repack", "w4a8_dequant", "w4a8_quantize_rows",
                    "w4a8_gemm")
_OUT_DTYPE = {"fp16": torch.float16, "bf16": torch.bfloat16, "i32": torch.int32}

_declared = False


def _lib():
    global _declared
    lib = load_library()
    if not _declared:
        p, i64, ci, u32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                               ctypes.c_size_t)
        lib.w4a8_packed_bytes.argtypes = [i64, i64, ci]
        lib.w4a8_packed_bytes.restype = sz
        lib.w4a8_repack.argtypes = [p, p, p, p, i64, i64, ci, p, sz, p]
        lib.w4a8_repack.restype = ci
        lib.w4a8_dequant.argtypes = [p, sz, p, i64, i64, ci, p]
        lib.w4a8_dequant.restype = ci
        lib.w4a8_quantize_rows.argtypes = [p, p, p, i64, i64, u32, p]
        lib.w4a8_quantize_rows.restype = ci
        lib.w4a8_gemm.argtypes = [p, p, p, sz, p, i64, i64, i64, ci, u32, p]
        lib.w4a8_gemm.restype = ci
        _declared = True
    return lib


def plan_flags_w8(plan) -> int:
    """None, "stream", "tiled" or ("stream", parts of K)."""
    if plan is None:
        return 0
    name, param = (plan, 0) if isinstance(plan, str) else plan
    if name not in W4A8_PLAN or not 0 <= int(param) <= 255:
        raise ValueError(f"bad plan hint {plan!r}")
    return W4A8_PLAN[name] | (int(param) << W4A16_PLAN_PARAM_SHIFT)


@dataclass
class PackedW8:
    """A W4A8 blob and the shape it was made for."""
    data: torch.Tensor   # uint8 device tensor
    K: int
    N: int
    group_size: int


def w4a8_packed_bytes(K: int, N: int, group_size: int) -> int:
    return int(_lib().w4a8_packed_bytes(K, N, group_size))


def w4a8_repack(qweight: torch.Tensor, s8: torch.Tensor, a: torch.Tensor, sw: torch.Tensor,
                K: int, N: int, group_size: int, stream=None) -> PackedW8:
    """qweight int32 [K/8][N], s8 and a uint8 [K/G][N], sw float32 [N] -> PackedW8."""
    nbytes = w4a8_packed_bytes(K, N, group_size)
    if nbytes == 0:
        raise W4A16Error(W4A16_ERR_UNSUPPORTED if (N % 128 or K % 256) else
                         W4A16_ERR_INVALID_ARG, "w4a8_packed_bytes")
    dev = qweight.device
    if qweight.dtype not in (torch.int32, torch.uint32) or qweight.numel() != (K // 8) * N \
            or not qweight.is_contiguous() or not qweight.is_cuda:
        _bad("w4a8_repack: qweight must be a contiguous int32 device tensor of K/8*N elements")
    ng = (K // group_size) * N
    _require(s8, "w4a8_repack: s8", torch.uint8, ng, dev)
    _require(a, "w4a8_repack: a", torch.uint8, ng, dev)
    _require(sw, "w4a8_repack: sw", torch.float32, N, dev)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(_lib().w4a8_repack(_ptr(qweight), _ptr(s8), _ptr(a), _ptr(sw), K, N, group_size,
                              _ptr(packed), nbytes, _stream(stream)), "w4a8_repack")
    return PackedW8(packed, K, N, group_size)


def trailer_flags(packed: PackedW8) -> int:
    """Feature flags of the blob trailer (reads 4 bytes back: synchronizes)."""
    t = packed.data[-16:].cpu().numpy().view("<u4")
    return int(t[2])


def w4a8_dequant(packed: PackedW8, stream=None) -> torch.Tensor:
    K, N, G = packed.K, packed.N, packed.group_size
    W = torch.empty((K, N), dtype=torch.int8, device=packed.data.device)
    _check(_lib().w4a8_dequant(_ptr(packed.data), packed.data.numel(), _ptr(W), K, N, G,
                               _stream(stream)), "w4a8_dequant")
    return W


def w4a8_quantize_rows(X: torch.Tensor, xq: Optional[torch.Tensor] = None,
                       sx: Optional[torch.Tensor] = None, stream=None):
    """X fp16/bf16 [M][K] -> (xq int8 [M][K], sx float32 [M])."""
    if X.dim() != 2 or X.dtype not in (torch.float16, torch.bfloat16) or not X.is_cuda \
            or not X.is_contiguous():
        _bad("w4a8_quantize_rows: X must be a contiguous fp16/bf16 [M][K] device tensor")
    M, K = X.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if sx is None:
        sx = torch.empty(M, dtype=torch.float32, device=X.device)
    _require(xq, "w4a8_quantize_rows: xq", torch.int8, M * K, X.device)
    _require(sx, "w4a8_quantize_rows: sx", torch.float32, M, X.device)
    flags = W4A8_X["bf16" if X.dtype == torch.bfloat16 else "fp16"]
    _check(_lib().w4a8_quantize_rows(_ptr(X), _ptr(xq), _ptr(sx), M, K, flags, _stream(stream)),
           "w4a8_quantize_rows")
    return xq, sx


def w4a8_gemm(xq: torch.Tensor, sx: Optional[torch.Tensor], packed: PackedW8, out: str = "fp16",
              Y: Optional[torch.Tensor] = None, plan=None, stream=None) -> torch.Tensor:
    """Y [M][N] (fp16, bf16 or int32 per `out`) of the W4A8 product."""
    if xq.dim() != 2 or xq.dtype != torch.int8 or not xq.is_cuda or not xq.is_contiguous():
        _bad("w4a8_gemm: xq must be a contiguous int8 [M][K] device tensor")
    M, K = xq.shape
    if K != packed.K:
        _bad(f"w4a8_gemm: xq has K = {K}, the blob {packed.K}")
    if out not in W4A8_OUT:
        raise ValueError(f"bad output kind {out!r}")
    N = packed.N
    if out != "i32" or sx is not None:
        _require(sx, "w4a8_gemm: sx", torch.float32, M, xq.device)
    if Y is None:
        Y = torch.empty((M, N), dtype=_OUT_DTYPE[out], device=xq.device)
    _require(Y, "w4a8_gemm: Y", _OUT_DTYPE[out], M * N, xq.device)
    if packed.data.device != xq.device:
        _bad("w4a8_gemm: the blob is on another device")
    flags = W4A8_OUT[out] | plan_flags_w8(plan)
    _check(_lib().w4a8_gemm(_ptr(xq), _ptr(sx), _ptr(packed.data), packed.data.numel(), _ptr(Y),
                            M, N, K, packed.group_size, flags, _stream(stream)), "w4a8_gemm")
    return Y
