"""Python binding of the MI355X fused W4A16 dequantize-GEMM library.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libw4a16.so`` (built from ``csrc/`` by ``build.py``).  PyTorch
provides device memory and the current stream.  There is no fallback: if the
library is missing, importing the C functions raises.

The functions carry the names of the C entry points in ``include/w4a16.h``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4a16.so")

W4A16_OK = 0
W4A16_ERR_INVALID_ARG = 1
W4A16_ERR_UNSUPPORTED = 2
W4A16_ERR_WORKSPACE = 3
W4A16_ERR_HIP = 4

W4A16_FP16 = 0x0
W4A16_BF16 = 0x1
W4A16_ASYM = 0x0
W4A16_SYM = 0x2
# plan hints (flags of w4a16_workspace_bytes and the GEMM calls only)
W4A16_PLAN = {"decode": 0x10, "splitk": 0x20, "tiled": 0x30, "wide": 0x40}
W4A16_PLAN_PARAM_SHIFT = 8


def plan_flags(plan) -> int:
    """Flag bits of a plan hint: None, a variant name ("decode", "splitk",
    "tiled") or (name, parameter) -- tiles per decode item, split-K workgroups
    in units of 8, or the tiled kernel's split count."""
    if plan is None:
        return 0
    name, param = (plan, 0) if isinstance(plan, str) else plan
    if name not in W4A16_PLAN or not 0 <= int(param) <= 255:
        raise ValueError(f"bad plan hint {plan!r}")
    return W4A16_PLAN[name] | (int(param) << W4A16_PLAN_PARAM_SHIFT)

# entry points declared in include/w4a16.h
C_FUNCTIONS = (
    "w4a16_abi_version", "w4a16_layout_version", "w4a16_status_string", "w4a16_packed_bytes",
    "w4a16_repack", "w4a16_unrepack", "w4a16_workspace_bytes", "w4a16_gemm", "w4a16_dequant",
    "w4a16_mfma_layout_probe", "w4a16_gemm_ex", "w4a16_read_probe", "w4a16_read_probe_out_bytes",
    "w4a16_gemm_noalloc",
)
W4A16_NOALLOC_SCRATCH_BYTES = 16 << 20


class W4A16Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Epilogue(ctypes.Structure):
    """w4a16_epilogue_t of include/w4a16.h."""
    _fields_ = [("col_scale", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("aux", ctypes.c_void_p), ("activation", ctypes.c_int32),
                ("aux_op", ctypes.c_int32)]


W4A16_ACT = {"none": 0, "relu": 1, "silu": 2}
W4A16_AUX = {"add": 0, "mul": 1}

_lib = None
_layout_version = None
_ws_bytes = {}


def load_library(path: str = LIB_PATH):
    """Load libw4a16.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m "
                           "w4a16_dequant_gemm_amd.build` (or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    p, i64, ci, u32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32,
                           ctypes.c_size_t)
    lib.w4a16_abi_version.restype = ci
    lib.w4a16_layout_version.restype = ci
    lib.w4a16_status_string.argtypes = [ci]
    lib.w4a16_status_string.restype = ctypes.c_char_p
    lib.w4a16_packed_bytes.argtypes = [i64, i64, ci, u32]
    lib.w4a16_packed_bytes.restype = sz
    lib.w4a16_repack.argtypes = [p, p, p, i64, i64, ci, u32, p, sz, p]
    lib.w4a16_repack.restype = ci
    lib.w4a16_unrepack.argtypes = [p, sz, p, p, p, i64, i64, ci, u32, p]
    lib.w4a16_unrepack.restype = ci
    lib.w4a16_workspace_bytes.argtypes = [i64, i64, i64, ci, u32]
    lib.w4a16_workspace_bytes.restype = sz
    lib.w4a16_gemm.argtypes = [p, p, sz, p, i64, i64, i64, ci, u32, p, sz, p]
    lib.w4a16_gemm.restype = ci
    lib.w4a16_gemm_ex.argtypes = [p, p, sz, p, i64, i64, i64, ci, u32, ctypes.POINTER(Epilogue), p,
                                  sz, p]
    lib.w4a16_gemm_ex.restype = ci
    lib.w4a16_gemm_noalloc.argtypes = [p, p, sz, p, i64, i64, i64, ci, u32,
                                       ctypes.POINTER(Epilogue), p]
    lib.w4a16_gemm_noalloc.restype = ci
    lib.w4a16_dequant.argtypes = [p, sz, p, i64, i64, ci, u32, p]
    lib.w4a16_dequant.restype = ci
    lib.w4a16_mfma_layout_probe.argtypes = [p, p, p, u32, p]
    lib.w4a16_mfma_layout_probe.restype = ci
    lib.w4a16_read_probe_out_bytes.restype = sz
    lib.w4a16_read_probe.argtypes = [p, sz, p, sz, p]
    lib.w4a16_read_probe.restype = ci
    global _layout_version
    _layout_version = lib.w4a16_layout_version()
    _ws_bytes.clear()
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().w4a16_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != W4A16_OK:
        raise W4A16Error(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream) -> int:
    """hipStream_t of `stream` (a torch stream, a raw handle, or None = torch's
    current stream on the current device) as an integer."""
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _stream(stream) -> ctypes.c_void_p:
    return ctypes.c_void_p(_stream_handle(stream))


def _bad(where: str):
    raise W4A16Error(W4A16_ERR_INVALID_ARG, where)


def _require(t: Optional[torch.Tensor], where: str, dtype, numel: int, device=None):
    """A device tensor of the given dtype and element count, contiguous, on
    `device` when given: the checks the C entry points cannot make themselves
    (they see only pointers), so an undersized buffer never reaches a kernel."""
    if t is None:
        _bad(f"{where}: missing")
    if (t.dtype != dtype or t.numel() != numel or not t.is_contiguous() or not t.is_cuda
            or (device is not None and t.device != device)):
        _bad(f"{where}: need a contiguous {dtype} device tensor of {numel} elements"
             f"{'' if device is None else ' on ' + str(device)}, got {t.dtype} "
             f"{tuple(t.shape)} on {t.device}")


def flags_of(dtype: str, sym: bool) -> int:
    return (W4A16_BF16 if dtype in ("bf16", "bfloat16") else W4A16_FP16) | (W4A16_SYM if sym else 0)


def torch_dtype(flags: int) -> torch.dtype:
    return torch.bfloat16 if flags & W4A16_BF16 else torch.float16


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def w4a16_abi_version() -> int:
    return load_library().w4a16_abi_version()


def w4a16_layout_version() -> int:
    return load_library().w4a16_layout_version()


def w4a16_packed_bytes(K: int, N: int, group_size: int, flags: int) -> int:
    return int(load_library().w4a16_packed_bytes(K, N, group_size, flags))


def w4a16_workspace_bytes(M: int, N: int, K: int, group_size: int, flags: int) -> int:
    return int(load_library().w4a16_workspace_bytes(M, N, K, group_size, flags))


def _workspace_need(M, N, K, G, flags) -> int:
    # the plan depends on the shape and the flags (plan hints included) only
    key = (M, N, K, G, flags)
    need = _ws_bytes.get(key)
    if need is None:
        need = _ws_bytes[key] = w4a16_workspace_bytes(M, N, K, G, flags)
    return need


@dataclass
class PackedW4:
    """A repacked weight blob and the parameters it was made for."""
    data: torch.Tensor          # uint8 device tensor
    K: int
    N: int
    group_size: int
    flags: int
    layout_version: int


def w4a16_repack(qweight: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor],
                 K: int, N: int, group_size: int, flags: int, stream=None) -> PackedW4:
    """Canonical qweight int32/uint32-bits [K/8][N], scales [K/G][N] (fp16 or bf16 per
    flags) and zeros uint8 [K/G][N] (None for the symmetric format) -> PackedW4."""
    nbytes = w4a16_packed_bytes(K, N, group_size, flags)
    if nbytes == 0:
        raise W4A16Error(W4A16_ERR_UNSUPPORTED if (N % 128 or K % 256) else
                         W4A16_ERR_INVALID_ARG, "w4a16_packed_bytes")
    dev = qweight.device
    if qweight.dtype not in (torch.int32, torch.uint32) or qweight.numel() != (K // 8) * N \
            or not qweight.is_contiguous() or not qweight.is_cuda:
        _bad("w4a16_repack: qweight must be a contiguous int32 device tensor of K/8*N elements")
    _require(scales, "w4a16_repack: scales", torch_dtype(flags), (K // group_size) * N, dev)
    if flags & W4A16_SYM:
        if zeros is not None:
            _bad("w4a16_repack: the symmetric format takes no zeros")
    else:
        _require(zeros, "w4a16_repack: zeros", torch.uint8, (K // group_size) * N, dev)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check(load_library().w4a16_repack(_ptr(qweight), _ptr(scales), _ptr(zeros), K, N,
                                       group_size, flags, _ptr(packed), nbytes, _stream(stream)),
           "w4a16_repack")
    return PackedW4(packed, K, N, group_size, flags, w4a16_layout_version())


def w4a16_unrepack(packed: PackedW4, stream=None):
    dev = packed.data.device
    K, N, G, flags = packed.K, packed.N, packed.group_size, packed.flags
    qweight = torch.empty((K // 8, N), dtype=torch.int32, device=dev)
    scales = torch.empty((K // G, N), dtype=torch_dtype(flags), device=dev)
    zeros = None if flags & W4A16_SYM else torch.empty((K // G, N), dtype=torch.uint8, device=dev)
    _check(load_library().w4a16_unrepack(_ptr(packed.data), packed.data.numel(), _ptr(qweight),
                                         _ptr(scales), _ptr(zeros), K, N, G, flags,
                                         _stream(stream)), "w4a16_unrepack")
    return qweight, scales, zeros


# Workspaces cached per (device, stream): calls on different streams may run
# concurrently and must not share counters or partial tiles.  A workspace
# that has to grow is replaced, and the old one is kept alive for the rest of
# the process: a kernel still running on its stream, or a captured graph, may
# hold its address.
_workspaces = {}
_retired_workspaces = []


def workspace_for(nbytes: int, device: torch.device, stream=None) -> Optional[torch.Tensor]:
    """A zero-filled workspace of at least nbytes for calls on `stream` (default:
    torch's current stream) on `device`.  The library leaves its counters zero
    after every call, so the buffer is reused as it is."""
    if nbytes == 0:
        return None
    index = device.index if device.index is not None else torch.cuda.current_device()
    return _workspace_at(nbytes, index, _stream_handle(stream))


def _workspace_at(nbytes: int, device_index: int, stream_handle: int) -> torch.Tensor:
    key = (device_index, stream_handle)
    ws = _workspaces.get(key)
    if ws is not None and ws.numel() >= nbytes:
        return ws
    size = 1 << 20
    while size < nbytes:
        size *= 2
    if ws is not None:
        _retired_workspaces.append(ws)
    ws = torch.zeros(size, dtype=torch.uint8, device=torch.device("cuda", device_index))
    _workspaces[key] = ws
    return ws


_TORCH_DT = {0: torch.float16, W4A16_BF16: torch.bfloat16}


def _gemm_args(where, X, packed, M, Y, col_scale=None, bias=None, aux=None, activation="none",
               aux_op="add"):
    """Checks of the tensor arguments of the GEMM entry points; returns (M, Y, ep)
    with Y allocated if not given and ep the w4a16_epilogue_t (None if no
    epilogue operand or activation is given)."""
    if packed.layout_version != _layout_version:
        _bad(f"{where}: blob layout version {packed.layout_version}, library {_layout_version}")
    K, N, flags = packed.K, packed.N, packed.flags
    if M is None:
        M = X.shape[0]
    dt = _TORCH_DT[flags & W4A16_BF16]
    if (X.dtype != dt or X.numel() != M * K or not X.is_contiguous() or not X.is_cuda):
        _require(X, f"{where}: X", dt, M * K)     # raises with the details
    dev_index = X.get_device()
    if packed.data.get_device() != dev_index:
        _bad(f"{where}: the blob is on {packed.data.device}, X on {X.device}")
    if Y is None:
        Y = torch.empty((M, N), dtype=dt, device=X.device)
    elif (Y.dtype != dt or Y.numel() != M * N or not Y.is_contiguous() or not Y.is_cuda
          or Y.get_device() != dev_index):
        _require(Y, f"{where}: Y", dt, M * N, X.device)
    if col_scale is not None:
        _require(col_scale, f"{where}: col_scale", torch.float32, N, X.device)
    if bias is not None:
        _require(bias, f"{where}: bias", dt, N, X.device)
    if aux is not None:
        _require(aux, f"{where}: aux", dt, M * N, X.device)
    if activation not in W4A16_ACT or aux_op not in W4A16_AUX:
        _bad(f"{where}: activation {activation!r} / aux_op {aux_op!r}")
    ep = None
    if col_scale is not None or bias is not None or aux is not None or activation != "none":
        ep = Epilogue(None if col_scale is None else col_scale.data_ptr(),
                      None if bias is None else bias.data_ptr(),
                      None if aux is None else aux.data_ptr(), W4A16_ACT[activation],
                      W4A16_AUX[aux_op])
    return M, Y, ep


def w4a16_gemm(X: torch.Tensor, packed: PackedW4, M: Optional[int] = None,
               Y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None, plan=None) -> torch.Tensor:
    """Y[M][N] = X[M][K] . dequant(packed); X is [M][K] fp16/bf16 on the device.
    `plan`: an optional kernel hint (see plan_flags)."""
    lib = _lib if _lib is not None else load_library()
    M, Y, _ = _gemm_args("w4a16_gemm", X, packed, M, Y)
    K, N, G = packed.K, packed.N, packed.group_size
    flags = packed.flags if plan is None else packed.flags | plan_flags(plan)
    sh = _stream_handle(stream)
    if workspace is None:
        need = _workspace_need(M, N, K, G, flags)
        if need:
            workspace = _workspace_at(need, X.get_device(), sh)
    st = lib.w4a16_gemm(X.data_ptr(), packed.data.data_ptr(), packed.data.numel(), Y.data_ptr(),
                        M, N, K, G, flags, None if workspace is None else workspace.data_ptr(),
                        0 if workspace is None else workspace.numel(), sh)
    if st:
        _check(st, "w4a16_gemm")
    return Y


def w4a16_gemm_ex(X: torch.Tensor, packed: PackedW4, M: Optional[int] = None,
                  Y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None, *, col_scale: Optional[torch.Tensor] = None,
                  bias: Optional[torch.Tensor] = None, aux: Optional[torch.Tensor] = None,
                  activation: str = "none", aux_op: str = "add", plan=None) -> torch.Tensor:
    """w4a16_gemm with the fused output epilogue
    Y = aux_op(act(X.deq * col_scale + bias), aux): col_scale fp32 [N], bias [N]
    and aux [M][N] in X's dtype, each optional (device tensors)."""
    lib = load_library()
    M, Y, ep = _gemm_args("w4a16_gemm_ex", X, packed, M, Y, col_scale, bias, aux, activation,
                          aux_op)
    K, N, G = packed.K, packed.N, packed.group_size
    flags = packed.flags | plan_flags(plan)
    if workspace is None:
        workspace = workspace_for(_workspace_need(M, N, K, G, flags), X.device, stream)
    _check(lib.w4a16_gemm_ex(_ptr(X), _ptr(packed.data), packed.data.numel(), _ptr(Y), M, N, K,
                             G, flags, None if ep is None else ctypes.byref(ep), _ptr(workspace),
                             0 if workspace is None else workspace.numel(), _stream(stream)),
           "w4a16_gemm_ex")
    return Y


def w4a16_gemm_noalloc(X: torch.Tensor, packed: PackedW4, Y: torch.Tensor,
                       M: Optional[int] = None, stream=None, *,
                       col_scale: Optional[torch.Tensor] = None,
                       bias: Optional[torch.Tensor] = None, aux: Optional[torch.Tensor] = None,
                       activation: str = "none", aux_op: str = "add", plan=None) -> torch.Tensor:
    """w4a16_gemm_ex without a workspace: the library's static per-GPU scratch
    (W4A16_NOALLOC_SCRATCH_BYTES) serves instead, and nothing is allocated.
    The caller provides Y.  Calls that may overlap in time on one GPU race."""
    if Y is None:
        _bad("w4a16_gemm_noalloc: Y must be provided")
    lib = load_library()
    M, Y, ep = _gemm_args("w4a16_gemm_noalloc", X, packed, M, Y, col_scale, bias, aux,
                          activation, aux_op)
    _check(lib.w4a16_gemm_noalloc(_ptr(X), _ptr(packed.data), packed.data.numel(), _ptr(Y), M,
                                  packed.N, packed.K, packed.group_size,
                                  packed.flags | plan_flags(plan),
                                  None if ep is None else ctypes.byref(ep), _stream(stream)),
           "w4a16_gemm_noalloc")
    return Y


def w4a16_dequant(packed: PackedW4, W_out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    K, N = packed.K, packed.N
    if W_out is None:
        W_out = torch.empty((K, N), dtype=torch_dtype(packed.flags), device=packed.data.device)
    _check(load_library().w4a16_dequant(_ptr(packed.data), packed.data.numel(), _ptr(W_out), K,
                                        N, packed.group_size, packed.flags, _stream(stream)),
           "w4a16_dequant")
    return W_out


def w4a16_read_probe_out_bytes() -> int:
    return int(load_library().w4a16_read_probe_out_bytes())


def w4a16_read_probe(buf: torch.Tensor, nbytes: Optional[int] = None,
                     out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Read nbytes (default: all of buf, rounded down to 1 KiB) of a device
    buffer with the decode kernel's load pattern; returns the per-thread XORs
    (uint8 tensor of w4a16_read_probe_out_bytes() bytes)."""
    lib = load_library()
    if nbytes is None:
        nbytes = (buf.numel() * buf.element_size()) // 1024 * 1024
    if out is None:
        out = torch.empty(w4a16_read_probe_out_bytes(), dtype=torch.uint8, device=buf.device)
    _check(lib.w4a16_read_probe(_ptr(buf), nbytes, _ptr(out), out.numel(), _stream(stream)),
           "w4a16_read_probe")
    return out


def w4a16_mfma_layout_probe(A: torch.Tensor, B: torch.Tensor, flags: int,
                            stream=None) -> torch.Tensor:
    D = torch.empty((32, 32), dtype=torch.float32, device=A.device)
    _check(load_library().w4a16_mfma_layout_probe(_ptr(A), _ptr(B), _ptr(D), flags,
                                                  _stream(stream)), "w4a16_mfma_layout_probe")
    return D


# ---------------------------------------------------------------------------
# host <-> device plumbing for the canonical numpy tensors of w4a16_synth
# ---------------------------------------------------------------------------

def to_device(problem, device="cuda"):
    """Canonical numpy tensors of a w4a16_synth.Problem -> device tensors."""
    tdt = torch.bfloat16 if problem.dtype == "bf16" else torch.float16
    X = torch.from_numpy(problem.X.view("int16")).view(tdt).to(device)
    qw = torch.from_numpy(problem.qweight.view("int32")).to(device)
    sc = torch.from_numpy(problem.scales.view("int16")).view(tdt).to(device)
    zr = None if problem.zeros is None else torch.from_numpy(problem.zeros).to(device)
    return X, qw, sc, zr


def bits_of(t: torch.Tensor):
    """Device fp16/bf16 tensor -> numpy uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")
