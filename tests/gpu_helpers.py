"""Helpers for the GPU parity tests: run the HIP library through its C ABI
(via the Python binding) and compare with the CPU oracle."""
import os
import sys

import numpy as np

import oracle
import w4a16_synth as synth

TOL = {"fp16": 2e-3, "bf16": 1e-2}


def lib():
    import w4a16_dequant_gemm_amd as w4
    from w4a16_dequant_gemm_amd import build as hipbuild
    if not os.path.exists(hipbuild.LIB):
        hipbuild.build()
    w4.load_library()
    return w4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check_shapes(p):
    """Host-side check of the operand shapes the kernels assume, before a launch."""
    assert p.X.shape == (p.M, p.K) and p.X.dtype == np.uint16
    assert p.qweight.shape == (p.K // 8, p.N) and p.qweight.dtype == np.uint32
    assert p.scales.shape == (p.K // p.G, p.N) and p.scales.dtype == np.uint16
    if p.sym:
        assert p.zeros is None
    else:
        assert p.zeros.shape == (p.K // p.G, p.N) and p.zeros.dtype == np.uint8
        assert int(p.zeros.max()) <= 15
    assert p.N % 128 == 0 and p.K % 256 == 0 and p.K % p.G == 0 and p.G in (32, 64, 128)


class OnDevice:
    """A problem's canonical tensors, its repacked blob and a GEMM runner."""

    def __init__(self, p, device="cuda"):
        self.w4 = lib()
        check_shapes(p)
        self.p = p
        self.flags = self.w4.flags_of(p.dtype, p.sym)
        self.X, self.qw, self.sc, self.zr = self.w4.to_device(p, device)
        self.packed = self.w4.w4a16_repack(self.qw, self.sc, self.zr, p.K, p.N, p.G, self.flags)

    def gemm(self, X=None, M=None, plan=None):
        import torch
        Xd = self.X if X is None else X
        Y = self.w4.w4a16_gemm(Xd, self.packed, M=M, plan=plan)
        torch.cuda.synchronize()
        return Y

    def y_float(self, Y):
        return oracle.bits_to_float(self.w4.bits_of(Y), self.p.dtype)


def same_bits(a, b):
    """Bit-identical after mapping -0 to +0 (a zero product may carry either sign)."""
    a = np.where(a == 0x8000, 0, a)
    b = np.where(b == 0x8000, 0, b)
    return np.array_equal(a, b)


def assert_gemm_close(p, Yg_float, Yref, B, what=""):
    rel, zero_ok = oracle.max_rel_error(Yg_float, Yref, B)
    tol = TOL[p.dtype]
    assert zero_ok, f"{what}: an output with bound 0 is not 0"
    assert rel <= tol, f"{what}: max|Y-Yref|/B = {rel:.3e} > {tol}"
    return rel


def column_slice(p, cols):
    """The sub-problem made of the given output columns (weights only)."""
    cols = np.asarray(cols)
    return synth.Problem(p.M, p.K, len(cols), p.G, p.dtype, p.sym, p.X,
                         np.ascontiguousarray(p.qweight[:, cols]),
                         np.ascontiguousarray(p.scales[:, cols]),
                         None if p.zeros is None else np.ascontiguousarray(p.zeros[:, cols]))
