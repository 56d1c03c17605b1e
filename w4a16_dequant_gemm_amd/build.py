"""Build step: compile the HIP sources into the in-tree shared library
``w4a16_dequant_gemm_amd/libw4a16.so`` with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
HEADERS = ["w4a16_layout.h", "w4a16_device.h", "w4a16_internal.h", "w4a16_epilogue.h",
           "w4a8_internal.h", "w4a8_device.h", "mx_internal.h"]

COMMON = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-fp32 instructions (v_pk_{add,mul,fma}_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]

# (source, extra defines): the kernel sources are compiled
# once per (activation dtype, epilogue) pair so that their kernel
# instantiations compile in parallel.
UNITS = [
    ("w4a16_api.cpp", []),
    ("w4a16_repack.hip", []),
    ("w4a16_noalloc.hip", []),
    ("w4a16_gemm.hip", ["-DW4A16_TU_BF16=0", "-DW4A16_TU_EP=0"]),
    ("w4a16_gemm.hip", ["-DW4A16_TU_BF16=1", "-DW4A16_TU_EP=0"]),
    ("w4a16_gemm.hip", ["-DW4A16_TU_BF16=0", "-DW4A16_TU_EP=1"]),
    ("w4a16_gemm.hip", ["-DW4A16_TU_BF16=1", "-DW4A16_TU_EP=1"]),
    ("w4a16_decode.hip", ["-DW4A16_TU_BF16=0", "-DW4A16_TU_EP=0"]),
    ("w4a16_decode.hip", ["-DW4A16_TU_BF16=1", "-DW4A16_TU_EP=0"]),
    ("w4a16_decode.hip", ["-DW4A16_TU_BF16=0", "-DW4A16_TU_EP=1"]),
    ("w4a16_decode.hip", ["-DW4A16_TU_BF16=1", "-DW4A16_TU_EP=1"]),
    ("w4a16_wide.hip", ["-DW4A16_TU_BF16=0", "-DW4A16_TU_EP=0"]),
    ("w4a16_wide.hip", ["-DW4A16_TU_BF16=1", "-DW4A16_TU_EP=0"]),
    ("w4a16_wide.hip", ["-DW4A16_TU_BF16=0", "-DW4A16_TU_EP=1"]),
    ("w4a16_wide.hip", ["-DW4A16_TU_BF16=1", "-DW4A16_TU_EP=1"]),
    ("w4a8_api.cpp", []),
    ("w4a8_prep.hip", []),
    ("w4a8_gemm.hip", ["-DW4A8_TU_OUT=0"]),
    ("w4a8_gemm.hip", ["-DW4A8_TU_OUT=1"]),
    ("w4a8_gemm.hip", ["-DW4A8_TU_OUT=2"]),
    ("mx_api.cpp", []),
    ("mx_prep.hip", []),
    ("mx_gemm.hip", ["-DMXFP4_TU_BF16=0"]),
    ("mx_gemm.hip", ["-DMXFP4_TU_BF16=1"]),
]


def _filter(text: str):
    return [ln for ln in text.splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + f".tmp{os.getpid()}"
    with tempfile.TemporaryDirectory(prefix="w4a16_build_") as td:
        procs, objs = [], []
        for i, (src, defs) in enumerate(UNITS):
            obj = os.path.join(td, f"{i}_{os.path.splitext(src)[0]}.o")
            cmd = [hipcc, *COMMON, *defs, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                          text=True))
            objs.append(obj)
        msgs, failed = [], False
        for pr in procs:
            out, _ = pr.communicate()
            msgs += _filter(out)
            failed |= pr.returncode != 0
        if failed:
            raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
        cmd = [hipcc, *COMMON, "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        msgs += _filter(res.stdout + res.stderr)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
