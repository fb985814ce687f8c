"""Build libusw.so (host encoder + gfx950 kernels) in-tree with hipcc.

Usage: python -m unstructured_sparse_weight_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libusw.so")

SOURCES = ["usw_host.cpp", "usw_reorder.cpp", "usw_spmm.hip", "usw_union.hip", "usw_cbc.hip", "usw_encode.hip", "usw_prefill.hip", "usw_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
    # the LDS-DMA helper sets M0 itself; nothing else in these kernels keeps a value there
    "-Wno-inline-asm",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP toolchain is required to build libusw")


def build(verbose: bool = False, tuning: bool = False) -> str:
    """Compile every source into libusw.so next to this file; returns its path.

    ``tuning`` also compiles the alternative decode launch configurations,
    selected at run time by the USW_DECODE_CFG environment variable.
    """
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmp = LIB + ".tmp"
    extra = ["-DUSW_TUNING"] if tuning else []
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True, tuning="--tuning" in sys.argv[1:]))
