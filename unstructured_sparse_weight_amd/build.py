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


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer: every flag
# applies to the host compilation only (the GPU code is built as usual).
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-shared-libsan", "-O1"]


DEBUG_LIB = os.path.join(PKG, "libusw_debug.so")


def build(verbose: bool = False, sanitize: bool = False, debug: bool = False, out: str = "") -> str:
    """Compile every source into libusw.so next to this file (or into
    ``out``); returns its path.

    ``sanitize`` instruments the host code with ASan and UBSan; such a build
    needs the sanitizer runtime preloaded and is meant for the CPU tests of
    the C ABI.  ``debug`` (-DUSW_DEBUG) poisons the kernels' LDS staging
    buffers with NaNs before use (libusw_debug.so, for the GPU test that
    checks no kernel reads LDS that no stage wrote).
    """
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    # Sanitized and debug builds never replace the product library.
    default = os.path.join(PKG, "libusw_sanitized.so") if sanitize else (DEBUG_LIB if debug else LIB)
    lib_path = out or default
    tmp = lib_path + ".tmp"
    extra = list(SANITIZE_FLAGS) if sanitize else []
    if debug:
        extra.append("-DUSW_DEBUG")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:], debug="--debug" in sys.argv[1:]))
