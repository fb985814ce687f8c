"""The C-ABI tests run against a build of the library whose host code is
instrumented with AddressSanitizer and UndefinedBehaviorSanitizer: the host
encoders (TCA-BME, IE-BME plain and reordered, Tiled-CBC), the validators,
the multithreaded parallel_for and the row-reordering solver, plus every
entry point's argument checks.  Any report aborts the run.

The instrumented library is built into a temporary directory (the GPU code is
compiled as usual; only host code is instrumented) and the ABI tests run in a
subprocess with the sanitizer runtime preloaded.  No kernel is launched.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ABI_TESTS = ["tests/test_abi.py", "tests/test_abi_union.py", "tests/test_abi_cbc.py", "tests/test_abi_reorder.py",
             "tests/test_abi_union_reordered.py", "tests/test_abi_w2.py", "tests/test_properties.py",
             "tests/test_store.py"]


def asan_runtime():
    clang = "/opt/rocm/llvm/bin/clang++"
    if not os.path.exists(clang):
        return None
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_abi_tests_pass_under_asan_and_ubsan(tmp_path):
    rt = asan_runtime()
    if rt is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("no HIP toolchain with the ASan runtime")
    sys.path.insert(0, ROOT)
    from unstructured_sparse_weight_amd import build
    lib = build.build(sanitize=True, out=str(tmp_path / "libusw_sanitized.so"))
    env = dict(os.environ)
    env.update({
        "USW_LIB_PATH": lib,
        "LD_PRELOAD": rt,
        "ASAN_OPTIONS": f"detect_leaks=0:abort_on_error=1:log_path={tmp_path}/asan",
        "UBSAN_OPTIONS": f"print_stacktrace=1:halt_on_error=1:log_path={tmp_path}/ubsan",
    })
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu and not slow",
                          *ABI_TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    reports = sorted(p for p in os.listdir(tmp_path) if p.startswith(("asan", "ubsan")))
    text = "".join(open(tmp_path / p).read() for p in reports)
    assert not reports, text[:4000]
    assert res.returncode == 0, (res.stdout[-3000:] + res.stderr[-3000:])
    assert " passed" in res.stdout
