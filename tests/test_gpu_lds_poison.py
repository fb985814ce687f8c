"""GPU test of the LDS-poisoning debug build (libusw_debug.so, -DUSW_DEBUG):
every kernel family fills its LDS staging buffers with fp16 NaNs at entry,
and the ring decode kernel refills each ring slot before its next loads.  A
kernel that read LDS no stage wrote, or read a slot before its load landed,
would put NaN into Y; here every family must still match the oracle (bit
for bit on integer-exact inputs) with no NaN anywhere.

The debug library is loaded beside the product library and called through
the same C ABI; it is never the product path.
"""
import ctypes
import os
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import ie_bme as ou
from oracle import tca_bme as ob
from oracle import tiled_cbc as oc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import unstructured_sparse_weight_amd as usw  # noqa: E402
from unstructured_sparse_weight_amd import _lib  # noqa: E402
from unstructured_sparse_weight_amd import build as _build  # noqa: E402

DEV = "cuda:0"
B = ctypes.byref


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dbg():
    if not os.path.exists(_build.DEBUG_LIB):
        pytest.fail(f"{_build.DEBUG_LIB} is missing: build() compiles it beside libusw.so")
    return _lib._declare(ctypes.CDLL(_build.DEBUG_LIB))


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def workspace(nbytes):
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=DEV)


def exact_case(M, K, N, keep, seed, i4=False):
    rng = np.random.default_rng(seed)
    mask = wl.mask_bernoulli(M, K, keep, rng)
    W = wl.weight_int4_exact(M, K, rng, mask) if i4 else wl.weight_dyadic(M, K, rng)
    X = wl.activations_small_int(N, K, rng)
    return W, mask, X


def check(y, Yref, what):
    a = y.float().cpu().numpy().astype(np.float64)
    say(f"[poison] {what}")
    assert not np.isnan(a).any(), what
    assert np.array_equal(a, Yref), what


# (M, K, N, keep, splits): the ring decode kernel (N <= 16, <= 55% dense), its
# unpipelined path (dense GroupTiles in a lean matrix), the per-wave kernel
# (17-32 tokens, denser matrices), and both prefill kernels (stream-K and
# split K).
TCA_CASES = [(1024, 2048, 16, 0.5, 0), (1024, 2048, 1, 0.5, 3), (512, 1024, 8, 0.5, 1),
             (1024, 2048, 24, 0.5, 0), (1024, 2048, 16, 0.8, 0), (640, 1024, 32, 0.3, 2),
             (1024, 1024, 200, 0.5, 0), (2048, 1024, 600, 0.5, 0), (1024, 2048, 300, 0.5, 3)]


@pytest.mark.parametrize("M,K,N,keep,splits", TCA_CASES)
def test_tca_bme_kernels_under_lds_poison(dbg, M, K, N, keep, splits):
    W, mask, X = exact_case(M, K, N, keep, M + K + N)
    if keep == 0.5 and N == 16 and splits == 0:
        # A few GroupTiles far denser than the rest: the ring kernel's
        # workgroups that meet them take the unpipelined path.
        mask[:64, :256] = True
    enc = usw.to_device(usw.encode_host(W, mask), DEV)
    f = enc.fmt()
    x = torch.from_numpy(X).to(DEV)
    y = torch.empty((N, M), dtype=torch.float32, device=DEV)
    need = usw.spmm_workspace_bytes(enc, N, splits)
    ws = workspace(need)
    assert dbg.usw_spmm_ex(B(f), x.data_ptr(), y.data_ptr(), 3, N, splits, ws.data_ptr(), need, stream()) == 0
    torch.cuda.synchronize()
    check(y, ob.spmm_fp64(np.where(mask, W, np.float16(0)), X), f"TCA-BME {M}x{K} N={N} keep={keep}")


@pytest.mark.parametrize("N", [2, 40])
def test_int4_kernel_under_lds_poison(dbg, N):
    M, K = 1024, 2048
    W, mask, X = exact_case(M, K, N, 0.5, 50 + N, i4=True)
    enc = usw.to_device(usw.encode_host(W, mask, (64, 64), "i4"), DEV)
    f = enc.fmt()
    x = torch.from_numpy(X).to(DEV)
    y = torch.empty((N, M), dtype=torch.float32, device=DEV)
    need = usw.spmm_workspace_bytes(enc, N, 0)
    ws = workspace(need)
    assert dbg.usw_spmm_ex(B(f), x.data_ptr(), y.data_ptr(), 3, N, 0, ws.data_ptr(), need, stream()) == 0
    torch.cuda.synchronize()
    check(y, ob.spmm_fp64(np.where(mask, W, np.float16(0)), X), f"INT4 N={N}")


@pytest.mark.parametrize("lt,areas,dtype,reorder", [((64, 64), (2, 2), "i4", False), ((16, 64), (2, 2), "i4", True),
                                                   ((64, 64), (2, 2), "i2", False), ((16, 64), (2, 2), "i2", True),
                                                   ((16, 64), (4, 1), "i4", True), ((32, 64), (1, 4), "i4", False),
                                                   ((64, 64), (4, 4), "i2", False)])
def test_union_kernels_under_lds_poison(dbg, lt, areas, dtype, reorder):
    M, K, N = 512, 2048, 16
    rng = np.random.default_rng(70 + lt[0])
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    W = (wl.weight_int4_exact if dtype == "i4" else wl.weight_int2_exact)(M, K, rng, mask)
    X = wl.activations_small_int(N, K, rng)
    perms = usw.union_reorder(W, mask, lt, areas)[0] if reorder else None
    enc = usw.union_to_device(usw.union_encode_host(W, mask, lt, areas, dtype, perm=perms), DEV)
    f = enc.fmt()
    x = torch.from_numpy(X).to(DEV)
    y = torch.empty((N, M), dtype=torch.float32, device=DEV)
    need, _ = usw.union_workspace_bytes(enc, N, 0)
    ws = workspace(need)
    assert dbg.usw_union_spmm(B(f), x.data_ptr(), y.data_ptr(), 3, N, 0, ws.data_ptr(), need, stream()) == 0
    torch.cuda.synchronize()
    check(y, ob.spmm_fp64(np.where(mask, W, np.float16(0)), X), f"union {lt} {areas} {dtype} reorder={reorder}")


def test_cbc_kernel_under_lds_poison(dbg):
    M, K = 1024, 2048
    rng = np.random.default_rng(90)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    W = wl.weight_dyadic(M, K, rng)
    x = wl.activations_small_int(1, K, rng)[0]
    tau = 2.0
    h = usw.cbc_encode_host(W, mask)
    enc = usw.cbc_to_device(h, DEV)
    f = enc.fmt()
    xd = torch.from_numpy(x).to(DEV)
    y = torch.empty(M, dtype=torch.float32, device=DEV)
    need, _ = usw.cbc_workspace_bytes(enc, 0)
    ws = workspace(need)
    assert dbg.usw_cbc_spmspv(B(f), xd.data_ptr(), y.data_ptr(), 3, tau, 0, ws.data_ptr(), need, stream()) == 0
    torch.cuda.synchronize()
    ref = oc.spmspv(oc.encode_cbc(W, mask), x, tau)
    check(y.reshape(1, -1), ref.reshape(1, -1), "Tiled-CBC tau=2")
