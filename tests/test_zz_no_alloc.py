"""GPU test of usw_spmm_noalloc, the entry point that allocates nothing: its
split-K counters and partial sums live in the library's static per-GPU
scratch array.  Through the C ABI it must give the same Y as usw_spmm_ex
(same kernels, same split factor, so the same bits) and pass the oracle's
acceptance test, on two calls in a row, the second with a smaller input,
for the decode (fp16 ring and per-wave kernels, INT4) and prefill kernels.
"""
import ctypes
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import tca_bme as ob

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import unstructured_sparse_weight_amd as usw  # noqa: E402

DEV = "cuda:0"
SCRATCH_BYTES = 16 << 20
SCRATCH_COUNTER_BYTES = 16 << 10


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def make(M, K, N, dtype, seed):
    rng = np.random.default_rng(seed)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    h = usw.encode_host(W, mask, (64, 64), dtype)
    enc = ob.encode(W, mask) if dtype == "f16" else ob.encode_i4(W, mask)
    Wd = ob.dense_weight(enc)
    return usw.to_device(h, DEV), torch.from_numpy(X).to(DEV), ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X)


def with_workspace(enc, x, splits, yt):
    """usw_spmm_ex with a fresh zero-filled workspace (the reference call)."""
    L = usw.lib()
    f = enc.fmt()
    N = x.shape[0]
    need = usw.spmm_workspace_bytes(enc, N, splits)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    y = torch.empty((N, enc.M), dtype=torch.float16 if yt == 1 else torch.float32, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.usw_spmm_ex(ctypes.byref(f), x.data_ptr(), y.data_ptr(), yt, N, splits, ws.data_ptr(), need, st) == 0
    torch.cuda.synchronize()
    return y


def no_alloc(enc, x, splits, yt):
    L = usw.lib()
    f = enc.fmt()
    N = x.shape[0]
    y = torch.empty((N, enc.M), dtype=torch.float16 if yt == 1 else torch.float32, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.usw_spmm_noalloc(ctypes.byref(f), x.data_ptr(), y.data_ptr(), yt, N, splits, st)
    assert rc == 0, usw.lib().usw_status_str(rc)
    torch.cuda.synchronize()
    return y


def fits(enc, N, splits):
    need = usw.spmm_workspace_bytes(enc, N, splits)
    cb = usw.spmm_counter_bytes(enc, N, splits)
    return cb <= SCRATCH_COUNTER_BYTES and need - cb <= SCRATCH_BYTES - SCRATCH_COUNTER_BYTES


# Pairs of calls in a row, the second on a smaller input: (M, K, N, values, splits).
CASES = [
    ("fp16 ring N=16 then smaller", (4096, 5120, 16, "f16", 0), (1024, 2048, 8, "f16", 0)),
    ("fp16 forced split then smaller", (2048, 4096, 16, "f16", 5), (512, 2048, 1, "f16", 3)),
    ("fp16 per-wave N=32 then ring", (3072, 4096, 32, "f16", 0), (2048, 2048, 16, "f16", 0)),
    ("INT4 N=2 then smaller", (4096, 5120, 2, "i4", 0), (1024, 1024, 2, "i4", 4)),
    ("prefill N=600 then decode", (2048, 2048, 600, "f16", 0), (1024, 2048, 16, "f16", 0)),
    ("prefill forced split then smaller", (1024, 4096, 300, "f16", 4), (512, 2048, 200, "f16", 2)),
]


@pytest.mark.parametrize("name,first,second", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("yt", [1, 3])
def test_noalloc_matches_workspace_call(name, first, second, yt):
    for i, (M, K, N, dt, splits) in enumerate((first, second)):
        say(f"[no-alloc] {name}: call {i} M={M} K={K} N={N} {dt} splits={splits} y_type={yt}")
        enc, x, Yref, Bnd = make(M, K, N, dt, 700 + 31 * i + M + N)
        eff = splits if (splits > 0 or fits(enc, N, 0)) else 1
        y_ref = with_workspace(enc, x, eff, yt)
        y = no_alloc(enc, x, splits, yt)
        a = y.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(a, y_ref.float().cpu().numpy().astype(np.float64)), f"{name} call {i}"
        ok, rel, worst = ob.compare(a, Yref, Bnd)
        say(f"[no-alloc]   rel_l2={rel:.3e} worst/bound={worst:.3f}")
        assert ok


def test_noalloc_repeated_and_after_workspace_calls():
    """The scratch keeps the last call's partial sums; calls of different
    counter sizes in turn, with usw_spmm_ex calls in between, stay exact."""
    seq = [(2048, 4096, 16, 4), (4096, 2048, 8, 2), (2048, 4096, 16, 4), (1024, 4096, 24, 3)]
    for i, (M, K, N, splits) in enumerate(seq):
        say(f"[no-alloc] sequence {i}: M={M} K={K} N={N} splits={splits}")
        enc, x, Yref, Bnd = make(M, K, N, "f16", 800 + i)
        y1 = no_alloc(enc, x, splits, 3)
        y2 = with_workspace(enc, x, splits, 3)
        y3 = no_alloc(enc, x, splits, 3)
        assert torch.equal(y1, y2) and torch.equal(y1, y3)
        ok, _, _ = ob.compare(y1.cpu().numpy().astype(np.float64), Yref, Bnd)
        assert ok


def test_noalloc_rejects_what_does_not_fit():
    """Partial sums beyond the scratch are refused before anything is
    launched (WORKSPACE); the automatic factor falls back to 1 instead."""
    L = usw.lib()
    M, K, N = 16384, 4096, 32
    rng = np.random.default_rng(900)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    enc = usw.to_device(usw.encode_host(W, mask), DEV)
    assert not fits(enc, N, 16)
    f = enc.fmt()
    x = torch.zeros((N, K), dtype=torch.float16, device=DEV)
    y = torch.empty((N, M), dtype=torch.float16, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.usw_spmm_noalloc(ctypes.byref(f), x.data_ptr(), y.data_ptr(), 1, N, 16, st)
    assert rc == -7                                  # USW_ERR_WORKSPACE
    torch.cuda.synchronize()


def test_noalloc_prefill_falls_back_to_256_token_tiles():
    """N > 256 whose 512-token kernel needs a copy of X larger than the
    scratch (1536 x 8192 fp16 = 24 MiB) runs on the 256-token prefill
    kernel, which needs no workspace at one split: bit for bit on
    integer-exact inputs, twice in a row, and within the tolerance on
    general inputs."""
    M, K, N = 512, 8192, 1100
    rng = np.random.default_rng(910)
    W = wl.weight_dyadic(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_small_int(N, K, rng)
    enc = usw.to_device(usw.encode_host(W, mask), DEV)
    assert not fits(enc, N, 1)
    say(f"[no-alloc] prefill fallback M={M} K={K} N={N}")
    x = torch.from_numpy(X).to(DEV)
    Yref = ob.spmm_fp64(np.where(mask, W, np.float16(0)), X)
    for _ in range(2):
        y = no_alloc(enc, x, 0, 3)
        assert np.array_equal(y.cpu().numpy().astype(np.float64), Yref)
    enc2, x2, Yref2, Bnd2 = make(M, K, N, "f16", 911)
    ok, rel, worst = ob.compare(no_alloc(enc2, x2, 0, 1).float().cpu().numpy().astype(np.float64), Yref2, Bnd2)
    say(f"[no-alloc]   general inputs rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok
