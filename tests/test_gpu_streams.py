"""GPU tests of the workspace contract and of calls on several streams.

The split-K kernels take the last workgroup of an output tile from per-tile
counters at the start of the workspace: those bytes must be zero when a call
starts (each call leaves them zero), the partial sums after them need no
initialisation, and calls that may run at the same time need separate
workspaces.  These tests hold the C ABI and the Python binding to that,
against the CPU oracle.
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


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    Wd = ob.dense_weight(ob.encode(W, mask))
    return W, mask, X, ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X)


def check(Y, Yref, Bnd, what):
    ok, rel, worst = ob.compare(Y, Yref, Bnd)
    say(f"[streams] {what}: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok, f"{what}: rel_l2={rel:.3e} worst={worst:.3f}"


def sizes(L, f, N, splits):
    need, cb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.usw_spmm_workspace_ex(ctypes.byref(f), N, splits, ctypes.byref(need)) == 0
    assert L.usw_spmm_counter_bytes(ctypes.byref(f), N, splits, ctypes.byref(cb)) == 0
    return need.value, cb.value


@pytest.mark.parametrize("N", [16, 24, 512])
def test_abi_only_counters_need_zero(N):
    """A workspace whose counter bytes (usw_spmm_counter_bytes) are zero and
    whose partial-sum bytes hold garbage gives the oracle's Y with split K;
    the call leaves the counters zero."""
    L = usw.lib()
    M, K = 1024, 4096
    W, mask, X, Yref, Bnd = case(M, K, N, 600 + N)
    enc = usw.to_device(usw.encode_host(W, mask), DEV)
    f = enc.fmt()
    need, cb = sizes(L, f, N, 4)
    assert need > cb > 0
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=DEV)
    ws[:cb].zero_()
    x = torch.from_numpy(X).to(DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for rep in range(2):
        y = torch.empty((N, M), dtype=torch.float32, device=DEV)
        assert L.usw_spmm_ex(ctypes.byref(f), x.data_ptr(), y.data_ptr(), 3, N, 4, ws.data_ptr(), need, stream) == 0
        torch.cuda.synchronize()
        assert not ws[:cb].any()
        check(y.cpu().numpy().astype(np.float64), Yref, Bnd, f"garbage partials N={N} rep={rep}")


def test_abi_two_streams_separate_workspaces():
    """Two matrices multiplied on two streams at the same time, each call with
    its own workspace (split K on both), several rounds without a host
    synchronisation in between: both outputs match the oracle every round."""
    L = usw.lib()
    K, N = 5120, 16
    cases = [case(2048, K, N, 610), case(3072, K, N, 611)]
    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    setup = []
    for (W, mask, X, _, _), st in zip(cases, streams):
        enc = usw.to_device(usw.encode_host(W, mask), DEV)
        f = enc.fmt()
        need, cb = sizes(L, f, N, 5)
        assert need > cb > 0
        ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
        x = torch.from_numpy(X).to(DEV)
        setup.append((enc, f, ws, need, x, st))
    torch.cuda.synchronize()
    rounds = 4
    outs = [[torch.empty((N, c[0].shape[0]), dtype=torch.float16, device=DEV) for _ in range(rounds)] for c in cases]
    torch.cuda.synchronize()
    for r in range(rounds):
        for i, (enc, f, ws, need, x, st) in enumerate(setup):
            rc = L.usw_spmm_ex(ctypes.byref(f), x.data_ptr(), outs[i][r].data_ptr(), 1, N, 5, ws.data_ptr(), need,
                               ctypes.c_void_p(st.cuda_stream))
            assert rc == 0
    torch.cuda.synchronize()
    for i, (_, _, _, Yref, Bnd) in enumerate(cases):
        for r in range(rounds):
            check(outs[i][r].float().cpu().numpy().astype(np.float64), Yref, Bnd, f"stream {i} round {r}")


def test_python_side_stream_counter_size_changes():
    """The binding on a non-default stream: matrices of different M and N
    (so different counter sizes, decode and prefill) in turn, with the
    binding's per-stream workspace growing and its counters re-cleared on the
    launch stream; every output matches the oracle."""
    side = torch.cuda.Stream(device=DEV)
    seq = [(1024, 2048, 16), (4096, 2048, 16), (1024, 2048, 8), (2048, 2048, 600), (4096, 2048, 16)]
    results = []
    for i, (M, K, N) in enumerate(seq):
        W, mask, X, Yref, Bnd = case(M, K, N, 620 + i)
        enc = usw.to_device(usw.encode_host(W, mask), DEV)
        x = torch.from_numpy(X).to(DEV)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            y = torch.empty((N, M), dtype=torch.float16, device=DEV)
        usw.spmm(enc, x, y=y, splits=4 if N <= 32 else 0, stream=side)
        results.append((y, Yref, Bnd, f"side stream M={M} N={N}"))
        # No synchronisation between the calls: the side stream orders them.
    torch.cuda.synchronize()
    for y, Yref, Bnd, what in results:
        check(y.float().cpu().numpy().astype(np.float64), Yref, Bnd, what)


def test_python_two_streams_get_separate_workspaces():
    """The binding's workspace cache is keyed by (device, stream): two streams
    never share one, and a stream keeps its own across calls."""
    W, mask, X, Yref, Bnd = case(1024, 4096, 16, 630)
    enc = usw.to_device(usw.encode_host(W, mask), DEV)
    x = torch.from_numpy(X).to(DEV)
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    for s in (s1, s2):
        s.wait_stream(torch.cuda.current_stream())
    y1 = usw.spmm(enc, x, splits=4, stream=s1)
    y2 = usw.spmm(enc, x, splits=4, stream=s2)
    torch.cuda.synchronize()
    k1 = (str(torch.device(DEV)), int(s1.cuda_stream))
    k2 = (str(torch.device(DEV)), int(s2.cuda_stream))
    assert k1 in usw._WS and k2 in usw._WS
    assert usw._WS[k1][0].data_ptr() != usw._WS[k2][0].data_ptr()
    for y, what in ((y1, "stream 1"), (y2, "stream 2")):
        check(y.float().cpu().numpy().astype(np.float64), Yref, Bnd, what)
