"""GPU parity of the prefill (MFMA) kernel, which usw_spmm takes for fp16
values and N > 32, against the CPU oracle on the same seeded inputs.

Same bar as the decode tests: the oracle's acceptance test for general
inputs, bit-for-bit equality for integer-exact inputs (dyadic W, small
integer X), and identical bits across repeated split-K calls.
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


def gpu(h, X, out=torch.float16, splits=0):
    enc = usw.to_device(h, DEV)
    x = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    y = usw.spmm(enc, x, out_dtype=out, splits=splits)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def ref(W, mask, X):
    Wd = ob.decode(ob.encode(W, mask)).astype(np.float64)
    return ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X)


def check(Y, Yref, Bnd, what):
    ok, rel, worst = ob.compare(Y, Yref, Bnd)
    say(f"[parity] {what}: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok, f"{what}: rel_l2={rel:.3e} worst={worst:.3f}"


@pytest.mark.parametrize("N", [33, 40, 64, 100, 255, 256, 257, 300, 511, 512, 513, 700])
def test_prefill_ragged_n(N):
    rng = np.random.default_rng(200 + N)
    M, K = 320, 448           # 5 x 7 GroupTiles
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    h = usw.encode_host(W, mask)
    Yref, Bnd = ref(W, mask, X)
    for out in (torch.float16, torch.float32):
        check(gpu(h, X, out), Yref, Bnd, f"prefill ragged N={N} out={out}")


@pytest.mark.parametrize("N,splits", [(48, 1), (48, 3), (300, 0), (512, 1), (512, 4), (1000, 2)])
def test_prefill_integer_exact_bitwise(N, splits):
    rng = np.random.default_rng(300 + N + splits)
    M, K = 256, 1024
    W = wl.weight_dyadic(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_small_int(N, K, rng)
    h = usw.encode_host(W, mask)
    Wd = np.where(mask, W, np.float16(0))
    Yref = ob.spmm_fp64(Wd, X)
    assert np.array_equal(gpu(h, X, torch.float32, splits), Yref)
    assert np.array_equal(gpu(h, X, torch.float16, splits), Yref.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 7, 16])
def test_prefill_forced_splits_and_determinism(splits):
    rng = np.random.default_rng(400 + splits)
    M, K, N = 192, 1024, 300
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    h = usw.encode_host(W, mask)
    Ya = gpu(h, X, torch.float32, splits)
    Yb = gpu(h, X, torch.float32, splits)
    assert np.array_equal(Ya, Yb)
    Yref, Bnd = ref(W, mask, X)
    check(Ya, Yref, Bnd, f"prefill splits={splits}")


@pytest.mark.parametrize("density", [0.0, 1.0, 0.97, "single", "row", "col"])
def test_prefill_masks(density):
    M, K, N = 128, 512, 96
    rng = np.random.default_rng(57)
    W = wl.weight_normal(M, K, rng)
    if density == "single":
        mask = np.zeros((M, K), bool)
        mask[77, 301] = True
    elif density == "row":
        mask = np.zeros((M, K), bool)
        mask[5, :] = True
    elif density == "col":
        mask = np.zeros((M, K), bool)
        mask[:, 511] = True
    elif density == 0.97:
        mask = wl.mask_bernoulli(M, K, 0.97, rng)
    else:
        mask = np.full((M, K), bool(density))
    X = wl.activations_normal(N, K, rng)
    h = usw.encode_host(W, mask)
    Yref, Bnd = ref(W, mask, X)
    for splits in (0, 2):
        Y = gpu(h, X, torch.float32, splits)
        if not mask.any():
            assert not Y.any()
        check(Y, Yref, Bnd, f"prefill mask {density} splits={splits}")


def test_prefill_kept_zeros():
    rng = np.random.default_rng(67)
    M, K, N = 128, 256, 80
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.6, rng)
    W[rng.random((M, K)) < 0.2] = np.float16(0.0)
    W[rng.random((M, K)) < 0.2] = np.float16(-0.0)
    X = wl.activations_normal(N, K, rng)
    Yref, Bnd = ref(W, mask, X)
    check(gpu(usw.encode_host(W, mask), X), Yref, Bnd, "prefill kept zeros")


@pytest.mark.parametrize("shape,N", [((64, 64), 100), ((1024, 64), 600), ((64, 65536), 40), ((64, 66560), 40)])
def test_prefill_shapes(shape, N):
    """One GroupTile column; many strips; 1024 columns (the most one
    workgroup streams); 1040 columns (forces two splits)."""
    M, K = shape
    rng = np.random.default_rng(M + K + N)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.4, rng)
    X = wl.activations_normal(N, K, rng)
    Yref, Bnd = ref(W, mask, X)
    check(gpu(usw.encode_host(W, mask), X), Yref, Bnd, f"prefill shape {shape} N={N}")


def test_prefill_workspace_reuse_across_counter_sizes():
    """The Python binding clears the counter bytes when a call's counter size
    differs from the previous call's on the shared workspace: alternate
    prefill and decode split-K calls of different shapes."""
    cases = []
    for (M, K, N, sp) in [(256, 4096, 512, 4), (1024, 3072, 16, 4), (512, 2048, 300, 3), (256, 4096, 512, 4)]:
        rng = np.random.default_rng(M + K + N)
        W = wl.weight_normal(M, K, rng)
        mask = wl.mask_bernoulli(M, K, 0.5, rng)
        X = wl.activations_normal(N, K, rng)
        cases.append((usw.encode_host(W, mask), W, mask, X, sp))
    for rep in range(2):
        for h, W, mask, X, sp in cases:
            Yref, Bnd = ref(W, mask, X)
            check(gpu(h, X, torch.float32, sp), Yref, Bnd, f"reuse M={h.M} N={X.shape[0]} rep={rep}")


def test_prefill_counters_via_c_abi():
    """Through the C ABI on a caller-owned workspace: each call leaves its
    counter bytes at zero, and calls in a row give identical bits."""
    L = usw.lib()
    rng = np.random.default_rng(81)
    M, K, N = 512, 4096, 512
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    enc = usw.to_device(usw.encode_host(W, mask), DEV)
    f = enc.fmt()
    need = ctypes.c_size_t()
    cb = ctypes.c_size_t()
    assert L.usw_spmm_workspace_ex(ctypes.byref(f), N, 0, ctypes.byref(need)) == 0
    assert L.usw_spmm_counter_bytes(ctypes.byref(f), N, 0, ctypes.byref(cb)) == 0
    assert need.value > cb.value > 0          # 8 strips x 1 token tile: split K
    ws = torch.zeros(need.value, dtype=torch.uint8, device=DEV)
    x = torch.from_numpy(X).to(DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    outs = []
    for _ in range(3):
        y = torch.empty((N, M), dtype=torch.float32, device=DEV)
        assert L.usw_spmm(ctypes.byref(f), x.data_ptr(), y.data_ptr(), 3, N, ws.data_ptr(), need.value, stream) == 0
        torch.cuda.synchronize()
        assert not ws[:cb.value].any()
        outs.append(y.cpu().numpy().astype(np.float64))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    Yref, Bnd = ref(W, mask, X)
    check(outs[0], Yref, Bnd, "prefill C ABI")


@pytest.mark.parametrize("N", [512, 2048])
@pytest.mark.parametrize("name", ["up", "down"])
def test_prefill_full_size_integer_exact_bitwise(name, N):
    """Llama-7B-shaped layer at N = 512 and 2048 (the prefill sizes), every
    output compared bit for bit."""
    M, K = wl.LAYERS_PREFILL[name]
    rng = np.random.default_rng((91 if name == "up" else 92) + 1000 * (N != 512))
    W = wl.weight_dyadic(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_small_int(N, K, rng)
    say(f"[prefill full-size] {name} {M}x{K} N={N}")
    Y = gpu(usw.encode_host(W, mask), X, torch.float32)
    Wd = np.where(mask, W, np.float16(0))
    assert np.array_equal(Y, ob.spmm_fp64(Wd, X))


# Work-split cases of the 512-token kernel (automatic split): the tile count a
# multiple of the workgroup count (whole tiles only), fewer tiles than
# workgroups (every tile split), whole rounds plus a split remainder, and a
# remainder too small to give every workgroup a column (one round goes back
# into the split part).
@pytest.mark.parametrize("M,K,N", [(4096, 512, 512), (1024, 1024, 600), (1280, 1024, 1100), (16448, 64, 512),
                                   (2048, 448, 1024)])
def test_prefill_stream_k_integer_exact_bitwise(M, K, N):
    rng = np.random.default_rng(M + 3 * K + N)
    W = wl.weight_dyadic(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_small_int(N, K, rng)
    say(f"[prefill stream-K] {M}x{K} N={N}")
    h = usw.encode_host(W, mask)
    Wd = np.where(mask, W, np.float16(0))
    Yref = ob.spmm_fp64(Wd, X)
    assert np.array_equal(gpu(h, X, torch.float32), Yref)
    assert np.array_equal(gpu(h, X, torch.float16), Yref.astype(np.float16).astype(np.float64))


def test_prefill_stream_k_deterministic():
    """Split tiles are summed in a fixed order: repeated calls give the same
    bits for general inputs."""
    rng = np.random.default_rng(123)
    M, K, N = 1280, 2048, 700
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    h = usw.encode_host(W, mask)
    Ya = gpu(h, X, torch.float32)
    Yb = gpu(h, X, torch.float32)
    assert np.array_equal(Ya, Yb)
    Yref, Bnd = ref(W, mask, X)
    check(Ya, Yref, Bnd, "prefill stream-K")


def test_prefill_ws_long_k_split():
    """N > 256 with K > 65536 (1040 GroupTile columns): more columns than the
    512-token kernel stages per workgroup, so the automatic split falls back
    from stream-K to split K (two splits); integer-exact, so bit for bit."""
    M, K, N = 64, 66560, 300
    rng = np.random.default_rng(515)
    W = wl.weight_dyadic(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_small_int(N, K, rng)
    say(f"[prefill long K] {M}x{K} N={N}")
    h = usw.encode_host(W, mask)
    Wd = np.where(mask, W, np.float16(0))
    assert np.array_equal(gpu(h, X, torch.float32), ob.spmm_fp64(Wd, X))
