"""GPU parity: the HIP kernels (called through the C ABI) against the CPU
oracle on the same seeded inputs.

Floating-point outputs must pass the oracle's acceptance test (relative L2
error <= 1e-3 and |error| <= 2e-3 * sum|w||x| per output); integer-exact
inputs (dyadic W, small-integer X, power-of-two INT4 scales) must match the
oracle bit for bit, whatever the summation order.
"""
import ctypes
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import ie_bme as ou
from oracle import tca_bme as ob

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import unstructured_sparse_weight_amd as usw  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_gpu(W, mask, X, dtype="f16", out=torch.float16, splits=0, host=None):
    h = host if host is not None else usw.encode_host(W, mask, (64, 64), dtype)
    enc = usw.to_device(h, DEV)
    x = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    y = usw.spmm(enc, x, out_dtype=out, splits=splits)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def oracle_ref(W, mask, X, dtype="f16", rows=None):
    enc = (ob.encode if dtype == "f16" else ob.encode_i4)(W, mask)
    Wd = ob.dense_weight(enc)
    Xs = X if rows is None else X[rows]
    return ob.spmm_fp64(Wd, Xs), ob.abs_bound(Wd, Xs)


def assert_parity(Y, Yref, Bnd, what):
    ok, rel, worst = ob.compare(Y, Yref, Bnd)
    say(f"[parity] {what}: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok, f"{what}: rel_l2={rel:.3e} worst={worst:.3f}"


# ---------------------------------------------------------------------------
# Tiny workload and edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("out", [torch.float16, torch.float32])
def test_tiny(out):
    W, mask, X = wl.config_case(1, 256, 256, 8, 0.5)
    Y = run_gpu(W, mask, X, out=out)
    Yref, Bnd = oracle_ref(W, mask, X)
    assert_parity(Y, Yref, Bnd, f"tiny out={out}")


@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_tiny_integer_exact_bitwise(dtype):
    W, mask, X = wl.config_case(1, 256, 256, 8, 0.5, exact=True)
    if dtype == "i4":
        W = wl.weight_int4_exact(256, 256, np.random.default_rng(12), mask)
    Y32 = run_gpu(W, mask, X, dtype, out=torch.float32)
    Yref, _ = oracle_ref(W, mask, X, dtype)
    assert np.array_equal(Y32, Yref)
    Y16 = run_gpu(W, mask, X, dtype, out=torch.float16)
    assert np.array_equal(Y16, Yref.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("N,splits", [(33, 0), (64, 0), (64, 3), (100, 0), (128, 2)])
@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_four_block_passes_integer_exact_bitwise(dtype, N, splits):
    """Decode passes of up to 64 tokens (four 16-token blocks per wave), alone
    and followed by a shorter pass, with and without split K: on
    integer-exact inputs every partial sum is exact, so Y equals the fp64
    oracle bit for bit."""
    M, K = 320, 1024
    W, mask, X = wl.config_case(1, M, K, N, 0.5, exact=True)
    if dtype == "i4":
        W = wl.weight_int4_exact(M, K, np.random.default_rng(30 + N), mask)
    Yref, _ = oracle_ref(W, mask, X, dtype)
    assert np.array_equal(run_gpu(W, mask, X, dtype, out=torch.float32, splits=splits), Yref)
    assert np.array_equal(run_gpu(W, mask, X, dtype, out=torch.float16, splits=splits),
                          Yref.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("N", [80, 90])
@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_short_last_pass_with_its_own_split_factor_bitwise(dtype, N):
    """200 strips of 24 GroupTile columns: a 64-token pass takes one split
    (one workgroup per compute unit), the shorter last pass (16 or 26
    tokens) two, so only the last pass uses the split-K workspace."""
    M, K = 64 * 200, 64 * 24
    W, mask, X = wl.config_case(1, M, K, N, 0.5, exact=True)
    if dtype == "i4":
        W = wl.weight_int4_exact(M, K, np.random.default_rng(40 + N), mask)
    Yref, _ = oracle_ref(W, mask, X, dtype)
    assert np.array_equal(run_gpu(W, mask, X, dtype, out=torch.float32), Yref)
    assert np.array_equal(run_gpu(W, mask, X, dtype, out=torch.float16), Yref.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("N", [1, 2, 3, 7, 15, 16, 17, 24, 31, 32, 33, 40, 48, 63, 64, 65, 80, 96, 97, 112, 128,
                               129])
def test_ragged_n(N):
    rng = np.random.default_rng(100 + N)
    M, K = 320, 448          # 5 x 7 GroupTiles: uneven column ranges per wave
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    Y = run_gpu(W, mask, X)
    Yref, Bnd = oracle_ref(W, mask, X)
    assert_parity(Y, Yref, Bnd, f"ragged N={N}")


@pytest.mark.parametrize("shape", [(64, 64), (64, 1024), (1024, 64), (192, 320), (128, 4096), (64, 32768)])
@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_shapes(shape, dtype):
    M, K = shape
    rng = np.random.default_rng(M * 7 + K)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.4, rng)
    X = wl.activations_normal(5, K, rng)
    Y = run_gpu(W, mask, X, dtype)
    Yref, Bnd = oracle_ref(W, mask, X, dtype)
    assert_parity(Y, Yref, Bnd, f"shape {shape} {dtype}")


@pytest.mark.parametrize("dtype", ["f16", "i4"])
@pytest.mark.parametrize("density", [0.0, 1.0, "single", "row", "col"])
def test_degenerate_masks(dtype, density):
    M, K, N = 128, 512, 9
    rng = np.random.default_rng(55)
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
    else:
        mask = np.full((M, K), bool(density))
    X = wl.activations_normal(N, K, rng)
    Y = run_gpu(W, mask, X, dtype)
    Yref, Bnd = oracle_ref(W, mask, X, dtype)
    if not mask.any():
        assert not Y.any()
    assert_parity(Y, Yref, Bnd, f"mask {density} {dtype}")


def test_kept_zeros_and_negative_zero():
    rng = np.random.default_rng(66)
    M, K, N = 128, 256, 4
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.6, rng)
    W[rng.random((M, K)) < 0.2] = np.float16(0.0)
    W[rng.random((M, K)) < 0.2] = np.float16(-0.0)
    X = wl.activations_normal(N, K, rng)
    Y = run_gpu(W, mask, X)
    Yref, Bnd = oracle_ref(W, mask, X)
    assert_parity(Y, Yref, Bnd, "kept zeros")


@pytest.mark.parametrize("density", [0.8, 0.97])
@pytest.mark.parametrize("splits", [0, 1, 2])
def test_dense_groups(density, splits):
    """GroupTiles denser than a pipeline slot holds are staged in halves."""
    rng = np.random.default_rng(int(density * 100) + splits)
    M, K, N = 512, 2048, 16
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, density, rng)
    X = wl.activations_normal(N, K, rng)
    h = usw.encode_host(W, mask)
    Y = run_gpu(W, mask, X, splits=splits, host=h)
    Yref, Bnd = oracle_ref(W, mask, X)
    assert_parity(Y, Yref, Bnd, f"density {density} splits={splits}")


@pytest.mark.parametrize("N", [1, 16, 24])
def test_dense_groups_in_a_sparse_matrix(N):
    """A matrix at most 55% dense on average gets the five-chunk value slot;
    its few GroupTiles too dense for that slot (70% here) send their waves
    down the two-half path, one at 60% still fits.  Integer-exact inputs, so
    bit for bit."""
    rng = np.random.default_rng(300 + N)
    M, K = 256, 1024            # 4 x 16 GroupTiles
    W = wl.weight_dyadic(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.45, rng)
    mask[64:128, 192:384] = rng.random((64, 192)) < 0.7     # GroupTiles (1, 3..5)
    mask[192:256, 640:704] = rng.random((64, 64)) < 0.6     # GroupTile (3, 10)
    assert mask.mean() <= 0.55
    X = wl.activations_small_int(N, K, rng)
    Y = run_gpu(W, mask, X, out=torch.float32)
    Wd = np.where(mask, W, np.float16(0))
    assert np.array_equal(Y, ob.spmm_fp64(Wd, X))


def test_split_k_counters_reset_across_calls():
    """Repeated split-K calls on one workspace (per-strip counters, XCD remap
    with 8 | workgroups) give identical bits every time."""
    rng = np.random.default_rng(78)
    M, K, N = 1024, 3072, 16      # 16 strips x 4 splits = 64 workgroups
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    enc = usw.to_device(usw.encode_host(W, mask), DEV)
    x = torch.from_numpy(X).to(DEV)
    outs = [usw.spmm(enc, x, splits=4).float().cpu().numpy() for _ in range(5)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    Yref, Bnd = oracle_ref(W, mask, X)
    assert_parity(outs[0].astype(np.float64), Yref, Bnd, "split-K repeated")


def test_workspace_reuse_across_shapes():
    """Through the C ABI: one zero-filled workspace serves a small-M then a
    larger-M matrix once the counter bytes the header names are re-zeroed,
    and two calls in a row on the same matrix need nothing in between."""
    import ctypes
    L = usw.lib()
    K, N = 3072, 16
    ws = torch.zeros(1 << 22, dtype=torch.uint8, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for M in (512, 2048, 2048):
        rng = np.random.default_rng(M)
        W = wl.weight_normal(M, K, rng)
        mask = wl.mask_bernoulli(M, K, 0.5, rng)
        X = wl.activations_normal(N, K, rng)
        enc = usw.to_device(usw.encode_host(W, mask), DEV)
        f = enc.fmt()
        x = torch.from_numpy(X).to(DEV)
        y = torch.empty((N, M), dtype=torch.float16, device=DEV)
        need = usw.spmm_workspace_bytes(enc, N, 4)
        assert 0 < need <= ws.numel()
        st = L.usw_spmm_ex(ctypes.byref(f), x.data_ptr(), y.data_ptr(), 1, N, 4, ws.data_ptr(), ws.numel(), stream)
        assert st == 0
        torch.cuda.synchronize()
        counter_bytes = (4 * (M // 64) + 255) // 256 * 256
        assert not ws[:counter_bytes].any()          # the call left its counters at zero
        Yref, Bnd = oracle_ref(W, mask, X)
        assert_parity(y.float().cpu().numpy().astype(np.float64), Yref, Bnd, f"workspace reuse M={M}")
        ws[:counter_bytes * 4].zero_()               # next shape may have larger counters


@pytest.mark.parametrize("splits", [1, 2, 3, 5])
def test_forced_splits_and_determinism(splits):
    rng = np.random.default_rng(77)
    M, K, N = 256, 1280, 16
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    h = usw.encode_host(W, mask)
    Ya = run_gpu(W, mask, X, splits=splits, host=h)
    Yb = run_gpu(W, mask, X, splits=splits, host=h)
    assert np.array_equal(Ya, Yb)
    Yref, Bnd = oracle_ref(W, mask, X)
    assert_parity(Ya, Yref, Bnd, f"splits={splits}")


# ---------------------------------------------------------------------------
# Full-size workloads
# ---------------------------------------------------------------------------

_CACHE = {}


def layer(config_id, name, M, K, s, N, layer_id):
    key = (config_id, name, s, layer_id)
    if key not in _CACHE:
        _CACHE.clear()
        W, mask, _ = wl.config_case(config_id, M, K, 1, s, layer_id=layer_id)
        _CACHE[key] = (W, mask)
    W, mask = _CACHE[key]
    X = wl.activations_normal(N, K, wl.seed_rng(config_id, layer_id, 2 + N))
    return W, mask, X


OPT = list(wl.LAYERS_OPT13B.items())


@pytest.mark.parametrize("lid", range(len(OPT)), ids=[n for n, _ in OPT])
def test_opt13b_decode_layers(lid):
    name, (M, K) = OPT[lid]
    W, mask, _ = layer(2, name, M, K, 0.5, 1, lid)
    h = usw.encode_host(W, mask)
    enc = ob.encode(W, mask)
    Wd = ob.decode(enc).astype(np.float64)
    for N in (1, 8, 16):
        X = wl.activations_normal(N, K, wl.seed_rng(2, lid, 2 + N))
        Y = run_gpu(W, mask, X, host=h)
        assert_parity(Y, ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X), f"opt13b {name} N={N}")


@pytest.mark.parametrize("s", [0.3, 0.4, 0.5, 0.6, 0.7])
def test_sparsity_sweep(s):
    M, K = 20480, 5120
    W, mask, _ = layer(3, "ffn_up", M, K, s, 1, int(s * 10))
    say(f"[sweep] realised sparsity {1 - mask.mean():.4f}")
    h = usw.encode_host(W, mask)
    Wd = ob.decode(ob.encode(W, mask)).astype(np.float64)
    for N in (1, 16, 32):
        X = wl.activations_normal(N, K, wl.seed_rng(3, int(s * 10), 2 + N))
        Y = run_gpu(W, mask, X, host=h)
        assert_parity(Y, ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X), f"sweep s={s} N={N}")


@pytest.mark.parametrize("lid,name", [(0, "up"), (1, "down")])
def test_prefill_layers(lid, name):
    M, K = wl.LAYERS_PREFILL[name]
    W, mask, _ = layer(4, name, M, K, 0.5, 1, lid)
    h = usw.encode_host(W, mask)
    Wd = ob.decode(ob.encode(W, mask)).astype(np.float64)
    for N in (512, 2048):
        X = wl.activations_normal(N, K, wl.seed_rng(4, lid, 2 + N))
        Y = run_gpu(W, mask, X, host=h)
        rows = np.random.default_rng(N).choice(N, 48, replace=False)
        rows.sort()
        Xs = X[rows]
        assert_parity(Y[rows], ob.spmm_fp64(Wd, Xs), ob.abs_bound(Wd, Xs), f"prefill {name} N={N} (48 sampled rows)")


@pytest.mark.parametrize("N", [33, 48, 100])
def test_int4_many_tokens(N):
    """INT4 values with more than 32 tokens run in 32-token decode passes;
    power-of-two scales and small-integer X make the result exact, so bit
    for bit against the oracle."""
    rng = np.random.default_rng(400 + N)
    M, K = 320, 448
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    W = wl.weight_int4_exact(M, K, rng, mask)
    X = wl.activations_small_int(N, K, rng)
    Y = run_gpu(W, mask, X, "i4", out=torch.float32)
    Yref, _ = oracle_ref(W, mask, X, "i4")
    assert np.array_equal(Y, Yref)


def test_int4_layer():
    M, K = 20480, 5120
    W, mask, X = wl.config_case(5, M, K, 2, 0.5)
    h = usw.encode_host(W, mask, (64, 64), "i4")
    enc = ob.encode_i4(W, mask)
    Wd = ob.dense_weight(enc)
    Y = run_gpu(W, mask, X, "i4", host=h)
    assert_parity(Y, ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X), "int4 ffn_up N=2")


def test_full_size_integer_exact_bitwise():
    M, K, N = 20480, 5120, 16
    rng = np.random.default_rng(99)
    W = wl.weight_dyadic(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_small_int(N, K, rng)
    Y = run_gpu(W, mask, X, out=torch.float32)
    Wd = np.where(mask, W, np.float16(0))
    assert np.array_equal(Y, ob.spmm_fp64(Wd, X))


def test_probe_read_runs():
    """The streaming-read probe bench.py reports the memory-bound kernels
    against: it reads a device buffer and returns OK; a ragged byte count
    reads the whole 16-byte units only."""
    L = usw.lib()
    buf = torch.randint(0, 255, (3 * 262144 + 100,), dtype=torch.uint8, device=DEV)
    sink = torch.zeros(8, dtype=torch.int32, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.usw_probe_read(buf.data_ptr(), buf.numel(), sink.data_ptr(), stream) == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("N", [2, 24])
@pytest.mark.parametrize("fmt", ["tca", "union"])
def test_low_bit_offset_cancels_on_large_activations(fmt, N):
    """The low-bit kernels multiply code + 72 and take 72 times X's column
    sums back out; activations with a large common offset (N(40, 1)) make
    those sums large.  The result must still pass the oracle's acceptance
    test (one token block: the matrix-core correction; two: v_dot2)."""
    M, K = 1024, 5120
    rng = np.random.default_rng(470 + N)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_magnitude(W, 0.5)
    X = (40.0 + rng.normal(0.0, 1.0, size=(N, K))).astype(np.float16)
    x = torch.from_numpy(X).to(DEV)
    if fmt == "tca":
        Y = run_gpu(W, mask, X, "i4", out=torch.float32)
        Yref, Bnd = oracle_ref(W, mask, X, "i4")
    else:
        enc = usw.union_to_device(usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4"), DEV)
        Y = usw.union_spmm(enc, x, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
        Wd = ou.dense_weight_union(ou.encode_union(W, mask, 64, 64, 2, 2, ob.VAL_I4))
        Yref, Bnd = ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X)
    assert_parity(Y, Yref, Bnd, f"{fmt} INT4 N={N}, activations N(40, 1)")
