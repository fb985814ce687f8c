"""GPU parity of the IE-BME union-mask INT4 kernel (usw_union_spmm, called
through the C ABI) against the CPU oracle of the union format on the same
seeded inputs.

Floating-point outputs must pass the oracle's acceptance test; integer-exact
inputs (INT4 codes with power-of-two scales, small-integer X) must match the
oracle bit for bit, whatever the summation order.
"""
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


def run_union(W, mask, X, out=torch.float16, splits=0, host=None):
    h = host if host is not None else usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4")
    enc = usw.union_to_device(h, DEV)
    x = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    y = usw.union_spmm(enc, x, out_dtype=out, splits=splits)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def union_ref(W, mask, X):
    Wd = ou.dense_weight_union(ou.encode_union(W, mask, 64, 64, 2, 2, ob.VAL_I4))
    return ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X)


def exact_case(M, K, N, keep, seed):
    rng = np.random.default_rng(seed)
    mask = wl.mask_bernoulli(M, K, keep, rng)
    W = wl.weight_int4_exact(M, K, rng, mask)
    X = wl.activations_small_int(N, K, rng)
    return W, mask, X


def assert_exact(W, mask, X, what, splits=0):
    say(f"[union] {what}")
    Yref, _ = union_ref(W, mask, X)
    Y32 = run_union(W, mask, X, out=torch.float32, splits=splits)
    assert np.array_equal(Y32, Yref), what
    Y16 = run_union(W, mask, X, out=torch.float16, splits=splits)
    assert np.array_equal(Y16, Yref.astype(np.float16).astype(np.float64)), what


def assert_parity(Y, Yref, Bnd, what):
    ok, rel, worst = ob.compare(Y, Yref, Bnd)
    say(f"[union parity] {what}: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok, f"{what}: rel_l2={rel:.3e} worst={worst:.3f}"


@pytest.mark.parametrize("out", [torch.float16, torch.float32])
def test_union_tiny(out):
    W, mask, X = wl.config_case(1, 256, 256, 8, 0.5)
    Y = run_union(W, mask, X, out=out)
    Yref, Bnd = union_ref(W, mask, X)
    assert_parity(Y, Yref, Bnd, f"tiny out={out}")


def test_union_tiny_integer_exact_bitwise():
    W, mask, X = exact_case(256, 256, 8, 0.5, 12)
    assert_exact(W, mask, X, "tiny exact")


@pytest.mark.parametrize("N", [1, 2, 3, 15, 16, 17, 31, 32, 33, 48, 64, 65, 70, 100, 128])
def test_union_ragged_n(N):
    W, mask, X = exact_case(192, 640, N, 0.5, 100 + N)
    assert_exact(W, mask, X, f"N={N}")


@pytest.mark.parametrize("N", [80, 90])
def test_union_short_last_pass_with_its_own_split_factor(N):
    """200 strips of 24 LT columns: the 64-token pass takes one split, the
    shorter last pass two, so only the last pass uses the workspace."""
    W, mask, X = exact_case(64 * 200, 64 * 24, N, 0.5, 400 + N)
    assert_exact(W, mask, X, f"N={N}")


@pytest.mark.parametrize("N,splits", [(64, 3), (100, 2)])
def test_union_64_token_passes_with_split_k(N, splits):
    """Passes of 64 tokens (four token blocks per wave) with split K."""
    W, mask, X = exact_case(256, 2048, N, 0.5, 300 + N)
    assert_exact(W, mask, X, f"N={N} splits={splits}", splits=splits)


@pytest.mark.parametrize("shape", [(64, 64), (64, 1024), (1024, 64), (192, 320), (128, 4096), (64, 32768)])
def test_union_shapes(shape):
    M, K = shape
    W, mask, X = exact_case(M, K, 5, 0.45, M + K)
    assert_exact(W, mask, X, f"shape={shape}")


@pytest.mark.parametrize("kind", ["empty", "full", "single", "row", "col", "one_area"])
def test_union_degenerate_masks(kind):
    """Empty (no payload at all), fully kept (1024 active positions per LT,
    the largest payload), a single weight, one row, one column, and a mask
    confined to one area of every LT (three all-zero streams)."""
    M, K, N = 128, 512, 9
    rng = np.random.default_rng(7)
    mask = np.zeros((M, K), dtype=bool)
    if kind == "full":
        mask[:] = True
    elif kind == "single":
        mask[77, 301] = True
    elif kind == "row":
        mask[40, :] = True
    elif kind == "col":
        mask[:, 200] = True
    elif kind == "one_area":
        sub = rng.random((M, K)) < 0.5
        for ti in range(M // 64):
            for tj in range(K // 64):
                mask[ti * 64 + 32:ti * 64 + 64, tj * 64:tj * 64 + 32] = sub[ti * 64:ti * 64 + 32, tj * 64:tj * 64 + 32]
    W = wl.weight_int4_exact(M, K, rng, mask)
    X = wl.activations_small_int(N, K, rng)
    assert_exact(W, mask, X, f"mask={kind}")


@pytest.mark.parametrize("splits", [1, 2, 3, 5])
def test_union_forced_splits_and_determinism(splits):
    rng = np.random.default_rng(31 + splits)
    M, K, N = 320, 2048, 16
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    W = wl.weight_normal(M, K, rng)
    X = wl.activations_normal(N, K, rng)
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4")
    Y1 = run_union(W, mask, X, out=torch.float32, splits=splits, host=h)
    Y2 = run_union(W, mask, X, out=torch.float32, splits=splits, host=h)
    assert np.array_equal(Y1, Y2)
    Yref, Bnd = union_ref(W, mask, X)
    assert_parity(Y1, Yref, Bnd, f"splits={splits}")


def test_union_counters_reset_across_calls():
    """Split-K counters come back to zero: repeated calls on one workspace
    give the same bits."""
    W, mask, X = exact_case(256, 4096, 16, 0.5, 55)
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4")
    enc = usw.union_to_device(h, DEV)
    x = torch.from_numpy(X).to(DEV)
    ys = [usw.union_spmm(enc, x, out_dtype=torch.float32, splits=4).cpu().numpy() for _ in range(4)]
    torch.cuda.synchronize()
    Yref, _ = union_ref(W, mask, X)
    for y in ys:
        assert np.array_equal(y.astype(np.float64), Yref)


def test_union_agrees_with_tca_bme_int4():
    """Both formats hold the same quantised W_sp: with integer-exact inputs
    their GPU results are the same bits."""
    W, mask, X = exact_case(512, 1024, 16, 0.5, 77)
    Yu = run_union(W, mask, X, out=torch.float32)
    h = usw.encode_host(W, mask, (64, 64), "i4")
    enc = usw.to_device(h, DEV)
    Yt = usw.spmm(enc, torch.from_numpy(X).to(DEV), out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    assert np.array_equal(Yu, Yt)


@pytest.mark.parametrize("N", [2, 16])
def test_union_int4_layer(N):
    """INT4 FFN-up 20480 x 5120, magnitude 50% (the INT4 workload), in the
    launch configuration the benchmark times."""
    M, K = 20480, 5120
    W, mask, X = wl.config_case(5, M, K, N, 0.5)
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4")
    Y = run_union(W, mask, X, host=h)
    Yref, Bnd = union_ref(W, mask, X)
    assert_parity(Y, Yref, Bnd, f"int4 ffn_up union N={N}")


def test_union_full_size_integer_exact_bitwise():
    W, mask, X = exact_case(20480, 5120, 16, 0.5, 98)
    assert_exact(W, mask, X, "full size exact")
