"""GPU parity of the reordered IE-BME path: bitmap-aware row reordering
(usw_union_reorder), the reordered encoder (usw_union_encode_reordered) and
the 16 x 64-LT union kernel (usw_union_spmm with a rowmap), against the CPU
oracle's product of the original W.

Reordering changes neither the surviving weights nor the product, so the
product of the reordered encoding must equal the oracle product of W
itself: bit for bit on integer-exact inputs (INT4 codes with power-of-two
scales, small-integer X), within the oracle's acceptance test otherwise.
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


def gpu(h, X, out=torch.float32, splits=0):
    enc = usw.union_to_device(h, DEV)
    x = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    y = usw.union_spmm(enc, x, out_dtype=out, splits=splits)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def plain_ref(W, mask, X):
    """The oracle product of W itself (no reordering): INT4 codes and scales
    of W's rows, dequantised, fp64 sums."""
    Wd = ob.dense_weight(ob.encode_i4(W, mask))
    return ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X)


def exact_case(M, K, N, keep, seed):
    rng = np.random.default_rng(seed)
    mask = wl.mask_bernoulli(M, K, keep, rng)
    W = wl.weight_int4_exact(M, K, rng, mask)
    X = wl.activations_small_int(N, K, rng)
    return W, mask, X


def random_perms(M, K, seed):
    rng = np.random.default_rng(seed)
    return np.array([rng.permutation(16) for _ in range((M // 16) * (K // 64))], dtype=np.int32)


@pytest.mark.parametrize("N", [1, 2, 8, 16, 17, 32, 40])
@pytest.mark.parametrize("order", ["solver", "random", "none"])
def test_reordered_integer_exact_bitwise(N, order):
    M, K = 320, 1024
    W, mask, X = exact_case(M, K, N, 0.5, 40 + N)
    say(f"[reordered] {M}x{K} N={N} order={order}")
    if order == "solver":
        perms, before, after = usw.union_reorder(W, mask, (16, 64), (2, 2))
        assert after.sum() <= before.sum()
    elif order == "random":
        perms = random_perms(M, K, N)
    else:
        perms = None
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    Yref, _ = plain_ref(W, mask, X)
    assert np.array_equal(gpu(h, X, torch.float32), Yref)
    assert np.array_equal(gpu(h, X, torch.float16), Yref.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16])
def test_reordered_forced_splits_bitwise_and_repeatable(splits):
    M, K, N = 256, 1024, 16
    W, mask, X = exact_case(M, K, N, 0.4, 70 + splits)
    perms = random_perms(M, K, splits)
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    Yref, _ = plain_ref(W, mask, X)
    Ya = gpu(h, X, splits=splits)
    assert np.array_equal(Ya, Yref)
    assert np.array_equal(gpu(h, X, splits=splits), Ya)


@pytest.mark.parametrize("keep", [0.0, 0.05, 1.0])
def test_reordered_density_edges(keep):
    M, K, N = 128, 512, 8
    W, mask, X = exact_case(M, K, N, keep, 90 + int(100 * keep))
    perms = random_perms(M, K, 3)
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    Yref, _ = plain_ref(W, mask, X)
    assert np.array_equal(gpu(h, X), Yref)


def test_reordered_general_inputs_tolerance():
    M, K, N = 1024, 2048, 16
    rng = np.random.default_rng(5)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_magnitude(W, 0.5)
    X = wl.activations_normal(N, K, rng)
    perms, _, _ = usw.union_reorder(W, mask, (16, 64), (2, 2))
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    Y = gpu(h, X, torch.float16)
    Yref, Bnd = plain_ref(W, mask, X)
    ok, rel, worst = ob.compare(Y, Yref, Bnd)
    say(f"[reordered] general 1024x2048 N=16: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok
    # The oracle of the reordered encoding gives the same dense weight.
    o = ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, ob.VAL_I4)
    assert np.array_equal(ou.dense_weight_union(o), ob.dense_weight(ob.encode_i4(W, mask)))


def test_reordered_full_size_ffn_up_int4():
    """OPT-13B FFN-up 20480 x 5120 at 50% magnitude pruning, INT4, N = 2 (the
    low-bit workload), reordered with the solver's row orders: general inputs
    within the tolerance, integer-exact inputs bit for bit."""
    W, mask, X = wl.config_case(5, 20480, 5120, 2, 0.5)
    perms, before, after = usw.union_reorder(W, mask, (16, 64), (2, 2))
    say(f"[reordered] FFN-up actives {int(before.sum())} -> {int(after.sum())}")
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    assert h.payload == 4 * int(after.sum())
    Y = gpu(h, X, torch.float16)
    Yref, Bnd = plain_ref(W, mask, X)
    ok, rel, worst = ob.compare(Y, Yref, Bnd)
    say(f"[reordered] FFN-up N=2: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok
    rng = np.random.default_rng(77)
    We = wl.weight_int4_exact(20480, 5120, rng, mask)
    Xe = wl.activations_small_int(2, 5120, rng)
    he = usw.union_encode_host(We, mask, (16, 64), (2, 2), "i4", perm=perms)
    Yr, _ = plain_ref(We, mask, Xe)
    assert np.array_equal(gpu(he, Xe, torch.float32), Yr)
