"""GPU parity of IE-BME on general area grids: usw_union_spmm with LTs of 16,
32 and 64 rows by 64 columns, R_A x C_A grids other than 2 x 2 (and 2 x 2
with row maps on 32- and 64-row LTs), INT4 and 2-bit payloads, with and
without reordered rows, against the CPU oracle on the same seeded inputs.

Integer-exact inputs (codes with power-of-two scales, small-integer X) must
match the oracle bit for bit; general inputs must pass the oracle's
acceptance test.  The area grid only changes how the weights are stored, so
on integer-exact inputs the oracle's product is also W's own.
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
VT = {"i4": ob.VAL_I4, "i2": ob.VAL_I2}

# (LT rows, (R_A, C_A)): every LT height the kernels take, area columns from
# 64 down to 8 wide, area rows from the whole LT down to one row.
GRIDS = [
    (16, (1, 1)), (16, (4, 1)), (16, (1, 2)), (16, (4, 2)), (16, (2, 4)), (16, (1, 8)), (16, (16, 1)),
    (16, (8, 2)),
    (32, (2, 2)), (32, (4, 1)), (32, (1, 4)), (32, (8, 2)), (32, (32, 1)),
    (64, (1, 1)), (64, (4, 4)), (64, (8, 1)), (64, (1, 8)), (64, (64, 1)),
]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu(h, X, out=torch.float32, splits=0):
    enc = usw.union_to_device(h, DEV)
    x = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    y = usw.union_spmm(enc, x, out_dtype=out, splits=splits)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def random_perms(M, K, ltm, seed):
    rng = np.random.default_rng(seed)
    return np.array([rng.permutation(ltm) for _ in range((M // ltm) * (K // 64))], dtype=np.int32)


def encode_both(W, mask, ltm, areas, dtype, perms):
    """The host encoding and the oracle's encoding of the same format."""
    h = usw.union_encode_host(W, mask, (ltm, 64), areas, dtype, perm=perms)
    if perms is None:
        o = ou.encode_union(W, mask, ltm, 64, areas[0], areas[1], VT[dtype])
    else:
        o = ou.encode_union_reordered(W, mask, perms, ltm, 64, areas[0], areas[1], VT[dtype])
    assert h.payload == o.payload
    return h, o


def exact_case(M, K, N, keep, seed, dtype):
    rng = np.random.default_rng(seed)
    mask = wl.mask_bernoulli(M, K, keep, rng)
    W = (wl.weight_int4_exact if dtype == "i4" else wl.weight_int2_exact)(M, K, rng, mask)
    X = wl.activations_small_int(N, K, rng)
    return W, mask, X


@pytest.mark.parametrize("N", [1, 17])
@pytest.mark.parametrize("order", ["none", "random"])
@pytest.mark.parametrize("ltm,areas", GRIDS)
def test_grid_integer_exact_bitwise(ltm, areas, order, N):
    M, K = 256, 1024
    W, mask, X = exact_case(M, K, N, 0.5, 1000 + 7 * ltm + 3 * areas[0] + areas[1] + N, "i4")
    perms = random_perms(M, K, ltm, N) if order == "random" else None
    say(f"[grid] {ltm}x64 areas {areas[0]}x{areas[1]} order={order} N={N}")
    h, o = encode_both(W, mask, ltm, areas, "i4", perms)
    Wd = ou.dense_weight_union(o)
    assert np.array_equal(Wd, ob.dense_weight(ob.encode_i4(W, mask)))
    Yref = ob.spmm_fp64(Wd, X)
    assert np.array_equal(gpu(h, X, torch.float32), Yref)
    assert np.array_equal(gpu(h, X, torch.float16), Yref.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("ltm", [32, 64])
@pytest.mark.parametrize("N", [2, 40])
def test_two_by_two_with_rowmaps_bitwise(ltm, N):
    """2 x 2 areas on 32- and 64-row LTs with reordered rows run on the
    area-grid kernel."""
    M, K = 320, 1024
    W, mask, X = exact_case(M, K, N, 0.4, 1200 + ltm + N, "i4")
    h, o = encode_both(W, mask, ltm, (2, 2), "i4", random_perms(M, K, ltm, ltm + N))
    Yref = ob.spmm_fp64(ou.dense_weight_union(o), X)
    assert np.array_equal(gpu(h, X), Yref)


@pytest.mark.parametrize("order", ["none", "random"])
@pytest.mark.parametrize("ltm,areas", [(16, (4, 1)), (16, (1, 8)), (32, (1, 4)), (64, (4, 4)), (64, (1, 1))])
def test_grid_w2_bitwise(ltm, areas, order):
    M, K, N = 256, 1024, 8
    W, mask, X = exact_case(M, K, N, 0.5, 1300 + ltm + areas[0], "i2")
    perms = random_perms(M, K, ltm, 5) if order == "random" else None
    h, o = encode_both(W, mask, ltm, areas, "i2", perms)
    Yref = ob.spmm_fp64(ou.dense_weight_union(o), X)
    assert np.array_equal(Yref, ob.spmm_fp64(np.where(mask, W, np.float16(0)), X))
    assert np.array_equal(gpu(h, X), Yref)


@pytest.mark.parametrize("ltm,areas", [(16, (4, 1)), (32, (8, 2)), (64, (1, 8))])
@pytest.mark.parametrize("splits", [1, 3, 8])
def test_grid_forced_splits_bitwise_and_repeatable(ltm, areas, splits):
    M, K, N = 128, 2048, 16
    W, mask, X = exact_case(M, K, N, 0.4, 1400 + splits + ltm, "i4")
    h, o = encode_both(W, mask, ltm, areas, "i4", None)
    Yref = ob.spmm_fp64(ou.dense_weight_union(o), X)
    Ya = gpu(h, X, splits=splits)
    assert np.array_equal(Ya, Yref)
    assert np.array_equal(gpu(h, X, splits=splits), Ya)


@pytest.mark.parametrize("keep", [0.0, 0.03, 1.0])
@pytest.mark.parametrize("ltm,areas", [(16, (1, 1)), (32, (4, 2)), (64, (8, 1))])
def test_grid_density_edges(ltm, areas, keep):
    M, K, N = 128, 512, 8
    W, mask, X = exact_case(M, K, N, keep, 1500 + int(100 * keep) + ltm, "i4")
    h, o = encode_both(W, mask, ltm, areas, "i4", random_perms(M, K, ltm, 9))
    Yref = ob.spmm_fp64(ou.dense_weight_union(o), X)
    assert np.array_equal(gpu(h, X), Yref)


@pytest.mark.parametrize("ltm,areas", [(16, (4, 1)), (32, (1, 4)), (64, (4, 4))])
def test_grid_general_inputs(ltm, areas):
    M, K, N = 1024, 2048, 16
    rng = np.random.default_rng(16 + ltm)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_magnitude(W, 0.5)
    X = wl.activations_normal(N, K, rng)
    h, o = encode_both(W, mask, ltm, areas, "i4", None)
    Wd = ou.dense_weight_union(o)
    Y = gpu(h, X, torch.float16)
    ok, rel, worst = ob.compare(Y, ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X))
    say(f"[grid] general {ltm}x64 {areas}: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok


def test_grid_full_size_ffn_up_reordered():
    """OPT-13B FFN-up 20480 x 5120 at 50% magnitude pruning, INT4, 16 x 64
    LTs with 4 x 1 areas and the solver's row orders, N = 2: general inputs
    within the tolerance, integer-exact inputs bit for bit."""
    W, mask, X = wl.config_case(5, 20480, 5120, 2, 0.5)
    perms, before, after = usw.union_reorder(W, mask, (16, 64), (4, 1))
    assert after.sum() <= before.sum()
    h, o = encode_both(W, mask, 16, (4, 1), "i4", perms)
    Wd = ou.dense_weight_union(o)
    Y = gpu(h, X, torch.float16)
    ok, rel, worst = ob.compare(Y, ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X))
    say(f"[grid] FFN-up 16x64 4x1 reordered N=2: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok
    rng = np.random.default_rng(79)
    We = wl.weight_int4_exact(20480, 5120, rng, mask)
    Xe = wl.activations_small_int(2, 5120, rng)
    he, oe = encode_both(We, mask, 16, (4, 1), "i4", perms)
    assert np.array_equal(gpu(he, Xe), ob.spmm_fp64(ou.dense_weight_union(oe), Xe))


@pytest.mark.parametrize("M,K,N", [(64, 64, 1), (64, 64, 33), (128, 192, 5), (64, 4096, 16)])
@pytest.mark.parametrize("ltm,areas", [(16, (4, 1)), (32, (2, 4)), (64, (1, 1)), (64, (8, 8))])
def test_grid_small_and_ragged_shapes(M, K, N, ltm, areas):
    """One strip, one LT column, token counts across pass boundaries, and a
    single long strip: bit for bit on integer-exact inputs."""
    if (ltm // areas[0]) * (64 // areas[1]) % 64:
        pytest.skip("not a valid IE-BME grid")
    W, mask, X = exact_case(M, K, N, 0.5, 1600 + M + K + N + ltm, "i4")
    h, o = encode_both(W, mask, ltm, areas, "i4", random_perms(M, K, ltm, 11))
    Yref = ob.spmm_fp64(ou.dense_weight_union(o), X)
    assert np.array_equal(gpu(h, X), Yref)
    assert np.array_equal(gpu(h, X, torch.float16), Yref.astype(np.float16).astype(np.float64))
