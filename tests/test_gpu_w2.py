"""GPU parity of the 2-bit (W2) IE-BME payload: usw_union_spmm on 64 x 64
and 16 x 64 LTs (plain and reordered) against the CPU oracle on the same
seeded inputs.

Integer-exact inputs (2-bit codes with power-of-two scales, small-integer
X) must match the oracle bit for bit; general inputs must pass the oracle's
acceptance test against the dequantised 2-bit weight.
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
I2 = ob.VAL_I2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def gpu(h, X, out=torch.float32, splits=0):
    enc = usw.union_to_device(h, DEV)
    x = torch.from_numpy(np.ascontiguousarray(X)).to(DEV)
    y = usw.union_spmm(enc, x, out_dtype=out, splits=splits)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def ref(W, mask, X, lt=(64, 64)):
    Wd = ou.dense_weight_union(ou.encode_union(W, mask, lt[0], lt[1], 2, 2, I2))
    return ob.spmm_fp64(Wd, X), ob.abs_bound(Wd, X)


def exact_case(M, K, N, keep, seed):
    rng = np.random.default_rng(seed)
    mask = wl.mask_bernoulli(M, K, keep, rng)
    W = wl.weight_int2_exact(M, K, rng, mask)
    X = wl.activations_small_int(N, K, rng)
    return W, mask, X


def encode(W, mask, layout):
    if layout == "lt64":
        return usw.union_encode_host(W, mask, (64, 64), (2, 2), "i2")
    if layout == "lt16":
        return usw.union_encode_host(W, mask, (16, 64), (2, 2), "i2")
    perms, _, _ = usw.union_reorder(W, mask, (16, 64), (2, 2))
    return usw.union_encode_host(W, mask, (16, 64), (2, 2), "i2", perm=perms)


@pytest.mark.parametrize("N", [1, 2, 8, 16, 17, 32, 40, 64, 80])
@pytest.mark.parametrize("layout", ["lt64", "lt16", "lt16_reordered"])
def test_w2_integer_exact_bitwise(N, layout):
    M, K = 320, 1024
    W, mask, X = exact_case(M, K, N, 0.5, 300 + N)
    say(f"[w2] {layout} {M}x{K} N={N}")
    h = encode(W, mask, layout)
    Yref, _ = ref(W, mask, X)
    # The weights quantise exactly, so the oracle's product is W's own.
    assert np.array_equal(Yref, ob.spmm_fp64(np.where(mask, W, np.float16(0)), X))
    assert np.array_equal(gpu(h, X, torch.float32), Yref)
    assert np.array_equal(gpu(h, X, torch.float16), Yref.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("layout", ["lt64", "lt16"])
@pytest.mark.parametrize("splits", [1, 3, 8])
def test_w2_forced_splits_bitwise_and_repeatable(layout, splits):
    M, K, N = 256, 2048, 16
    W, mask, X = exact_case(M, K, N, 0.4, 400 + splits)
    h = encode(W, mask, layout)
    Yref, _ = ref(W, mask, X)
    Ya = gpu(h, X, splits=splits)
    assert np.array_equal(Ya, Yref)
    assert np.array_equal(gpu(h, X, splits=splits), Ya)


@pytest.mark.parametrize("keep", [0.0, 0.05, 1.0])
@pytest.mark.parametrize("layout", ["lt64", "lt16_reordered"])
def test_w2_density_edges(keep, layout):
    M, K, N = 128, 512, 8
    W, mask, X = exact_case(M, K, N, keep, 500 + int(100 * keep))
    h = encode(W, mask, layout)
    Yref, _ = ref(W, mask, X)
    assert np.array_equal(gpu(h, X), Yref)


@pytest.mark.parametrize("layout", ["lt64", "lt16", "lt16_reordered"])
def test_w2_general_inputs(layout):
    M, K, N = 1024, 2048, 16
    rng = np.random.default_rng(6)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_magnitude(W, 0.5)
    X = wl.activations_normal(N, K, rng)
    h = encode(W, mask, layout)
    Y = gpu(h, X, torch.float16)
    Yref, Bnd = ref(W, mask, X)
    ok, rel, worst = ob.compare(Y, Yref, Bnd)
    say(f"[w2] general {layout}: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok


def test_w2_full_size_ffn_up():
    """OPT-13B FFN-up 20480 x 5120 at 50% magnitude pruning with 2-bit codes,
    N = 2: general inputs within the tolerance, integer-exact bit for bit."""
    W, mask, X = wl.config_case(5, 20480, 5120, 2, 0.5)
    h = encode(W, mask, "lt64")
    Y = gpu(h, X, torch.float16)
    Yref, Bnd = ref(W, mask, X)
    ok, rel, worst = ob.compare(Y, Yref, Bnd)
    say(f"[w2] FFN-up N=2: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok
    rng = np.random.default_rng(78)
    We = wl.weight_int2_exact(20480, 5120, rng, mask)
    Xe = wl.activations_small_int(2, 5120, rng)
    he = encode(We, mask, "lt64")
    Yr, _ = ref(We, mask, Xe)
    assert np.array_equal(gpu(he, Xe), Yr)
