"""GPU parity of the Tiled-CBC spMspV with dynamic pruning (usw_cbc_spmspv,
called through the C ABI) against the CPU oracle of the format on the same
seeded inputs.

Floating-point outputs must pass the oracle's acceptance test; integer-exact
inputs (dyadic W, small-integer x) must match the oracle bit for bit.
"""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import tca_bme as ob
from oracle import tiled_cbc as oc

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import unstructured_sparse_weight_amd as usw  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_cbc(W, mask, x, tau, out=torch.float16, splits=0, host=None):
    h = host if host is not None else usw.cbc_encode_host(W, mask)
    enc = usw.cbc_to_device(h, DEV)
    y = usw.cbc_spmspv(enc, torch.from_numpy(np.ascontiguousarray(x)).to(DEV), tau, out_dtype=out, splits=splits)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def cbc_ref(W, mask, x, tau):
    enc = oc.encode_cbc(W, mask)
    return oc.spmspv(enc, x, tau), oc.spmspv_bound(enc, x, tau)


def quantile_tau(x, dp):
    """Threshold that leaves a fraction dp of the columns inactive."""
    if dp <= 0:
        return 0.0
    return float(np.quantile(np.abs(x.astype(np.float32)), dp))


def assert_parity(y, yref, bnd, what):
    ok, rel, worst = ob.compare(y[None, :], yref[None, :], bnd[None, :])
    say(f"[cbc parity] {what}: rel_l2={rel:.3e} worst/bound={worst:.3f}")
    assert ok, f"{what}: rel_l2={rel:.3e} worst={worst:.3f}"


def exact_case(M, K, keep, seed):
    rng = np.random.default_rng(seed)
    W = wl.weight_dyadic(M, K, rng)
    mask = wl.mask_bernoulli(M, K, keep, rng)
    x = wl.activations_small_int(1, K, rng)[0]
    return W, mask, x


@pytest.mark.parametrize("dp", [0.0, 0.5, 0.9])
@pytest.mark.parametrize("out", [torch.float16, torch.float32])
def test_cbc_tiny(dp, out):
    rng = np.random.default_rng(3)
    W = wl.weight_normal(512, 256, rng)
    mask = wl.mask_bernoulli(512, 256, 0.5, rng)
    x = wl.activations_normal(1, 256, rng)[0]
    tau = quantile_tau(x, dp)
    y = run_cbc(W, mask, x, tau, out=out)
    yref, bnd = cbc_ref(W, mask, x, tau)
    assert_parity(y, yref, bnd, f"tiny dp={dp} out={out}")


@pytest.mark.parametrize("tau", [0.0, 1.0, 2.0, 3.0, 4.0])
def test_cbc_integer_exact_bitwise(tau):
    """Small-integer x: tau = 1, 2, 3 drop the columns below them (the
    boundary value itself is kept), tau = 4 drops every column."""
    W, mask, x = exact_case(768, 512, 0.5, 11)
    yref, _ = cbc_ref(W, mask, x, tau)
    y32 = run_cbc(W, mask, x, tau, out=torch.float32)
    assert np.array_equal(y32, yref)
    y16 = run_cbc(W, mask, x, tau, out=torch.float16)
    assert np.array_equal(y16, yref.astype(np.float16).astype(np.float64))
    if tau == 4.0:
        assert not y32.any()


@pytest.mark.parametrize("shape", [(256, 16), (256, 32), (512, 4096), (2048, 48), (256, 16384)])
def test_cbc_shapes(shape):
    M, K = shape
    W, mask, x = exact_case(M, K, 0.45, M + K)
    yref, _ = cbc_ref(W, mask, x, 2.0)
    assert np.array_equal(run_cbc(W, mask, x, 2.0, out=torch.float32), yref)


@pytest.mark.parametrize("kind", ["empty", "full", "single", "row", "col"])
def test_cbc_degenerate_masks(kind):
    M, K = 512, 128
    rng = np.random.default_rng(9)
    W = wl.weight_dyadic(M, K, rng)
    x = wl.activations_small_int(1, K, rng)[0]
    mask = np.zeros((M, K), dtype=bool)
    if kind == "full":
        mask[:] = True
    elif kind == "single":
        mask[300, 77] = True
    elif kind == "row":
        mask[129, :] = True
    elif kind == "col":
        mask[:, 45] = True
    for tau in (0.0, 2.0):
        yref, _ = cbc_ref(W, mask, x, tau)
        assert np.array_equal(run_cbc(W, mask, x, tau, out=torch.float32), yref), (kind, tau)


@pytest.mark.parametrize("splits", [1, 2, 7, 16])
def test_cbc_forced_splits_and_determinism(splits):
    rng = np.random.default_rng(40 + splits)
    M, K = 1024, 2048
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    x = wl.activations_normal(1, K, rng)[0]
    tau = quantile_tau(x, 0.5)
    h = usw.cbc_encode_host(W, mask)
    y1 = run_cbc(W, mask, x, tau, out=torch.float32, splits=splits, host=h)
    y2 = run_cbc(W, mask, x, tau, out=torch.float32, splits=splits, host=h)
    assert np.array_equal(y1, y2)
    yref, bnd = cbc_ref(W, mask, x, tau)
    assert_parity(y1, yref, bnd, f"splits={splits}")


def test_cbc_counters_reset_across_calls():
    W, mask, x = exact_case(512, 4096, 0.5, 55)
    h = usw.cbc_encode_host(W, mask)
    enc = usw.cbc_to_device(h, DEV)
    xt = torch.from_numpy(x).to(DEV)
    ys = [usw.cbc_spmspv(enc, xt, 1.0, out_dtype=torch.float32, splits=8).cpu().numpy() for _ in range(4)]
    yref, _ = cbc_ref(W, mask, x, 1.0)
    for y in ys:
        assert np.array_equal(y.astype(np.float64), yref)


def test_cbc_agrees_with_tca_bme_on_zeroed_x():
    """Skipping columns equals the TCA-BME kernel on x with those entries
    zeroed (integer-exact inputs: the same bits)."""
    W, mask, x = exact_case(1024, 2048, 0.5, 77)
    tau = 2.0
    y = run_cbc(W, mask, x, tau, out=torch.float32)
    xz = np.where(np.abs(x.astype(np.float32)) >= tau, x, np.float16(0))
    enc = usw.to_device(usw.encode_host(W, mask), DEV)
    yt = usw.spmm(enc, torch.from_numpy(xz[None, :]).to(DEV), out_dtype=torch.float32)[0].cpu().numpy()
    assert np.array_equal(y, yt.astype(np.float64))


@pytest.mark.parametrize("dp", [0.0, 0.5, 0.8])
def test_cbc_ffn_up_layer(dp):
    """FFN-up 20480 x 5120, magnitude 50%, one token, in the launch
    configuration the benchmark times."""
    W, mask, X = wl.config_case(2, 20480, 5120, 1, 0.5, layer_id=2)
    x = X[0]
    tau = quantile_tau(x, dp)
    h = usw.cbc_encode_host(W, mask)
    y = run_cbc(W, mask, x, tau, host=h)
    yref, bnd = cbc_ref(W, mask, x, tau)
    assert_parity(y, yref, bnd, f"ffn_up dp={dp}")


def test_cbc_full_size_integer_exact_bitwise():
    W, mask, x = exact_case(20480, 5120, 0.5, 98)
    yref, _ = cbc_ref(W, mask, x, 2.0)
    assert np.array_equal(run_cbc(W, mask, x, 2.0, out=torch.float32), yref)
