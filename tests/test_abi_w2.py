"""CPU tests of the 2-bit (W2) IE-BME payload in the C-ABI library: the host
encoder (plain and reordered LTs) writes exactly the oracle's bytes, the
validator accepts it, TCA-BME entry points refuse it, and the product entry
point sizes its workspace.  No kernel is launched here."""
import ctypes

import numpy as np
import pytest

import unstructured_sparse_weight_amd as usw
import workloads as wl
from oracle import ie_bme as ou
from oracle import tca_bme as ob

B = ctypes.byref


def assert_same(h, o):
    assert h.payload == o.payload
    assert np.array_equal(h.bitmaps, o.bitmaps)
    assert np.array_equal(h.offsets, o.offsets)
    vb = o.values.view(np.uint8).reshape(-1)
    assert h.values_bytes == vb.size == (o.payload + 3) // 4
    assert np.array_equal(h.values[: h.values_bytes], vb)
    assert not h.values[h.values_bytes:].any()
    assert np.array_equal(h.scales, o.scales.view(np.uint16))
    if o.rowmap is not None:
        assert np.array_equal(h.rowmap, o.rowmap.reshape(-1))


@pytest.mark.parametrize("lt,areas", [((64, 64), (2, 2)), ((16, 64), (2, 2)), ((32, 64), (2, 1)), ((64, 32), (1, 1))])
@pytest.mark.parametrize("density", [0.0, 0.3, 1.0])
def test_w2_union_encoder_matches_oracle(lt, areas, density):
    rng = np.random.default_rng(int(10 * density) + lt[0] + areas[0])
    M, K = 128, 256
    W = wl.weight_normal(M, K, rng)
    W[rng.random((M, K)) < 0.05] = np.float16(-0.0)
    mask = wl.mask_bernoulli(M, K, density, rng)
    h = usw.union_encode_host(W, mask, lt, areas, "i2")
    o = ou.encode_union(W, mask, lt[0], lt[1], areas[0], areas[1], ob.VAL_I2)
    assert_same(h, o)
    usw.union_validate(h)


def test_w2_ties_and_non_finite_match_oracle():
    W = np.zeros((64, 64), dtype=np.float16)
    W[0, :6] = [3.0, 1.5, -1.5, 2.0, -2.0, 0.75]
    W[1, :3] = [0.5, np.inf, -0.25]
    W[2, :3] = [0.5, np.nan, -0.25]
    mask = W != 0
    mask[2, 1] = True
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i2")
    o = ou.encode_union(W, mask, 64, 64, 2, 2, ob.VAL_I2)
    assert_same(h, o)
    assert h.scales[0] == np.float16(3.0).view(np.uint16)


def test_w2_reordered_matches_oracle():
    rng = np.random.default_rng(8)
    M, K = 128, 256
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_magnitude(W, 0.5)
    perms, _, after = usw.union_reorder(W, mask, (16, 64), (2, 2))
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i2", perm=perms)
    o = ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, ob.VAL_I2)
    assert_same(h, o)
    assert h.payload == 4 * int(after.sum())


@pytest.mark.slow
def test_w2_full_size_ffn_up_matches_oracle():
    W, mask, _ = wl.config_case(5, 20480, 5120, 2, 0.5)
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i2")
    o = ou.encode_union(W, mask, 64, 64, 2, 2, ob.VAL_I2)
    assert_same(h, o)


@pytest.mark.host_pointers
def test_w2_entry_points():
    L = usw.lib()
    rng = np.random.default_rng(9)
    W = wl.weight_normal(256, 512, rng)
    mask = wl.mask_bernoulli(256, 512, 0.5, rng)
    # TCA-BME takes fp16 and INT4 only
    nnz = ctypes.c_int64()
    assert L.usw_encode_query(W.ctypes.data, None, 256, 512, 64, 64, 3, B(nnz), None, None, None, None, None) == -3
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i2")
    f = h.fmt()
    assert f.val_type == 3
    sz = ctypes.c_size_t()
    assert L.usw_union_spmm_workspace(B(f), 8, 2, B(sz)) == 0 and sz.value == 256 + 2 * 16 * 256 * 4
    f.scales = None
    x = np.zeros((8, 512), np.uint16)
    y = np.zeros((8, 256), np.uint16)
    assert L.usw_union_spmm(B(f), x.ctypes.data, y.ctypes.data, 1, 8, 0, None, 0, None) == -1
    assert L.usw_union_validate(B(f)) == -1
