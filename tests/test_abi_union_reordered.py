"""CPU tests of the reordered IE-BME entry points (usw_union_encode_reordered
and its query): the host encoder writes exactly the oracle's bytes and row
map for any row order and for the solver's, the validator checks row maps,
and argument errors return before anything is launched.  No kernel is
launched here."""
import ctypes

import numpy as np
import pytest

import unstructured_sparse_weight_amd as usw
import workloads as wl
from oracle import ie_bme as ou
from oracle import tca_bme as ob

VT = {"f16": ob.VAL_F16, "i4": ob.VAL_I4}
B = ctypes.byref


def assert_same(h, o):
    assert h.payload == o.payload
    assert np.array_equal(h.bitmaps, o.bitmaps)
    assert np.array_equal(h.offsets, o.offsets)
    vb = o.values.view(np.uint8).reshape(-1)
    assert h.values_bytes == vb.size
    assert np.array_equal(h.values[: h.values_bytes], vb)
    assert not h.values[h.values_bytes:].any()
    if o.scales is not None:
        assert np.array_equal(h.scales, o.scales.view(np.uint16))
    assert np.array_equal(h.rowmap, o.rowmap.reshape(-1))


def random_perms(nlt, h, seed):
    rng = np.random.default_rng(seed)
    return np.array([rng.permutation(h) for _ in range(nlt)], dtype=np.int32)


@pytest.mark.parametrize("lt,areas", [((16, 64), (2, 2)), ((8, 64), (2, 2)), ((16, 64), (4, 1)), ((12, 32), (3, 2))])
@pytest.mark.parametrize("dtype", ["f16", "i4"])
@pytest.mark.parametrize("density", [0.0, 0.4, 1.0])
def test_reordered_encoder_matches_oracle(lt, areas, dtype, density):
    M, K = 4 * lt[0] * 2, 3 * lt[1]
    rng = np.random.default_rng(lt[0] + areas[0] + int(10 * density))
    W = wl.weight_normal(M, K, rng)
    W[rng.random((M, K)) < 0.05] = np.float16(-0.0)
    mask = wl.mask_bernoulli(M, K, density, rng)
    nlt = (M // lt[0]) * (K // lt[1])
    perms = random_perms(nlt, lt[0], 3)
    h = usw.union_encode_host(W, mask, lt, areas, dtype, perm=perms)
    o = ou.encode_union_reordered(W, mask, perms, lt[0], lt[1], areas[0], areas[1], VT[dtype])
    assert_same(h, o)
    usw.union_validate(h)


def test_solver_orders_match_oracle_and_shrink_the_payload():
    M, K = 256, 512
    rng = np.random.default_rng(21)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_magnitude(W, 0.5)
    perms, before, after = usw.union_reorder(W, mask, (16, 64), (2, 2))
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    o = ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, ob.VAL_I4)
    assert_same(h, o)
    plain = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4")
    assert h.payload == 4 * int(after.sum()) <= plain.payload == 4 * int(before.sum())


@pytest.mark.slow
def test_full_size_ffn_up_int4_matches_oracle():
    """OPT-13B FFN-up 20480 x 5120, 50% magnitude pruning, INT4, 16 x 64 LTs
    with the solver's row orders: the same bytes as the oracle."""
    W, mask, _ = wl.config_case(5, 20480, 5120, 2, 0.5)
    perms, before, after = usw.union_reorder(W, mask, (16, 64), (2, 2))
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    o = ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, ob.VAL_I4)
    assert_same(h, o)
    assert h.payload == 4 * int(after.sum())


def test_validate_checks_the_rowmap():
    M, K = 64, 128
    rng = np.random.default_rng(4)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    perms = random_perms(8, 16, 5)
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    L = usw.lib()
    assert L.usw_union_validate(B(h.fmt())) == 0
    bad = h.rowmap.copy()
    bad[17] = bad[18]                       # LT 1: a repeated stored row
    f = h.fmt()
    f.rowmap = bad.ctypes.data
    assert L.usw_union_validate(B(f)) == -8
    bad = h.rowmap.copy()
    bad[5] = 16                             # out of range
    f.rowmap = bad.ctypes.data
    assert L.usw_union_validate(B(f)) == -8


@pytest.mark.host_pointers
def test_reordered_argument_errors():
    L = usw.lib()
    M, K = 128, 128
    rng = np.random.default_rng(6)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    perms = random_perms(16, 16, 7)
    pl, bv, ba = ctypes.c_int64(), ctypes.c_size_t(), ctypes.c_size_t()
    mask8 = mask.astype(np.uint8)                               # kept alive across the calls
    wp, mp = W.ctypes.data, mask8.ctypes.data
    args = (M, K, 16, 64, 2, 2, 2)
    assert L.usw_union_encode_reordered_query(wp, mp, *args, perms.ctypes.data, B(pl), B(bv), B(ba)) == 0
    assert L.usw_union_encode_reordered_query(wp, mp, *args, None, B(pl), B(bv), B(ba)) == -1
    bad = perms.copy()
    bad[3, 0] = bad[3, 1]
    assert L.usw_union_encode_reordered_query(wp, mp, *args, bad.ctypes.data, B(pl), B(bv), B(ba)) == -2
    bad = perms.copy()
    bad[0, 0] = 16
    assert L.usw_union_encode_reordered_query(wp, mp, *args, bad.ctypes.data, B(pl), B(bv), B(ba)) == -2
    bm = np.zeros(16 * 4, np.uint64)
    off = np.zeros(17, np.uint32)
    vals = np.zeros(ba.value, np.uint8)
    sc = np.zeros(M, np.uint16)
    rm = np.zeros(16 * 16, np.uint8)
    assert L.usw_union_encode_reordered(wp, mp, *args, perms.ctypes.data, bm.ctypes.data, off.ctypes.data,
                                        vals.ctypes.data, vals.size, sc.ctypes.data, None) == -1
    assert L.usw_union_encode_reordered(wp, mp, *args, perms.ctypes.data, bm.ctypes.data, off.ctypes.data,
                                        vals.ctypes.data, 4, sc.ctypes.data, rm.ctypes.data) == -10
    assert L.usw_union_encode_reordered(wp, mp, *args, perms.ctypes.data, bm.ctypes.data, off.ctypes.data,
                                        vals.ctypes.data, vals.size, sc.ctypes.data, rm.ctypes.data) == 0
    # product entry points: LTs shorter than 64 rows need M a multiple of
    # 64; row maps run on LTs of 16, 32 and 64 rows
    h = usw.union_encode_host(W, mask, (16, 64), (2, 2), "i4", perm=perms)
    sz = ctypes.c_size_t()
    assert L.usw_union_spmm_workspace(B(h.fmt()), 8, 0, B(sz)) == 0
    f = h.fmt()
    f.M = 80
    assert L.usw_union_spmm_workspace(B(f), 8, 0, B(sz)) == -5
    h64 = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4")
    f = h64.fmt()
    f.rowmap = rm.ctypes.data
    assert L.usw_union_spmm_workspace(B(f), 8, 0, B(sz)) == 0
    h8 = usw.union_encode_host(W, mask, (8, 64), (2, 2), "i4", perm=random_perms(128 // 8 * 2, 8, 8))
    f = h8.fmt()
    assert L.usw_union_spmm_workspace(B(f), 8, 0, B(sz)) == -5
    x = np.zeros((8, K), np.uint16)
    y = np.zeros((8, M), np.uint16)
    assert L.usw_union_spmm(B(f), x.ctypes.data, y.ctypes.data, 1, 8, 0, None, 0, None) == -5
