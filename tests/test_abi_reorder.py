"""CPU tests of usw_union_reorder (bitmap-aware row reordering of IE-BME
LTs, host C++): permutations and active counts equal the oracle's subset DP
exactly (same tie order), the minimum equals brute force on tiny LTs, and
the IE-BME encoding of the permuted matrix stores Q x the reported minimum."""
import ctypes
import time

import numpy as np
import pytest

import unstructured_sparse_weight_amd as usw
import workloads as wl
from oracle import row_reorder as rr


def masked(M, K, density, seed):
    rng = np.random.default_rng(seed)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, density, rng)
    return W, mask


@pytest.mark.parametrize("lt,areas,density", [((8, 64), (2, 2), 0.3), ((16, 64), (2, 2), 0.2),
                                              ((12, 32), (3, 2), 0.25), ((16, 64), (4, 1), 0.15),
                                              ((16, 32), (2, 1), 0.5), ((8, 128), (2, 2), 0.05),
                                              ((16, 64), (1, 2), 0.3)])
def test_reorder_matches_oracle(lt, areas, density):
    W, mask = masked(2 * lt[0], 2 * lt[1], density, lt[0] * 7 + lt[1] + areas[0])
    perm, before, after = usw.union_reorder(W, mask, lt, areas)
    operm, obefore, oafter = rr.reorder_matrix(mask, lt[0], lt[1], *areas)
    assert np.array_equal(perm, operm)
    assert np.array_equal(before, obefore)
    assert np.array_equal(after, oafter)


@pytest.mark.parametrize("seed", range(6))
def test_minimum_equals_brute_force(seed):
    W, mask = masked(8, 16, [0.1, 0.2, 0.3, 0.4, 0.5, 0.7][seed], 500 + seed)
    perm, before, after = usw.union_reorder(W, mask, (8, 16), (2, 1))
    assert after[0] == rr.brute_force_min(mask, 2, 1) <= before[0]


def test_null_mask_keeps_ieee_nonzeros():
    rng = np.random.default_rng(3)
    W = wl.weight_normal(32, 128, rng)
    W[rng.random(W.shape) < 0.7] = np.float16(0.0)
    W[rng.random(W.shape) < 0.05] = np.float16(-0.0)
    perm, before, after = usw.union_reorder(W, None, (16, 64), (2, 2))
    operm, obefore, oafter = rr.reorder_matrix((W.view(np.uint16) & 0x7FFF) != 0, 16, 64, 2, 2)
    assert np.array_equal(perm, operm) and np.array_equal(after, oafter)


@pytest.mark.parametrize("areas", [(2, 2), (4, 1)])
def test_permuted_encoding_stores_the_minimum(areas):
    """usw_union_encode of the permuted matrix: payload = Q x sum(after),
    and never more than before."""
    W, mask = masked(64, 256, 0.3, 11)
    lt = (16, 64)
    perm, before, after = usw.union_reorder(W, mask, lt, areas)
    Q = areas[0] * areas[1]
    h0 = usw.union_encode_host(W, mask, lt, areas, "i4")
    h1 = usw.union_encode_host(usw.apply_row_permutation(W, perm, *lt),
                               usw.apply_row_permutation(mask, perm, *lt), lt, areas, "i4")
    assert h0.payload == Q * int(before.sum())
    assert h1.payload == Q * int(after.sum()) <= h0.payload
    for t in range(perm.shape[0]):
        assert sorted(perm[t]) == list(range(lt[0]))


def test_reorder_gain_on_a_pruned_layer():
    """Magnitude-pruned synthetic layer at 50%: the reordering never
    increases any LT's actives and shrinks the total (figures printed)."""
    W, mask, _ = wl.config_case(5, 1024, 1024, 2, 0.5)
    for lt, areas in (((16, 64), (2, 2)), ((16, 64), (4, 1)), ((8, 64), (2, 2))):
        t = time.perf_counter()
        perm, before, after = usw.union_reorder(W, mask, lt, areas)
        dt = time.perf_counter() - t
        assert (after <= before).all()
        print(f"lt={lt} areas={areas}: actives {before.sum()} -> {after.sum()} "
              f"({1 - after.sum() / before.sum():.2%} fewer), {perm.shape[0]} LTs in {dt:.2f} s")
        assert after.sum() < before.sum()


def test_argument_errors():
    L = usw.lib()
    W = np.zeros((64, 64), np.uint16)
    perm = np.zeros(64 * 64, np.int32)
    w, p = W.ctypes.data, perm.ctypes.data
    assert L.usw_union_reorder(None, None, 64, 64, 16, 64, 2, 2, p, None, None) == -1
    assert L.usw_union_reorder(w, None, 64, 64, 16, 64, 2, 2, None, None, None) == -1
    assert L.usw_union_reorder(w, None, 64, 60, 16, 64, 2, 2, p, None, None) == -2
    assert L.usw_union_reorder(w, None, 64, 64, 16, 64, 3, 2, p, None, None) == -2
    assert L.usw_union_reorder(w, None, 64, 64, 32, 64, 2, 2, p, None, None) == -5
    assert L.usw_union_reorder(w, None, 64, 64, 16, 64, 2, 2, p, None, None) == 0
    assert (perm[:16] == [0, 2, 4, 6, 8, 10, 12, 14, 1, 3, 5, 7, 9, 11, 13, 15]).all()
