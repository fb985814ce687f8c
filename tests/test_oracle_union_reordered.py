"""Pins of the oracle's reordered IE-BME encoding ("UnionSparse", sections on
IE-BME and on bitmap-aware row reordering): reordering rearranges the rows
of each LT before compression and changes neither the number nor the
values of the surviving weights.  So decoding must give back W itself, the
product must equal the plain product of W, the INT4 scales are those of
the original rows, the payload shrinks to Q times the solver's minimum, and
the identity order reproduces the plain encoding byte for byte.  A decoder
that applies the row order instead of its inverse must fail."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import ie_bme as ou
from oracle import row_reorder as rr
from oracle import tca_bme as ob
import workloads as wl

F16, I4 = ob.VAL_F16, ob.VAL_I4


def random_perms(nlt, h, seed):
    rng = np.random.default_rng(seed)
    return np.array([rng.permutation(h) for _ in range(nlt)], dtype=np.int32)


def case(M, K, density, seed, exact_i4=False):
    rng = np.random.default_rng(seed)
    mask = rng.random((M, K)) < density
    W = wl.weight_int4_exact(M, K, rng, mask) if exact_i4 else wl.weight_normal(M, K, rng, sigma=1.0)
    return W, mask


@pytest.mark.parametrize("vt", [F16, I4])
@pytest.mark.parametrize("lt,areas", [((16, 64), (2, 2)), ((8, 64), (2, 2)), ((16, 64), (4, 1)), ((12, 32), (3, 2))])
def test_round_trip_with_any_row_order(vt, lt, areas):
    M, K = 4 * lt[0], 2 * lt[1]
    W, mask = case(M, K, 0.4, lt[0] + areas[0])
    g = ou.UnionGeometry(M, K, lt[0], lt[1], *areas)
    perms = random_perms(g.nlt, lt[0], 11)
    enc = ou.encode_union_reordered(W, mask, perms, lt[0], lt[1], *areas, vt)
    plain = ou.encode_union(W, mask, lt[0], lt[1], *areas, vt)
    assert np.array_equal(ou.decode_union(enc), ou.decode_union(plain))
    assert np.array_equal(ou.decode_union_loop(enc), ou.decode_union(plain))
    if vt == F16:
        assert np.array_equal(ou.decode_union(enc), np.where(mask, W, np.float16(0)).view(np.uint16))
    else:
        assert np.array_equal(enc.scales.view(np.uint16), plain.scales.view(np.uint16))
    # The row map is the inverse of the row order.
    for t in range(g.nlt):
        assert [int(enc.rowmap[t][perms[t][s]]) for s in range(lt[0])] == list(range(lt[0]))


def test_identity_order_is_the_plain_encoding():
    W, mask = case(64, 128, 0.5, 3)
    g = ou.UnionGeometry(64, 128, 16, 64, 2, 2)
    ident = np.tile(np.arange(16, dtype=np.int32), (g.nlt, 1))
    for vt in (F16, I4):
        a = ou.encode_union_reordered(W, mask, ident, 16, 64, 2, 2, vt)
        b = ou.encode_union(W, mask, 16, 64, 2, 2, vt)
        assert a.payload == b.payload
        for f in ("bitmaps", "offsets", "values"):
            assert np.array_equal(getattr(a, f), getattr(b, f)), f
        assert (a.scales is None) == (b.scales is None)
        assert a.rowmap.tolist() == ident.tolist()


def test_int4_scales_follow_the_original_rows():
    """Per-row quantisation precedes reordering: the scales are the original
    rows'; quantising the rearranged matrix instead would mix rows of
    different LT columns and give other scales."""
    W, mask = case(64, 256, 0.5, 5)
    g = ou.UnionGeometry(64, 256, 16, 64, 2, 2)
    perms = random_perms(g.nlt, 16, 6)
    enc = ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, I4)
    scales, q = ob.quantize_rows_i4(W, mask)
    assert np.array_equal(enc.scales.view(np.uint16), scales.view(np.uint16))
    assert np.array_equal(ou.decode_union(enc), q)
    mixed, _ = ob.quantize_rows_i4(ou.permute_lt_rows(W, perms, 16, 64), ou.permute_lt_rows(mask, perms, 16, 64))
    assert not np.array_equal(mixed.view(np.uint16), scales.view(np.uint16))


@pytest.mark.parametrize("areas", [(2, 2), (4, 1)])
def test_solver_order_stores_q_times_the_minimum(areas):
    M, K, h, k = 64, 128, 16, 64
    rng = np.random.default_rng(9)
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_magnitude(W, 0.6)
    perms, before, after = rr.reorder_matrix(mask, h, k, *areas)
    Q = areas[0] * areas[1]
    enc = ou.encode_union_reordered(W, mask, perms, h, k, *areas, I4)
    plain = ou.encode_union(W, mask, h, k, *areas, I4)
    assert enc.payload == Q * int(after.sum()) <= plain.payload == Q * int(before.sum())
    assert np.array_equal(np.diff(enc.offsets.astype(np.int64)), Q * after.astype(np.int64))


def test_product_equals_the_plain_product():
    """Y of the reordered encoding is Y of W itself: exact Fraction sums on a
    small case, and the fp64 product of the plain encoding."""
    M, K, N = 32, 128, 2
    W, mask = case(M, K, 0.5, 13, exact_i4=True)
    X = wl.activations_small_int(N, K, np.random.default_rng(14))
    g = ou.UnionGeometry(M, K, 16, 64, 2, 2)
    perms = random_perms(g.nlt, 16, 15)
    enc = ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, I4)
    Y = ou.spmm_union(enc, X)
    for n in range(N):
        for m in range(M):
            exact = sum(Fraction(float(W[m, k])) * Fraction(float(X[n, k])) for k in range(K) if mask[m, k])
            assert Fraction(Y[n, m]) == exact
    assert np.array_equal(Y, ou.spmm_union(ou.encode_union(W, mask, 16, 64, 2, 2, I4), X))


def test_rejects_orders_that_are_not_permutations():
    W, mask = case(32, 64, 0.5, 17)
    perms = np.tile(np.arange(16, dtype=np.int32), (2, 1))
    perms[1, 3] = 2
    with pytest.raises(ValueError):
        ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, I4)
    with pytest.raises(ValueError):
        ou.encode_union_reordered(W, mask, perms[:1], 16, 64, 2, 2, I4)


def test_planted_forward_map_fails():
    """A reader that takes row r from stored row perms[t][r] (the order
    itself, not its inverse) misplaces rows whenever the order is not an
    involution."""
    W, mask = case(32, 128, 0.5, 19)
    g = ou.UnionGeometry(32, 128, 16, 64, 2, 2)
    perms = np.array([np.roll(np.arange(16), 1 + t) for t in range(g.nlt)], dtype=np.int32)
    enc = ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, F16)
    planted = ou.UnionEncoded(enc.geom, enc.val_type, enc.payload, enc.bitmaps, enc.offsets, enc.values,
                              enc.scales, perms.astype(np.uint8))
    expect = np.where(mask, W, np.float16(0)).view(np.uint16)
    assert np.array_equal(ou.decode_union(enc), expect)
    assert not np.array_equal(ou.decode_union(planted), expect)
