"""Pins of the oracle's 2-bit (W2) weight payload: the per-row rule with
b = 2 (scale fp16(max |w| / 1), codes clamp(round_half_even(w / scale),
-2, 1)), four codes per byte with the lowest bits first, exact
dequantisation, and the IE-BME union format carrying it (UnionSparse,
W2A4 kernel-level analysis, read as weight-only).  Expected codes and bytes
are written out by hand; planted mistakes (ties away from zero, the
asymmetric scale max/2, high crumb first) must fail."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import ie_bme as ou
from oracle import tca_bme as ob
import workloads as wl

I2 = ob.VAL_I2

# Row 0 keeps 3.0 as its largest magnitude, so scale = 3.0 and each code is
# round_half_even(w / 3): 1.5 / 3 = 0.5 and -1.5 / 3 = -0.5 are ties and go
# to 0; 2.0 / 3 = 0.667 -> 1; 0.75 / 3 = 0.25 -> 0; 1.6 / 3 = 0.533 -> 1.
# Row 1 keeps -0.5 (scale 0.5): w / 0.5 = 2 w, so 0.25 -> 0.5 -> 0 (tie),
# 0.375 -> 0.75 -> 1, -0.25 -> -0.5 -> 0 (tie), -0.375 -> -1.
W2_ROWS = [
    ([3.0, 1.5, -1.5, 2.0, -2.0, 0.75, -3.0, 1.6, -0.75, 0.0, -1.6, 2.5],
     [1, 0, 0, 1, -1, 0, -1, 1, 0, 0, -1, 1]),
    ([-0.5, 0.25, 0.375, -0.25, -0.375, 0.5, 0.125, -0.125, 0.0, 0.3125, -0.4375, 0.5],
     [-1, 0, 1, 0, -1, 1, 0, 0, 0, 1, -1, 1]),
]


def w2_case():
    W = np.zeros((16, 16), dtype=np.float16)
    mask = np.zeros((16, 16), bool)
    for r, (w, _) in enumerate(W2_ROWS):
        W[r, :len(w)] = w
        mask[r, :len(w)] = True
    return W, mask


def w2_codes_hold(quantize):
    W, mask = w2_case()
    scales, q = quantize(W, mask)
    if float(scales[0]) != 3.0 or float(scales[1]) != 0.5:
        return False
    return all(q[r, :len(c)].tolist() == c for r, (_, c) in enumerate(W2_ROWS))


def mutant_half_away(W, mask):
    Wd = W.astype(np.float64)
    amax = np.where(mask, np.abs(Wd), 0.0).max(axis=1)
    scales = ob.fp16_rne(amax)
    t = Wd / np.where(scales > 0, scales.astype(np.float64), 1.0)[:, None]
    q = np.sign(t) * np.floor(np.abs(t) + 0.5)
    return scales, np.where(mask, np.clip(q, -2, 1), 0).astype(np.int8)


def mutant_asymmetric(W, mask):
    """Scale max / 2 so that -2 is reachable (a different reading)."""
    Wd = W.astype(np.float64)
    amax = np.where(mask, np.abs(Wd), 0.0).max(axis=1)
    scales = ob.fp16_rne(amax / 2.0)
    t = Wd / np.where(scales > 0, scales.astype(np.float64), 1.0)[:, None]
    return scales, np.where(mask, np.clip(np.rint(t), -2, 1), 0).astype(np.int8)


def test_w2_codes_and_scales_by_hand():
    assert w2_codes_hold(ob.quantize_rows_i2)
    assert not w2_codes_hold(mutant_half_away)
    assert not w2_codes_hold(mutant_asymmetric)


def test_w2_rule_is_the_int4_rule_with_b_2():
    """b = 4 of the general rule is the pinned INT4 rule; b = 2 never needs
    the code -2 for finite weights (|w| <= max |w| = scale)."""
    rng = np.random.default_rng(3)
    W = wl.weight_normal(64, 128, rng)
    mask = wl.mask_bernoulli(64, 128, 0.5, rng)
    s4, q4 = ob.quantize_rows_int(W, mask, 4)
    t4, r4 = ob.quantize_rows_i4(W, mask)
    assert np.array_equal(s4.view(np.uint16), t4.view(np.uint16)) and np.array_equal(q4, r4)
    s2, q2 = ob.quantize_rows_i2(W, mask)
    assert q2.min() >= -1 and q2.max() <= 1
    amax = np.where(mask, np.abs(W.astype(np.float64)), 0).max(axis=1)
    assert np.array_equal(s2.astype(np.float64), amax)      # fp16 amax / 1 is exact


def test_w2_packing_by_hand():
    q = np.array([1, -1, 0, -2, 1], dtype=np.int8)
    # crumbs 01, 11, 00, 10 -> 0b10_00_11_01 = 0x8D; then 01 and zero padding
    assert ob.pack_crumbs(q).tolist() == [0x8D, 0x01]
    assert np.array_equal(ob.unpack_crumbs(ob.pack_crumbs(q), 5), q)
    high_first = lambda x: np.array([(int(x[0] & 3) << 6) | (int(x[1] & 3) << 4) | (int(x[2] & 3) << 2)  # noqa: E731
                                     | int(x[3] & 3)], dtype=np.uint8)
    assert high_first(q).tolist() != [0x8D]
    rng = np.random.default_rng(4)
    for n in (0, 1, 3, 4, 5, 64, 1001):
        r = rng.integers(-2, 2, size=n).astype(np.int8)
        p = ob.pack_crumbs(r)
        assert p.size == (n + 3) // 4
        assert np.array_equal(ob.unpack_crumbs(p, n), r)


def test_w2_exact_weights_quantise_exactly():
    rng = np.random.default_rng(5)
    mask = wl.mask_bernoulli(64, 128, 0.5, rng)
    W = wl.weight_int2_exact(64, 128, rng, mask)
    scales, q = ob.quantize_rows_i2(W, mask)
    deq = q.astype(np.float64) * scales.astype(np.float64)[:, None]
    assert np.array_equal(deq, np.where(mask, W.astype(np.float64), 0.0))


def test_w2_non_finite_reading_as_int4():
    W = np.zeros((16, 16), dtype=np.float16)
    W[0, :3] = [0.5, np.nan, -0.25]
    W[1, :3] = [0.5, np.inf, -np.inf]
    mask = np.zeros((16, 16), bool)
    mask[:2, :3] = True
    scales, q = ob.quantize_rows_i2(W, mask)
    assert np.isnan(scales[0]) and not q[0].any()
    assert scales[1] == np.inf and not q[1].any()


@pytest.mark.parametrize("lt,areas", [((64, 64), (2, 2)), ((16, 64), (2, 2)), ((32, 64), (2, 1))])
def test_union_w2_round_trip_and_two_encoders(lt, areas):
    rng = np.random.default_rng(lt[0] + areas[1])
    M, K = 128, 256
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    a = ou.encode_union(W, mask, lt[0], lt[1], *areas, I2)
    b = ou.encode_union_loop(W, mask, lt[0], lt[1], *areas, I2)
    for f in ("bitmaps", "offsets", "values", "scales"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert a.values.size == (a.payload + 3) // 4
    scales, q = ob.quantize_rows_i2(W, mask)
    assert np.array_equal(ou.decode_union(a), q)
    assert np.array_equal(ou.decode_union_loop(a), q)
    # The I2 payload is the INT4 payload's codes requantised; the union words
    # and offsets do not depend on the value type.
    a4 = ou.encode_union(W, mask, lt[0], lt[1], *areas, ob.VAL_I4)
    assert np.array_equal(a.bitmaps, a4.bitmaps) and np.array_equal(a.offsets, a4.offsets)
    assert ou.union_storage_bytes(a.geom.nlt, a.bitmaps.size, a.payload, 2) == \
        4 * (a.geom.nlt + 1) + 8 * a.bitmaps.size + a.payload / 4


def test_union_w2_stream_bytes_by_hand():
    """Row 0 of a 64 x 64 LT keeps 3.0, 1.5, -3.0, 2.0 at columns 0-3: scale 3,
    codes 1, 0 (tie), -1, 1, stored as area 0's first four payload elements:
    crumbs 01 00 11 01 -> byte 0b01_11_00_01 = 0x71."""
    W = np.zeros((64, 64), dtype=np.float16)
    mask = np.zeros((64, 64), bool)
    W[0, :4] = [3.0, 1.5, -3.0, 2.0]
    mask[0, :4] = True
    enc = ou.encode_union(W, mask, 64, 64, 2, 2, I2)
    assert enc.payload == 4 * 4 and float(enc.scales[0]) == 3.0
    assert enc.values[0] == 0x71
    assert ob.unpack_crumbs(enc.values, 4).tolist() == [1, 0, -1, 1]


def test_union_w2_product_brute_force():
    rng = np.random.default_rng(9)
    M, K, N = 64, 128, 2
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    W = wl.weight_int2_exact(M, K, rng, mask)
    X = wl.activations_small_int(N, K, rng)
    enc = ou.encode_union(W, mask, 64, 64, 2, 2, I2)
    Y = ou.spmm_union(enc, X)
    for n in range(N):
        for m in range(M):
            exact = sum(Fraction(float(W[m, k])) * Fraction(float(X[n, k])) for k in range(K) if mask[m, k])
            assert Fraction(Y[n, m]) == exact


def test_union_w2_reordered_round_trip():
    rng = np.random.default_rng(11)
    M, K = 64, 128
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    perms = np.array([rng.permutation(16) for _ in range(8)], dtype=np.int32)
    enc = ou.encode_union_reordered(W, mask, perms, 16, 64, 2, 2, I2)
    assert np.array_equal(ou.decode_union(enc), ob.quantize_rows_i2(W, mask)[1])
