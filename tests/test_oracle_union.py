"""Pins for the IE-BME union-mask oracle (UnionSparse, IE-BME and LSPD
sections): the Fig. 7 words and offsets, the kept area zero, the LSPD segment
example, independent constructions, closed forms, brute force on tiny inputs
and planted mistakes.

Runs on the CPU only.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import ie_bme as ou
from oracle import tca_bme as ob
import workloads as wl

F16, I4 = ob.VAL_F16, ob.VAL_I4


def rng(i):
    return np.random.default_rng((7, 11, i))


def rand_w(M, K, r):
    # Nonzero fp16 weights, so a position's value never vanishes by accident.
    w = r.normal(0.0, 1.0, size=(M, K))
    w = np.where(np.abs(w) < 1e-3, 1e-3, w)
    return w.astype(np.float16)


def fig7_mask(golden, r):
    """An 8x32 LT (R_A = C_A = 2, areas 4x16) whose union mask has the
    section's four logical rows; every active group keeps a random non-empty
    subset of its four area values."""
    g = golden("iebme_words_example.json")
    mask = np.zeros((8, 32), dtype=bool)
    for i, word in enumerate(g["words"]):
        for j in range(16):
            if (word >> j) & 1:
                sub = 0
                while sub == 0:
                    sub = int(r.integers(1, 16))
                for q in range(4):
                    if (sub >> q) & 1:
                        ar, ac = divmod(q, 2)
                        mask[ar * 4 + i, ac * 16 + j] = True
    return g, mask


# ---------------------------------------------------------------------------
# Fig. 7: union words, P_t and the next offset
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("enc_fn", [ou.encode_union, ou.encode_union_loop])
def test_fig7_words_and_offsets(golden, enc_fn):
    r = rng(0)
    g, m0 = fig7_mask(golden, r)
    # Two LTs side by side: the second starts at the first one's Q P_t.
    mask = np.concatenate([m0, m0], axis=1)
    W = rand_w(8, 64, r)
    enc = enc_fn(W, mask, h_l=8, k_l=32, r_a=2, c_a=2, val_type=F16)
    expect = sum(w << (16 * i) for i, w in enumerate(g["words"]))
    assert [int(x) for x in enc.bitmaps] == [expect, expect]
    assert [int(x) for x in enc.offsets] == [0, g["next_offset"], 2 * g["next_offset"]]
    assert enc.payload // g["Q"] // 2 == g["P_t"]


def test_fig7_group_keeps_area_zero():
    """The red-framed group [1, 30, 59, 0]: one union bit, one rank, four
    stream entries, the last a stored zero; an all-zero group stores nothing."""
    W = np.zeros((8, 32), dtype=np.float16)
    mask = np.zeros((8, 32), dtype=bool)
    # Logical position (1, 3): areas 0, 1, 2 hold 1, 30, 59; area 3 pruned.
    for q, v in enumerate([1.0, 30.0, 59.0]):
        ar, ac = divmod(q, 2)
        W[ar * 4 + 1, ac * 16 + 3] = v
        mask[ar * 4 + 1, ac * 16 + 3] = True
    # One earlier active group so the rank is not trivially 0.
    W[0, 0] = 5.0
    mask[0, 0] = True
    for enc_fn in (ou.encode_union, ou.encode_union_loop):
        enc = enc_fn(W, mask, h_l=8, k_l=32, r_a=2, c_a=2, val_type=F16)
        assert int(enc.bitmaps[0]) == (1 << 0) | (1 << (16 * 1 + 3))
        P_t = 2
        assert list(enc.offsets) == [0, 4 * P_t]
        streams = enc.values.view(np.float16).astype(np.float64).reshape(4, P_t)
        assert list(streams[:, 1]) == [1.0, 30.0, 59.0, 0.0]
        assert list(streams[:, 0]) == [5.0, 0.0, 0.0, 0.0]
    empty = ou.encode_union(np.zeros((8, 32), np.float16), np.zeros((8, 32), bool), 8, 32, 2, 2, F16)
    assert empty.payload == 0 and int(empty.bitmaps[0]) == 0


def test_kept_zero_is_active_and_stored():
    """The mask decides: a kept -0.0 makes its group active and keeps its bits."""
    W = np.zeros((8, 32), dtype=np.float16)
    W[5, 20] = np.float16(-0.0)
    mask = np.zeros((8, 32), dtype=bool)
    mask[5, 20] = True                   # area 3 (rows 4-7, cols 16-31), position (1, 4)
    enc = ou.encode_union(W, mask, 8, 32, 2, 2, F16)
    assert int(enc.bitmaps[0]) == 1 << (16 + 4)
    assert list(enc.values) == [0, 0, 0, 0x8000]


# ---------------------------------------------------------------------------
# LSPD segment (Fig. 9(c)): active bits 0, 2, 3, 5 read base .. base + 3
# ---------------------------------------------------------------------------

def test_lspd_segment_fig9(golden):
    gl = golden("lspd_segment_example.json")
    seg_bits = int(gl["segment_lsb_left"][::-1], 2)
    # LT 8x32, R_A = C_A = 2: logical rows of 16 bits; row 2 gets the 8-bit
    # segment in its second half (columns 8..15), after 3 + 5 earlier active bits.
    union = np.zeros((4, 16), dtype=bool)
    union[0, [1, 4, 9]] = True
    union[1, [0, 2, 3, 7, 15]] = True
    union[2, [2, 6]] = True              # two active bits earlier in the same row
    for p in range(8):
        union[2, 8 + p] = bool((seg_bits >> p) & 1)
    mask = np.zeros((8, 32), dtype=bool)
    mask[0:4, 0:16] = union              # area 0 only
    r = rng(1)
    W = rand_w(8, 32, r)
    enc = ou.encode_union(W, mask, 8, 32, 2, 2, F16)
    got = ou.lspd_segment(enc, 0, 2, 1, 8)
    assert [c - 8 for c, _ in got] == gl["active_positions"]
    base = 3 + 5 + 2
    P_t = int(union.sum())
    vals = enc.values
    for k, (c, area_vals) in enumerate(got):
        assert k == gl["payload_offsets_from_base"][k]
        assert area_vals == [vals[q * P_t + base + k] for q in range(4)]
        assert area_vals[0] == W[2, c].view(np.uint16)
        assert area_vals[1:] == [0, 0, 0]


# ---------------------------------------------------------------------------
# Independent constructions
# ---------------------------------------------------------------------------

SHAPES = [
    (64, 64, 64, 64, 2, 2),
    (128, 192, 64, 64, 2, 2),
    (64, 128, 32, 64, 2, 1),
    (32, 256, 16, 128, 1, 2),
    (128, 64, 64, 64, 4, 1),
    (64, 64, 32, 32, 1, 1),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("vt", [F16, I4])
def test_two_encoders_agree(shape, vt):
    M, K, h, k, ra, ca = shape
    r = rng(hash(shape) % 1000)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < 0.35
    a = ou.encode_union(W, mask, h, k, ra, ca, vt)
    b = ou.encode_union_loop(W, mask, h, k, ra, ca, vt)
    assert np.array_equal(a.bitmaps, b.bitmaps)
    assert np.array_equal(a.offsets, b.offsets)
    assert np.array_equal(a.values, b.values)
    assert a.payload == b.payload


@pytest.mark.parametrize("shape", SHAPES)
def test_round_trip_f16(shape):
    M, K, h, k, ra, ca = shape
    r = rng(50 + hash(shape) % 1000)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < 0.5
    enc = ou.encode_union(W, mask, h, k, ra, ca, F16)
    expect = np.where(mask, W, np.float16(0)).view(np.uint16)
    assert np.array_equal(ou.decode_union(enc), expect)
    assert np.array_equal(ou.decode_union_loop(enc), expect)


def test_round_trip_i4():
    M, K = 128, 128
    r = rng(3)
    mask = r.random((M, K)) < 0.5
    W = wl.weight_int4_exact(M, K, r, mask)
    enc = ou.encode_union(W, mask, 64, 64, 2, 2, I4)
    scales, q = ob.quantize_rows_i4(W, mask)
    assert np.array_equal(enc.scales.view(np.uint16), scales.view(np.uint16))
    assert np.array_equal(ou.decode_union(enc), q)
    assert np.array_equal(ou.decode_union_loop(enc), q)
    # The weights were built to quantise exactly: dequantisation gives W back.
    assert np.array_equal(ou.dense_weight_union(enc), np.where(mask, W, 0).astype(np.float64))


def test_i4_rounding_ties_half_even():
    """Exact .5 quotients in the union format's payload round to the even
    code.  Row 0 keeps 7.0 as its largest magnitude (scale 1), row 1 keeps
    14.0 (scale 2); the expected codes are written out by hand."""
    row0 = [7.0, 0.5, 1.5, 2.5, -0.5, -2.5, 6.5, 3.5, -3.5, 4.5, -4.5, 5.5, -1.5, -6.5, -5.5, 0.25]
    row1 = [14.0, 1.0, 3.0, 5.0, -1.0, -5.0, 13.0, 7.0, -7.0, 9.0, -9.0, 11.0, -3.0, -13.0, -11.0, -14.0]
    codes0 = [7, 0, 2, 2, 0, -2, 6, 4, -4, 4, -4, 6, -2, -6, -6, 0]
    codes1 = [7, 0, 2, 2, 0, -2, 6, 4, -4, 4, -4, 6, -2, -6, -6, -7]
    W = np.zeros((64, 64), dtype=np.float16)
    mask = np.zeros((64, 64), bool)
    W[0, :16], W[1, :16] = row0, row1
    mask[:2, :16] = True
    for enc in (ou.encode_union(W, mask, 64, 64, 2, 2, I4), ou.encode_union_loop(W, mask, 64, 64, 2, 2, I4)):
        assert enc.scales[0] == 1.0 and enc.scales[1] == 2.0
        q = ou.decode_union(enc)
        assert q[0, :16].tolist() == codes0 and q[1, :16].tolist() == codes1
        # Area 0's stream comes first: the 32 union-active positions of rows
        # 0 and 1 in row-major order, low nibble first.
        stream = ob.unpack_nibbles(enc.values, 32)
        assert stream.tolist() == codes0 + codes1


def test_single_area_is_plain_row_major_bitmap():
    """Q = 1: the union mask is the mask and each LT's payload is its kept
    values in row-major order (boolean indexing of each LT)."""
    M, K, h, k = 64, 128, 32, 64
    r = rng(4)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < 0.4
    enc = ou.encode_union(W, mask, h, k, 1, 1, F16)
    seq, bits, off = [], [], [0]
    for ti in range(M // h):
        for tj in range(K // k):
            blk = (slice(ti * h, ti * h + h), slice(tj * k, tj * k + k))
            seq.append(W[blk].view(np.uint16)[mask[blk]])
            bits.append(mask[blk].reshape(-1))
            off.append(off[-1] + int(mask[blk].sum()))
    assert np.array_equal(enc.values, np.concatenate(seq))
    assert list(enc.offsets) == off
    allbits = np.concatenate(bits)
    words = [sum(1 << b for b in range(64) if allbits[64 * w + b]) for w in range(allbits.size // 64)]
    assert [int(x) for x in enc.bitmaps] == words


def test_storage_closed_forms():
    """All kept: every group active, payload M K.  Only area 0 kept: payload
    Q times the kept count.  Bytes follow 4 (NLT + 1) + 8 NWORDS + payload/2."""
    M, K = 128, 128
    r = rng(5)
    W = rand_w(M, K, r)
    full = ou.encode_union(W, np.ones((M, K), bool), 64, 64, 2, 2, I4)
    assert full.payload == M * K
    assert full.bitmaps.size == (M * K) // 4 // 64
    mask = np.zeros((M, K), dtype=bool)
    sub = r.random((32, 32)) < 0.5
    mask[0:32, 0:32] = sub               # area 0 of LT 0 only
    enc = ou.encode_union(W, mask, 64, 64, 2, 2, I4)
    assert enc.payload == 4 * int(sub.sum())
    b = ou.union_storage_bytes(full.geom.nlt, full.geom.nwords, full.payload, 4)
    assert b == enc.offsets.nbytes + full.bitmaps.nbytes + full.values.nbytes
    assert b == 4 * 5 + 8 * 64 + M * K / 2


def test_union_activity_is_the_or_of_the_areas():
    """P_t counts groups with any kept value: for Bernoulli(keep) masks the
    mean activity approaches 1 - (1 - keep)^Q."""
    M, K = 512, 512
    r = rng(6)
    for keep in (0.3, 0.5):
        mask = r.random((M, K)) < keep
        enc = ou.encode_union(np.ones((M, K), np.float16), mask, 64, 64, 2, 2, F16)
        act = enc.payload / 4 / (M * K / 4)
        assert abs(act - (1 - (1 - keep) ** 4)) < 0.01


# ---------------------------------------------------------------------------
# The product
# ---------------------------------------------------------------------------

def test_product_brute_force_fraction():
    M, K, N = 16, 32, 3
    r = rng(7)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < 0.5
    X = r.normal(size=(N, K)).astype(np.float16)
    enc = ou.encode_union(W, mask, 8, 32, 2, 2, F16)
    Y = ou.spmm_union(enc, X)
    for n in range(N):
        for m in range(M):
            s = sum(Fraction(float(W[m, k])) * Fraction(float(X[n, k])) for k in range(K) if mask[m, k])
            assert abs(float(s) - Y[n, m]) <= 1e-12 * max(1.0, abs(float(s)))


def test_product_i4_integer_exact():
    M, K, N = 128, 128, 4
    r = rng(8)
    mask = r.random((M, K)) < 0.5
    W = wl.weight_int4_exact(M, K, r, mask)
    X = wl.activations_small_int(N, K, r)
    enc = ou.encode_union(W, mask, 64, 64, 2, 2, I4)
    Y = ou.spmm_union(enc, X)
    ref = X.astype(np.float64) @ np.where(mask, W, 0).astype(np.float64).T
    assert np.array_equal(Y, ref)


def test_matches_tca_bme_product():
    """The two formats describe the same W_sp: their oracle products agree bit for bit."""
    M, K, N = 128, 128, 5
    r = rng(9)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < 0.45
    X = r.normal(size=(N, K)).astype(np.float16)
    a = ou.spmm_union(ou.encode_union(W, mask, 64, 64, 2, 2, I4), X)
    b = ob.spmm(ob.encode_i4(W, mask), X)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# Planted mistakes (in copies of the oracle's steps) must fail a pin
# ---------------------------------------------------------------------------

def _encode_variant(W, mask, h, k, ra, ca, area_of, drop_zeros=False):
    g = ou.UnionGeometry(W.shape[0], W.shape[1], h, k, ra, ca)
    src = np.where(mask, W.view(np.uint16), 0).astype(np.uint16)
    bits, seq, off = [], [], [0]
    for ti in range(g.lt_rows):
        for tj in range(g.lt_cols):
            r0, c0 = ti * h, tj * k
            act = []
            for i in range(g.am):
                for j in range(g.ak):
                    on = any(mask[r0 + area_of(q, g)[0] * g.am + i, c0 + area_of(q, g)[1] * g.ak + j]
                             for q in range(g.Q))
                    bits.append(on)
                    if on:
                        act.append((i, j))
            n = 0
            for q in range(g.Q):
                ar, ac = area_of(q, g)
                for (i, j) in act:
                    v = int(src[r0 + ar * g.am + i, c0 + ac * g.ak + j])
                    if drop_zeros and v == 0:
                        continue
                    seq.append(v)
                    n += 1
            off.append(off[-1] + n)
    return np.array(seq, dtype=np.uint16), off


def test_planted_mistakes_fail():
    r = rng(10)
    W = rand_w(64, 128, r)
    mask = r.random((64, 128)) < 0.5
    good = ou.encode_union(W, mask, 64, 64, 2, 2, F16)
    seq, off = _encode_variant(W, mask, 64, 64, 2, 2, lambda q, g: divmod(q, g.c_a))
    assert np.array_equal(seq, good.values) and off == list(good.offsets)
    # Areas taken column-major over the grid.
    seq, off = _encode_variant(W, mask, 64, 64, 2, 2, lambda q, g: (q % g.r_a, q // g.r_a))
    assert not np.array_equal(seq, good.values)
    # Area zeros dropped from the streams (per-area ranks): offsets change.
    seq, off = _encode_variant(W, mask, 64, 64, 2, 2, lambda q, g: divmod(q, g.c_a), drop_zeros=True)
    assert off != list(good.offsets)
    # A rank that counts the position itself: the round trip breaks.
    assert not np.array_equal(_decode_variant(good, lambda w, p: ou.union_rank(w, p) + 1, 0),
                              ou.decode_union(good))
    # Ranks restarted per 64-bit word: the round trip breaks.
    assert not np.array_equal(_decode_variant(good, lambda w, p: ob.masked_popcount(int(w[p // 64]), p % 64), 0),
                              ou.decode_union(good))
    # Area streams read at o_t + q (P_t - 1) + rank: the round trip breaks.
    assert not np.array_equal(_decode_variant(good, ou.union_rank, -1), ou.decode_union(good))
    assert np.array_equal(_decode_variant(good, ou.union_rank, 0), ou.decode_union(good))


def test_planted_bit_order_fails_fig7(golden):
    """Union rows packed most-significant bit first do not give the Fig. 7 words."""
    g = golden("iebme_words_example.json")
    r = rng(12)
    _, mask = fig7_mask(golden, r)
    union = mask[0:4, 0:16] | mask[0:4, 16:32] | mask[4:8, 0:16] | mask[4:8, 16:32]
    msb_first = [int("".join("1" if b else "0" for b in row), 2) for row in union]
    lsb_first = [int("".join("1" if b else "0" for b in row[::-1]), 2) for row in union]
    assert lsb_first == g["words"]
    assert msb_first != g["words"]


def _decode_variant(enc, rank_fn, stride_delta):
    """decode_union_loop's steps with the rank rule and stream stride swappable."""
    g = enc.geom
    vals = enc.values
    out = np.zeros((g.M, g.K), dtype=np.uint16)
    t = 0
    for ti in range(g.lt_rows):
        for tj in range(g.lt_cols):
            words = enc.bitmaps[t * g.words_per_lt:(t + 1) * g.words_per_lt]
            o_t = int(enc.offsets[t])
            P_t = (int(enc.offsets[t + 1]) - o_t) // g.Q
            for i in range(g.am):
                for j in range(g.ak):
                    p = i * g.ak + j
                    if not (int(words[p // 64]) >> (p % 64)) & 1:
                        continue
                    rank = rank_fn(words, p)
                    for q in range(g.Q):
                        ar, ac = divmod(q, g.c_a)
                        idx = min(o_t + q * (P_t + stride_delta) + rank, vals.size - 1)
                        out[ti * g.h_l + ar * g.am + i, tj * g.k_l + ac * g.ak + j] = vals[idx]
            t += 1
    return out
