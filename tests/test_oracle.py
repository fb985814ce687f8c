"""Pins for the CPU oracle: values the pages print, closed forms, invariants,
brute force on tiny inputs, and planted mistakes that the pins must catch.

Runs on the CPU only.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import tca_bme as ob
import workloads as wl


def f16(x):
    return np.float16(x)


# ---------------------------------------------------------------------------
# The blog's 8-bit worked example (SpInfer blog, "The Values array and why
# it's confusing at first"): bitmap 10010110 (bits 7..0) keeps positions
# 1, 2, 4, 7; position 4 reads Values[2].
# ---------------------------------------------------------------------------

def blog_example_checks(golden, encode_fn, rank_fn):
    g = golden("blog_bitmap_example.json")
    bm = int(g["bitmap_bits_msb_to_lsb"], 2)
    if bm != g["bitmap_value"]:
        return False
    positions = [p for p in range(8) if (bm >> p) & 1]
    if positions != g["nonzero_positions"]:
        return False
    if rank_fn(bm, g["query_position"]) != g["query_index"]:
        return False
    if [rank_fn(bm, p) for p in positions] != list(range(len(positions))):
        return False
    # The same row as the first row of an 8x8 BitmapTile inside a 16x16 matrix.
    W = np.zeros((16, 16), dtype=np.float16)
    for p, v in zip(positions, g["values"]):
        W[0, p] = v
    enc = encode_fn(W, None, 16, 16)
    if int(enc.bitmaps[0]) != bm:
        return False
    if not np.array_equal(enc.values, np.array(g["values"], dtype=np.float16)):
        return False
    if enc.values[rank_fn(int(enc.bitmaps[0]), g["query_position"])] != f16(0.05):
        return False
    return True


def test_blog_example(golden):
    assert blog_example_checks(golden, ob.encode, ob.masked_popcount)
    assert blog_example_checks(golden, ob.encode_loop, ob.masked_popcount)


def test_blog_example_decodes(golden):
    g = golden("blog_bitmap_example.json")
    W = np.zeros((16, 16), dtype=np.float16)
    for p, v in zip(g["nonzero_positions"], g["values"]):
        W[0, p] = v
    enc = ob.encode(W, None, 16, 16)
    for dec in (ob.decode, ob.decode_loop):
        D = dec(enc)
        assert D[0, g["query_position"]] == f16(g["values"][g["query_index"]])
        assert np.array_equal(D.view(np.uint16), W.view(np.uint16))


def test_smbd_lane_recipe_matches_decoder():
    """Blog SMBD recipe: lane l owns positions 2l and 2l+1; it counts the set
    bits below 2l, reads Values[count] for a set bit and writes 0 otherwise.
    Reconstructing every 8x8 tile that way must equal the oracle decoder."""
    rng = np.random.default_rng(5)
    W = wl.weight_normal(32, 32, rng)
    mask = wl.mask_bernoulli(32, 32, 0.45, rng)
    enc = ob.encode(W, mask, 16, 16)
    dense = ob.decode(enc)
    base = 0
    for t in range(enc.bitmaps.size):
        bm = int(enc.bitmaps[t])
        vals = enc.values[base: base + ob.popcount(bm)]
        tile = np.zeros(64, dtype=np.float16)
        for lane in range(32):
            offset = lane * 2
            count = ob.popcount(bm & ((1 << offset) - 1))
            for j in range(2):
                if (bm >> (offset + j)) & 1:
                    tile[offset + j] = vals[count]
                    count += 1
        # tile t in storage order -> location in the matrix (16x16 GroupTiles)
        gid, b = divmod(t, 4)
        gi, gj = divmod(gid, 2)
        bi, bj = divmod(b, 2)
        r0, c0 = 16 * gi + 8 * bi, 16 * gj + 8 * bj
        assert np.array_equal(tile.reshape(8, 8).view(np.uint16), dense[r0:r0 + 8, c0:c0 + 8].view(np.uint16))
        base += ob.popcount(bm)


# ---------------------------------------------------------------------------
# UnionSparse pins: LSPD segment example and IE-BME words
# ---------------------------------------------------------------------------

def test_lspd_segment_example(golden):
    g = golden("lspd_segment_example.json")
    seg = int(g["segment_lsb_left"][::-1], 2)       # leftmost displayed bit = LSB
    assert seg == 0x2D
    active = [p for p in range(8) if (seg >> p) & 1]
    assert active == g["active_positions"]
    assert [ob.masked_popcount(seg, p) for p in active] == g["payload_offsets_from_base"]


def test_iebme_words_popcount(golden):
    g = golden("iebme_words_example.json")
    assert [int(h, 16) for h in g["words_hex"]] == g["words"]
    counts = [ob.popcount(w) for w in g["words"]]
    assert counts == [g["active_per_row"]] * 4
    assert sum(counts) == g["P_t"]
    assert g["Q"] * sum(counts) == g["next_offset"]


# ---------------------------------------------------------------------------
# Storage equation and compression ratio
# ---------------------------------------------------------------------------

def encoded_bytes(enc):
    return enc.bitmaps.nbytes + enc.offsets.nbytes + enc.values.nbytes


def test_storage_equation_exact(golden):
    g = golden("storage_example.json")
    for case in g["cases"]:
        geo = ob.Geometry(case["M"], case["K"], case["gt_m"], case["gt_k"])
        assert geo.ngt == case["ngt"] and geo.nbt == case["nbt"]
        assert ob.storage_bytes(geo.ngt, geo.nbt, 0) == case["fixed_bytes"]
    W, mask, _ = wl.config_case(1, 256, 256, 8, 0.5)
    enc = ob.encode(W, mask)
    assert encoded_bytes(enc) == ob.storage_bytes(enc.geom.ngt, enc.geom.nbt, enc.nnz)
    assert encoded_bytes(enc) == 8260 + 2 * int(mask.sum())


def test_cr_above_one_at_30_percent(golden):
    g = golden("storage_example.json")
    rng = np.random.default_rng(11)
    W = wl.weight_normal(1024, 1024, rng)
    mask = wl.mask_bernoulli(1024, 1024, 0.7, rng)
    enc = ob.encode(W, mask)
    cr = ob.compression_ratio(1024, 1024, encoded_bytes(enc))
    assert cr > 1.0
    assert abs(cr - g["cr_closed_form_large_matrix"]["0.3"]) < 0.01
    # closed form with exactly (1 - s) M K nonzeros on the FFN-up geometry; the
    # fixture's values neglect the offsets (4 B per 4096 elements at 64x64)
    geo = ob.Geometry(20480, 5120, 64, 64)
    for s, ref in g["cr_closed_form_large_matrix"].items():
        nnz = round((1 - float(s)) * geo.M * geo.K)
        cr = ob.compression_ratio(geo.M, geo.K, ob.storage_bytes(geo.ngt, geo.nbt, nnz))
        assert cr < ref and abs(cr - ref) < 2e-3
    # break-even: CR = 1 at s = 1/16 when offsets are neglected (2 = 1/8 + 2(1 - s))
    s0 = g["cr_break_even_sparsity"]
    assert abs(2.0 / (8 / 64 + 2 * (1 - s0)) - 1.0) < 1e-12


def test_compute_intensity_limits():
    """SpInfer blog, 'Limitations and what's next': CI_SpMM -> CI_GEMM as N
    grows, so the CR advantage vanishes in prefill."""
    M = 20480
    cr = 1.7777777
    small = ob.compute_intensity(M, 16, cr) / ob.compute_intensity(M, 16, 1.0)
    big = ob.compute_intensity(M, 10 ** 9, cr) / ob.compute_intensity(M, 10 ** 9, 1.0)
    assert small > 1.7
    assert abs(big - 1.0) < 1e-4
    assert ob.compute_intensity(M, 1, 1.0) == pytest.approx(M / (M + 1))


def test_pmr_low_bit_shrinks():
    """UnionSparse motivation: quantisation shrinks payload but not metadata,
    so PMR falls from FP16 to INT4 (by 4x on the same mask)."""
    geo = ob.Geometry(20480, 5120, 64, 64)
    nnz = geo.M * geo.K // 2
    p16 = ob.payload_metadata_ratio(nnz, geo.ngt, geo.nbt, 2.0)
    p4 = ob.payload_metadata_ratio(nnz, geo.ngt, geo.nbt, 0.5)
    assert p16 == pytest.approx(7.94, abs=0.01)
    assert p4 == pytest.approx(p16 / 4)


# ---------------------------------------------------------------------------
# Bit order and tile order
# ---------------------------------------------------------------------------

def expected_slot(R, C, K, gt_m=64, gt_k=64):
    Gc = K // gt_k
    gid = (R // gt_m) * Gc + C // gt_k
    t = ((R % gt_m) // 16) * (gt_k // 16) + (C % gt_k) // 16
    b = ((R % 16) // 8) * 2 + (C % 16) // 8
    return int(gid * (gt_m * gt_k // 64) + 4 * t + b), int((R % 8) * 8 + (C % 8))


def test_single_nonzero_bit_positions():
    M, K = 128, 192
    rng = np.random.default_rng(3)
    cells = [(r, c) for r in range(8) for c in range(8)]
    cells += [tuple(x) for x in np.stack([rng.integers(0, M, 300), rng.integers(0, K, 300)], 1)]
    for (R, C) in cells:
        W = np.zeros((M, K), dtype=np.float16)
        W[R, C] = 1.5
        enc = ob.encode(W, None)
        idx, bit = expected_slot(R, C, K)
        nz = np.nonzero(enc.bitmaps)[0]
        assert list(nz) == [idx]
        assert int(enc.bitmaps[idx]) == 1 << bit
        assert enc.nnz == 1 and enc.values[0] == f16(1.5)
        gid = idx // 64
        assert list(enc.offsets[: gid + 1]) == [0] * (gid + 1)
        assert np.all(enc.offsets[gid + 1:] == 1)


@pytest.mark.parametrize("shape,gt", [((64, 64), (64, 64)), ((128, 192), (64, 64)), ((96, 64), (32, 64)),
                                      ((48, 80), (16, 16)), ((64, 128), (64, 32))])
@pytest.mark.parametrize("density", [0.0, 0.3, 0.5, 1.0])
def test_two_encoders_agree(shape, gt, density):
    M, K = shape
    rng = np.random.default_rng(int(density * 100) + M + K)
    W = wl.weight_normal(M, K, rng)
    W[rng.random((M, K)) < 0.05] = np.float16(0.0)
    W[rng.random((M, K)) < 0.05] = np.float16(-0.0)
    mask = wl.mask_bernoulli(M, K, density, rng)
    a = ob.encode(W, mask, *gt)
    b = ob.encode_loop(W, mask, *gt)
    assert a.nnz == b.nnz == int(mask.sum())
    assert np.array_equal(a.bitmaps, b.bitmaps)
    assert np.array_equal(a.offsets, b.offsets)
    assert np.array_equal(a.values.view(np.uint16), b.values.view(np.uint16))
    # round trip, bitwise: kept entries (including +-0) keep their bits
    for dec in (ob.decode, ob.decode_loop):
        D = dec(a)
        expect = np.where(mask, W.view(np.uint16), np.uint16(0))
        assert np.array_equal(D.view(np.uint16), expect)


def test_offsets_invariants():
    W, mask, _ = wl.config_case(1, 256, 256, 8, 0.5)
    enc = ob.encode(W, mask)
    off = enc.offsets.astype(np.int64)
    assert off[0] == 0 and off[-1] == enc.nnz == mask.sum()
    assert np.all(np.diff(off) >= 0)
    per_gt = [sum(ob.popcount(int(x)) for x in enc.bitmaps[64 * g: 64 * (g + 1)]) for g in range(enc.geom.ngt)]
    assert list(np.diff(off)) == per_gt
    ob.check_offsets(enc)


def test_corrupt_offsets_detected():
    W, mask, _ = wl.config_case(1, 256, 256, 8, 0.5)
    enc = ob.encode(W, mask)
    bad = ob.Encoded(**{**enc.__dict__, "offsets": enc.offsets.copy()})
    bad.offsets[3] += 1
    with pytest.raises(ValueError):
        ob.decode(bad)
    with pytest.raises(ValueError):
        ob.decode_loop(bad)


def test_null_mask_keeps_ieee_nonzeros():
    W = np.array([[0.0, -0.0, 1.0, np.nan] + [0.0] * 12] + [[0.0] * 16] * 15, dtype=np.float16)
    enc = ob.encode(W, None, 16, 16)
    assert int(enc.bitmaps[0]) == 0b1100
    assert enc.nnz == 2


def test_geometry_rejects_bad_shapes():
    for args in [(100, 64, 64, 64), (64, 64, 24, 64), (64, 64, 64, 0), (0, 64, 64, 64)]:
        with pytest.raises(ValueError):
            ob.Geometry(*args)


# ---------------------------------------------------------------------------
# The product
# ---------------------------------------------------------------------------

def test_spmm_brute_force_fractions():
    rng = np.random.default_rng(7)
    M, K, N = 32, 48, 3
    W = wl.weight_normal(M, K, rng, sigma=1.0)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    enc = ob.encode(W, mask, 16, 16)
    Y = ob.spmm(enc, X)
    assert Y.shape == (N, M)
    for n in range(N):
        for m in range(M):
            exact = sum(Fraction(float(W[m, k])) * Fraction(float(X[n, k])) for k in range(K) if mask[m, k])
            bnd = sum(abs(float(W[m, k]) * float(X[n, k])) for k in range(K))
            assert abs(Fraction(Y[n, m]) - exact) <= Fraction(K * 2.0 ** -52) * Fraction(bnd)


def test_spmm_integer_exact_bitwise():
    W, mask, X = wl.config_case(1, 256, 256, 8, 0.5, exact=True)
    enc = ob.encode(W, mask)
    Y = ob.spmm(enc, X)
    Wi = np.where(mask, W.astype(np.float64) * 8, 0).astype(np.int64)
    Yi = X.astype(np.int64) @ Wi.T
    assert np.array_equal(Y * 8, Yi.astype(np.float64))


def test_spmm_special_cases():
    rng = np.random.default_rng(9)
    W = wl.weight_normal(64, 128, rng)
    X = wl.activations_normal(5, 128, rng)
    # s = 0: the dense product
    enc = ob.encode(W, np.ones(W.shape, bool))
    assert np.array_equal(ob.spmm(enc, X), X.astype(np.float64) @ W.astype(np.float64).T)
    # everything pruned: no values, Y = 0
    enc0 = ob.encode(W, np.zeros(W.shape, bool))
    assert enc0.nnz == 0 and enc0.values.size == 0 and not enc0.bitmaps.any()
    assert not ob.spmm(enc0, X).any()
    # N = 1 is a GEMV
    mask = wl.mask_bernoulli(64, 128, 0.5, rng)
    enc1 = ob.encode(W, mask)
    y = ob.spmm(enc1, X[:1])
    gemv = np.array([sum(float(W[m, k]) * float(X[0, k]) for k in range(128) if mask[m, k]) for m in range(64)])
    assert np.allclose(y[0], gemv, rtol=0, atol=1e-12)


def test_compare_accepts_fp32_sequential_and_rejects_dropped_term():
    """The acceptance bound is met by plain sequential fp32 accumulation with
    fp16 output at K = 20480, and fails when one product is dropped."""
    rng = np.random.default_rng(21)
    K, M, N = 20480, 24, 2
    W = wl.weight_normal(M, K, rng)
    mask = wl.mask_bernoulli(M, K, 0.5, rng)
    X = wl.activations_normal(N, K, rng)
    Wm = np.where(mask, W, np.float16(0)).astype(np.float32)
    prod = X.astype(np.float32)[:, None, :] * Wm[None, :, :]
    Yf32 = np.cumsum(prod, axis=2, dtype=np.float32)[:, :, -1]
    Y16 = Yf32.astype(np.float16)
    Wd = np.where(mask, W, np.float16(0))
    Yref = ob.spmm_fp64(Wd, X)
    Bnd = ob.abs_bound(Wd, X)
    ok, rel, worst = ob.compare(Y16, Yref, Bnd)
    assert ok and rel < 1e-3 and worst < 1.0
    # drop the largest product of one output: must fail
    m = 3
    kk = int(np.argmax(np.abs(prod[0, m])))
    Ybad = Yf32.copy()
    Ybad[0, m] -= prod[0, m, kk]
    assert not ob.compare(Ybad, Yref, Bnd)[0]
    # closed form: fp32 sequential worst case plus fp16 output rounding
    assert K * 2.0 ** -24 + 2.0 ** -11 < ob.ABS_BOUND_FACTOR


def test_compare_zero_reference_requires_zero():
    z = np.zeros((2, 3))
    assert ob.compare(z, z, z)[0]
    assert not ob.compare(z + 1e-30, z, z)[0]


# ---------------------------------------------------------------------------
# INT4 values
# ---------------------------------------------------------------------------

def test_fp16_rne_known_values():
    # 0.1 lies between 0x2E66 (0.0999755859375) and 0x2E67 (0.10009765625),
    # nearer the first; 1 + 2^-11 is a tie between 1 and 1 + 2^-10 -> even (1).
    assert ob.fp16_rne(0.1).view(np.uint16) == 0x2E66
    assert ob.fp16_rne(1 + 2 ** -11).view(np.uint16) == 0x3C00
    assert ob.fp16_rne(1 + 3 * 2 ** -11).view(np.uint16) == 0x3C02


def test_int4_quantisation_rule():
    W = np.zeros((16, 16), dtype=np.float16)
    W[0, :5] = [0.7, -0.35, 0.05, -0.7, 0.0]
    W[1, :2] = [0.0, 0.0]
    mask = np.zeros((16, 16), bool)
    mask[0, :5] = True
    mask[1, :2] = True           # kept zeros: amax = 0 -> scale 0, q 0
    scales, q = ob.quantize_rows_i4(W, mask)
    amax = float(np.float16(0.7))
    assert scales[0] == ob.fp16_rne(amax / 7)
    s = float(scales[0])
    for k in range(5):
        expect = int(np.clip(np.rint(float(W[0, k]) / s), -8, 7))
        assert q[0, k] == expect
    assert q[0, 0] == 7 and q[0, 3] == -7 and q[0, 4] == 0
    assert scales[1] == 0 and not q[1].any()
    assert scales[2:].tolist() == [0.0] * 14
    assert q.min() >= -8 and q.max() <= 7


# Exact .5 quotients, written out by hand.  Row 0 keeps 7.0 as its largest
# magnitude, so scale = fp16(7 / 7) = 1 and each code is the weight rounded to
# an integer; row 1 keeps 14.0, scale 2, so each code is half the weight.
# Round half to even sends every tie to the even neighbour: 0.5 -> 0,
# 1.5 -> 2, 2.5 -> 2, 3.5 -> 4, 4.5 -> 4, 5.5 -> 6, 6.5 -> 6, and the same
# with signs; half away from zero (C's round) would give 1, 2, 3, 4, 5, 6, 7.
INT4_TIE_ROWS = [
    # (weights of the kept entries, expected codes)
    ([7.0, 0.5, 1.5, 2.5, -0.5, -2.5, 6.5, 3.5, -3.5, 4.5, -4.5, 5.5, -1.5, -6.5, -5.5, 0.25],
     [7, 0, 2, 2, 0, -2, 6, 4, -4, 4, -4, 6, -2, -6, -6, 0]),
    ([14.0, 1.0, 3.0, 5.0, -1.0, -5.0, 13.0, 7.0, -7.0, 9.0, -9.0, 11.0, -3.0, -13.0, -11.0, -14.0],
     [7, 0, 2, 2, 0, -2, 6, 4, -4, 4, -4, 6, -2, -6, -6, -7]),
]


def int4_tie_case():
    W = np.zeros((16, 16), dtype=np.float16)
    mask = np.zeros((16, 16), bool)
    for r, (w, _) in enumerate(INT4_TIE_ROWS):
        W[r] = w
        mask[r] = True
    return W, mask


def int4_ties_hold(quantize):
    W, mask = int4_tie_case()
    scales, q = quantize(W, mask)
    if scales[0] != 1.0 or scales[1] != 2.0:
        return False
    return all(q[r].tolist() == codes for r, (_, codes) in enumerate(INT4_TIE_ROWS))


def mutant_quantize_half_away(W, mask):
    """The INT4 rule with C's round (ties away from zero) in place of rint."""
    Wd = W.astype(np.float64)
    amax = np.where(mask, np.abs(Wd), 0.0).max(axis=1)
    scales = ob.fp16_rne(amax / 7.0)
    s64 = scales.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = Wd / s64[:, None]
    q = np.where(s64[:, None] > 0, np.sign(t) * np.floor(np.abs(t) + 0.5), 0.0)
    return scales, np.where(mask, np.clip(q, -8, 7), 0).astype(np.int8)


def test_int4_rounding_ties_half_even():
    """Exact .5 quotients round to the even code (the RTN rule with ties to
    even); a quantiser that rounds ties away from zero fails this pin."""
    assert int4_ties_hold(ob.quantize_rows_i4)
    assert not int4_ties_hold(mutant_quantize_half_away)
    # The same codes come out of the encoded INT4 buffers.
    W, mask = int4_tie_case()
    enc = ob.encode_i4(W, mask, 16, 16)
    q, Wd = ob.decode_i4(enc)
    for r, (w, codes) in enumerate(INT4_TIE_ROWS):
        assert q[r].tolist() == codes
        assert Wd[r].tolist() == [c * (1.0 if r == 0 else 2.0) for c in codes]


def test_int4_non_finite_weights_reading():
    """The pages state the INT4 rule for finite weights only; the reading
    taken: a kept NaN makes the row's maximum (so its scale) NaN and every
    code of the row 0; a kept infinity makes the scale infinite, so finite
    weights of the row quantise to 0 and the infinity itself (inf / inf) to 0."""
    W = np.zeros((16, 16), dtype=np.float16)
    W[0, :3] = [0.5, np.nan, -0.25]
    W[1, :3] = [0.5, np.inf, -np.inf]
    W[2, :2] = [0.7, -0.7]
    mask = np.zeros((16, 16), bool)
    mask[:3, :3] = True
    scales, q = ob.quantize_rows_i4(W, mask)
    assert np.isnan(scales[0]) and not q[0].any()
    assert scales[1] == np.inf and not q[1].any()
    assert q[2, 0] == 7 and q[2, 1] == -7            # finite rows unaffected
    W[0, 1] = np.float16(0.0)                         # a NaN outside the mask is ignored
    mask[0, 1] = False
    scales, q = ob.quantize_rows_i4(W, mask)
    assert scales[0] == ob.fp16_rne(0.5 / 7) and q[0, 0] == 7


def test_int4_nibble_packing():
    q = np.array([1, -1, 7, -8, 3], dtype=np.int8)
    assert list(ob.pack_nibbles(q)) == [0xF1, 0x87, 0x03]
    assert np.array_equal(ob.unpack_nibbles(ob.pack_nibbles(q), 5), q)


def test_int4_dequant_exact_and_roundtrip():
    rng = np.random.default_rng(17)
    W = wl.weight_normal(128, 128, rng)
    mask = wl.mask_magnitude(W, 0.5)
    enc = ob.encode_i4(W, mask)
    scales, q = ob.quantize_rows_i4(W, mask)
    q2, Wd = ob.decode_i4(enc)
    assert np.array_equal(q2, q)
    assert np.array_equal(enc.scales.view(np.uint16), scales.view(np.uint16))
    for (m, k) in [(0, 0), (5, 17), (127, 127), (64, 3)]:
        assert Fraction(Wd[m, k]) == Fraction(int(q[m, k])) * Fraction(float(scales[m]))
    # bitmaps come from the mask even where q rounds to 0
    assert enc.nnz == int(mask.sum())
    enc16 = ob.encode(W, mask)
    assert np.array_equal(enc.bitmaps, enc16.bitmaps) and np.array_equal(enc.offsets, enc16.offsets)
    assert enc.values.size == (enc.nnz + 1) // 2
    # quantisation error bounded by half a step on every kept entry
    err = np.abs(Wd - np.where(mask, W.astype(np.float64), 0))
    assert np.all(err <= scales.astype(np.float64)[:, None] / 2 + 1e-12)


# ---------------------------------------------------------------------------
# Planted mistakes: each mutant oracle must fail at least one pin
# ---------------------------------------------------------------------------

def mutant_encode_colmajor_bits(W, mask, gt_m=64, gt_k=64):
    enc = ob.encode(W.T.copy(), None if mask is None else mask.T.copy(), gt_k, gt_m)
    return enc


def mutant_rank_inclusive(bm, p):
    return ob.popcount(bm & ((1 << (p + 1)) - 1))


def test_planted_mistakes_are_caught(golden):
    # column-major positions inside a BitmapTile
    assert not blog_example_checks(golden, mutant_encode_colmajor_bits, ob.masked_popcount)
    # rank counting the position itself
    assert not blog_example_checks(golden, ob.encode, mutant_rank_inclusive)
    # a storage formula without the offsets term
    W, mask, _ = wl.config_case(1, 256, 256, 8, 0.5)
    enc = ob.encode(W, mask)
    assert encoded_bytes(enc) != 8 * enc.geom.nbt + 2 * enc.nnz
    # a transposed operand in the product (Y = X W instead of X W^T on a
    # square W) misses the brute-force sums of the definition
    rng = np.random.default_rng(1)
    Ws = wl.weight_normal(16, 16, rng, sigma=1.0)
    Xs = wl.activations_normal(2, 16, rng)
    exact = [[sum(Fraction(float(Ws[m, k])) * Fraction(float(Xs[n, k])) for k in range(16)) for m in range(16)]
             for n in range(2)]
    Ygood = ob.spmm(ob.encode(Ws, np.ones(Ws.shape, bool), 16, 16), Xs)
    Ytrans = Xs.astype(np.float64) @ Ws.astype(np.float64)
    tol = Fraction(16 * 2.0 ** -52) * 64
    assert all(abs(Fraction(Ygood[n, m]) - exact[n][m]) <= tol for n in range(2) for m in range(16))
    assert not all(abs(Fraction(Ytrans[n, m]) - exact[n][m]) <= tol for n in range(2) for m in range(16))
    # a sign error in one product is outside the tolerance
    Wn = wl.weight_normal(32, 64, rng)
    X = wl.activations_normal(2, 64, rng)
    Wd = Wn.astype(np.float64)
    Yref = ob.spmm_fp64(Wd, X)
    Ybad = Yref.copy()
    k = int(np.argmax(np.abs(Wd[0] * X[0].astype(np.float64))))
    Ybad[0, 0] -= 2 * Wd[0, k] * float(X[0, k])
    assert not ob.compare(Ybad, Yref, ob.abs_bound(Wd, X))[0]


# ---------------------------------------------------------------------------
# Workload generators (shapes and statistics of the stand-in inputs)
# ---------------------------------------------------------------------------

def test_magnitude_mask_drops_smallest_with_index_ties():
    W = np.array([[0.5, -0.25, 0.25, 0.0], [0.125, -0.5, 0.25, 1.0]], dtype=np.float16)
    keep = wl.mask_magnitude(W, 0.5)
    # drop 4: 0.0, then 0.125, then the first two of the three 0.25s
    assert keep.tolist() == [[True, False, False, False], [False, True, True, True]]


def test_beta_rows_mask_mean():
    rng = np.random.default_rng(2)
    m = wl.mask_beta_rows(2048, 512, 0.6, rng)
    assert abs(m.mean() - 0.4) < 0.005
    per_row = m.mean(axis=1)
    assert per_row.std() > 0.1          # nonuniform rows
