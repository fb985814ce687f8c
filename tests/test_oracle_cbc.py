"""Pins for the Tiled-CBC / dynamic-pruning oracle ("Unified Static-Dynamic
Pruning for Efficient LLM Inference", sections 2.2, 3.2.3, 4.1 and 4.2):
the storage equation, the ColInfo packing, bit order, independent encoders,
round trips, the skip-equals-zero identity against the TCA-BME oracle,
brute force on tiny inputs, and planted mistakes.

Runs on the CPU only.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import tca_bme as ob
from oracle import tiled_cbc as oc
import workloads as wl


def rng(i):
    return np.random.default_rng((7, 23, i))


def rand_w(M, K, r):
    w = r.normal(0.0, 1.0, size=(M, K))
    w = np.where(np.abs(w) < 1e-3, 1e-3, w)
    return w.astype(np.float16)


def test_storage_equation_without_padding():
    """Every column keeps a multiple of 8 values: no padding, and the bytes
    are exactly 4 (NGT+1) + 4 NGT TILE_K + 8 NBM + 2 NNZ (section 4.1)."""
    M, K = 512, 64
    r = rng(0)
    mask = np.zeros((M, K), dtype=bool)
    for ti in range(M // 256):
        for k in range(K):
            rows = r.choice(256, size=8 * int(r.integers(0, 33)), replace=False)
            mask[ti * 256 + rows, k] = True
    W = rand_w(M, K, r)
    enc = oc.encode_cbc(W, mask)
    g = enc.geom
    assert enc.nnz == enc.nnz_padded == int(mask.sum())
    total = enc.tile_offsets.nbytes + enc.colinfo.nbytes + enc.bitmaps.nbytes + enc.values.nbytes
    assert total == oc.storage_bytes_cbc(g.ngt, g.tile_k, g.nbm, enc.nnz)
    assert oc.storage_bytes_cbc(g.ngt, 16, g.nbm, 0) == 4 * (g.ngt + 1) + 64 * g.ngt + 8 * M * K // 64


def test_colinfo_packing_and_padding():
    """ColInfo: column offset inside the tile in the upper 16 bits, kept
    count in the lower 16; runs padded to 8 values (16 bytes)."""
    W = np.zeros((256, 16), dtype=np.float16)
    mask = np.zeros((256, 16), dtype=bool)
    mask[[3, 70, 200], 0] = True           # 3 kept -> run of 8
    mask[:, 1] = True                      # 256 kept -> run of 256
    mask[5, 3] = True                      # column 2 empty, column 3 one kept
    W[[3, 70, 200], 0] = [1.0, 2.0, 3.0]
    W[:, 1] = np.arange(256, dtype=np.float16) / np.float16(4)
    W[5, 3] = 7.0
    for fn in (oc.encode_cbc, oc.encode_cbc_loop):
        enc = fn(W, mask)
        ci = [int(v) for v in enc.colinfo[:4]]
        assert ci == [(0 << 16) | 3, (8 << 16) | 256, (264 << 16) | 0, (264 << 16) | 1]
        assert int(enc.tile_offsets[1]) == 8 + 256 + 0 + 8
        vals = enc.values.view(np.float16).astype(np.float64)
        assert list(vals[:8]) == [1.0, 2.0, 3.0, 0, 0, 0, 0, 0]
        assert vals[8] == 0.0 and vals[9] == 0.25 and vals[8 + 255] == 63.75
        assert list(vals[264:272]) == [7.0, 0, 0, 0, 0, 0, 0, 0]


def test_bit_order():
    """A single kept weight at row r of column c sets bit r % 64 of word
    r // 64 of that column."""
    for r_ in (0, 1, 63, 64, 130, 255):
        for c in (0, 7, 15):
            W = np.ones((256, 16), dtype=np.float16)
            mask = np.zeros((256, 16), dtype=bool)
            mask[r_, c] = True
            enc = oc.encode_cbc(W, mask)
            words = enc.bitmaps.reshape(16, 4)
            expect = np.zeros((16, 4), dtype=np.uint64)
            expect[c, r_ // 64] = np.uint64(1) << np.uint64(r_ % 64)
            assert np.array_equal(words, expect)


@pytest.mark.parametrize("shape,keep", [((256, 16), 0.5), ((512, 96), 0.3), ((768, 48), 0.9), ((256, 32), 0.0),
                                        ((256, 32), 1.0)])
def test_two_encoders_and_round_trip(shape, keep):
    M, K = shape
    r = rng(int(keep * 10) + M + K)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < keep
    a = oc.encode_cbc(W, mask)
    b = oc.encode_cbc_loop(W, mask)
    for f in ("bitmaps", "tile_offsets", "colinfo", "values"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    expect = np.where(mask, W, np.float16(0)).view(np.uint16)
    assert np.array_equal(oc.decode_cbc(a), expect)
    assert np.array_equal(oc.decode_cbc_loop(a), expect)


def test_skip_equals_zeroed_activations():
    """Skipping the columns with |x_k| < tau is the static product with those
    entries of x set to zero, here through the TCA-BME oracle."""
    M, K = 512, 256
    r = rng(4)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < 0.5
    x = r.normal(size=K).astype(np.float16)
    enc = oc.encode_cbc(W, mask)
    for tau in (0.0, 0.3, 0.7, float(np.abs(x.astype(np.float32)).max()), 1e9):
        xz = np.where(np.abs(x.astype(np.float32)) >= np.float32(tau), x, np.float16(0))
        ref = ob.spmm(ob.encode(W, mask), xz[None, :])[0]
        assert np.array_equal(oc.spmspv(enc, x, tau), ref)
    assert not oc.spmspv(enc, x, 1e9).any()
    assert np.array_equal(oc.spmspv(enc, x, 0.0), ob.spmm(ob.encode(W, mask), x[None, :])[0])


def test_threshold_is_inclusive_in_fp32():
    x = np.array([0.5, -0.5, 0.49951171875, 0.0, -0.0], dtype=np.float16)
    assert list(oc.dp_active(x, 0.5)) == [True, True, False, False, False]
    assert list(oc.dp_active(x, 0.0)) == [True] * 5


def test_product_brute_force_fraction():
    M, K = 256, 32
    r = rng(5)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < 0.4
    x = r.normal(size=K).astype(np.float16)
    tau = 0.6
    enc = oc.encode_cbc(W, mask)
    y = oc.spmspv(enc, x, tau)
    for m in range(0, M, 7):
        s = sum(Fraction(float(W[m, k])) * Fraction(float(x[k])) for k in range(K)
                if mask[m, k] and abs(float(x[k])) >= tau)
        assert abs(float(s) - y[m]) <= 1e-12 * max(1.0, abs(float(s)))


def test_ci_equation():
    """Equation (3): s = 0 gives the static CI M N / (M / CR + N); the CI
    grows as 1 / (1 - s) when the weight term dominates."""
    assert oc.ci_spdp(8192, 1, 2.0, 0.0) == pytest.approx(8192 / (4096 + 1))
    assert oc.ci_spdp(8192, 1, 2.0, 0.5) == pytest.approx(8192 / (2048 + 1))


def test_planted_mistakes_fail():
    M, K = 256, 32
    r = rng(6)
    W = rand_w(M, K, r)
    mask = r.random((M, K)) < 0.5
    enc = oc.encode_cbc(W, mask)
    # Values taken row by row inside the tile instead of column by column.
    rowwise = W.view(np.uint16)[mask]
    assert not np.array_equal(enc.values[enc.values != 0][:rowwise.size], rowwise)
    # ColInfo fields swapped fails the consistency check.
    bad = oc.CbcEncoded(enc.geom, enc.nnz, enc.nnz_padded, enc.bitmaps, enc.tile_offsets,
                        ((enc.colinfo & 0xFFFF) << 16) | (enc.colinfo >> 16), enc.values)
    with pytest.raises(ValueError):
        oc.check_cbc(bad)
    # An exclusive threshold (>) drops the boundary column.
    x = np.zeros(K, dtype=np.float16)
    x[5] = np.float16(0.5)
    W1 = np.ones((M, K), dtype=np.float16)
    e1 = oc.encode_cbc(W1, None)
    assert oc.spmspv(e1, x, 0.5)[0] == 0.5
    assert (np.abs(x.astype(np.float32)) > np.float32(0.5)).sum() == 0
    # Bitmap words read most-significant bit first break the round trip.
    flipped = np.array([int(f"{int(w):064b}"[::-1], 2) for w in enc.bitmaps], dtype=np.uint64)
    bad2 = oc.CbcEncoded(enc.geom, enc.nnz, enc.nnz_padded, flipped, enc.tile_offsets, enc.colinfo, enc.values)
    assert not np.array_equal(oc.decode_cbc(bad2), oc.decode_cbc(enc))
