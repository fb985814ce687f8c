"""CPU tests of the IE-BME union-mask entry points of the C-ABI library: the
host encoder writes exactly the oracle's bytes, the validator catches
corruption, and every argument error returns before anything is launched.
No kernel is launched here."""
import ctypes

import numpy as np
import pytest

import unstructured_sparse_weight_amd as usw
import workloads as wl
from oracle import ie_bme as ou
from oracle import tca_bme as ob

VT = {"f16": ob.VAL_F16, "i4": ob.VAL_I4}
B = ctypes.byref


def assert_same_union(h, o):
    assert h.payload == o.payload
    assert np.array_equal(h.bitmaps, o.bitmaps)
    assert np.array_equal(h.offsets, o.offsets)
    vb = o.values.view(np.uint8).reshape(-1)
    assert h.values_bytes == vb.size
    assert np.array_equal(h.values[: h.values_bytes], vb)
    assert not h.values[h.values_bytes:].any()
    assert h.values.size % 16 == 0 and h.values.size >= max(16, vb.size)
    if o.scales is not None:
        assert np.array_equal(h.scales, o.scales.view(np.uint16))


@pytest.mark.parametrize("lt,areas", [((64, 64), (2, 2)), ((32, 64), (2, 1)), ((16, 128), (1, 2)),
                                      ((64, 64), (4, 1)), ((64, 32), (1, 1))])
@pytest.mark.parametrize("density", [0.0, 0.3, 1.0])
@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_union_encoder_matches_oracle(lt, areas, density, dtype):
    rng = np.random.default_rng(int(density * 10) + lt[0] + 3 * lt[1] + 11 * areas[0])
    M, K = 128, 256
    W = wl.weight_normal(M, K, rng)
    W[rng.random((M, K)) < 0.05] = np.float16(-0.0)
    mask = wl.mask_bernoulli(M, K, density, rng)
    h = usw.union_encode_host(W, mask, lt, areas, dtype)
    o = ou.encode_union(W, mask, lt[0], lt[1], areas[0], areas[1], VT[dtype])
    assert_same_union(h, o)
    usw.union_validate(h)


def test_union_encoder_null_mask_matches_oracle():
    rng = np.random.default_rng(5)
    W = wl.weight_normal(64, 128, rng)
    W[rng.random(W.shape) < 0.5] = np.float16(0.0)
    W[0, 0] = np.float16(-0.0)
    for dtype in ("f16", "i4"):
        Wt = W.copy()
        if dtype == "f16":
            Wt[3, 7] = np.float16(np.nan)    # kept without a mask (a NaN has no INT4 code)
        h = usw.union_encode_host(Wt, None, (64, 64), (2, 2), dtype)
        o = ou.encode_union(Wt, None, 64, 64, 2, 2, VT[dtype])
        assert_same_union(h, o)


def test_union_encoder_full_size_int4():
    """The INT4 FFN-up layer (20480 x 5120, magnitude 50%), bit for bit."""
    W, mask, _ = wl.config_case(5, 20480, 5120, 2, 0.5)
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4")
    o = ou.encode_union(W, mask, 64, 64, 2, 2, ob.VAL_I4)
    assert_same_union(h, o)
    usw.union_validate(h)


def fmt_of(h, **over):
    f = h.fmt()
    for k, v in over.items():
        setattr(f, k, v)
    return f


def test_union_validate_detects_corruption():
    rng = np.random.default_rng(6)
    W = wl.weight_normal(128, 256, rng)
    mask = wl.mask_bernoulli(128, 256, 0.4, rng)
    h = usw.union_encode_host(W, mask)
    L = usw.lib()
    for mutate in ("bump", "by_one_group", "last", "first", "word"):
        off = h.offsets.copy()
        bm = h.bitmaps.copy()
        if mutate == "bump":
            off[3] += 1
        elif mutate == "by_one_group":      # a multiple of Q that disagrees with the words
            off[3:] += 4
        elif mutate == "last":
            off[-1] += 4
        elif mutate == "first":
            off[0] = 4
        else:
            bm[20] ^= np.uint64(1 << 33)
        f = fmt_of(h, offsets=off.ctypes.data, bitmaps=bm.ctypes.data,
                   payload=int(off[-1]) if mutate == "by_one_group" else h.payload)
        assert L.usw_union_validate(B(f)) == -8, mutate


@pytest.mark.host_pointers
def test_union_argument_errors_return_before_launch():
    L = usw.lib()
    rng = np.random.default_rng(7)
    W = wl.weight_normal(256, 512, rng)
    mask = wl.mask_bernoulli(256, 512, 0.5, rng)
    h = usw.union_encode_host(W, mask)
    f = h.fmt()
    sz = ctypes.c_size_t()
    # workspace: 4 strips of counters (256 B) plus splits * 16 * M fp32
    assert L.usw_union_spmm_workspace(B(f), 8, 2, B(sz)) == 0 and sz.value == 256 + 2 * 16 * 256 * 4
    assert L.usw_union_spmm_workspace(B(f), 20, 2, B(sz)) == 0 and sz.value == 256 + 2 * 32 * 256 * 4
    assert L.usw_union_spmm_workspace(B(f), 8, 1, B(sz)) == 0 and sz.value == 0
    assert L.usw_union_spmm_counter_bytes(B(f), 8, 2, B(sz)) == 0 and sz.value == 256
    assert L.usw_union_spmm_counter_bytes(B(f), 8, 1, B(sz)) == 0 and sz.value == 0
    # the factor is clamped to K / 256
    assert L.usw_union_spmm_workspace(B(f), 8, 9, B(sz)) == 0 and sz.value == 256 + 2 * 16 * 256 * 4
    assert L.usw_union_spmm_workspace(B(f), 0, 0, B(sz)) == -4
    assert L.usw_union_spmm_workspace(None, 8, 0, B(sz)) == -1
    assert L.usw_union_spmm_workspace(B(f), 8, 0, None) == -1
    assert L.usw_union_spmm_workspace(B(fmt_of(h, M=250)), 8, 0, B(sz)) == -2
    assert L.usw_union_spmm_workspace(B(fmt_of(h, r_a=3)), 8, 0, B(sz)) == -2
    assert L.usw_union_spmm_workspace(B(fmt_of(h, val_type=7)), 8, 0, B(sz)) == -3
    # valid formats the kernel does not take
    assert L.usw_union_spmm_workspace(B(fmt_of(h, val_type=1)), 8, 0, B(sz)) == -5
    assert L.usw_union_spmm_workspace(B(fmt_of(h, lt_k=32)), 8, 0, B(sz)) == -5          # LTs 64 columns wide
    assert L.usw_union_spmm_workspace(B(fmt_of(h, c_a=16)), 8, 0, B(sz)) == -5           # areas 4 columns wide
    assert L.usw_union_spmm_workspace(B(fmt_of(h, lt_m=128)), 8, 0, B(sz)) == -5         # LTs taller than a strip
    assert L.usw_union_spmm_workspace(B(fmt_of(h, lt_m=8, r_a=1, c_a=4)), 8, 0, B(sz)) == -5
    # other area grids and LT heights of 16, 32 and 64 rows run
    assert L.usw_union_spmm_workspace(B(fmt_of(h, r_a=4, c_a=1)), 8, 0, B(sz)) == 0
    assert L.usw_union_spmm_workspace(B(fmt_of(h, lt_m=32)), 8, 0, B(sz)) == 0
    assert L.usw_union_spmm_workspace(B(fmt_of(h, r_a=1, c_a=8)), 8, 0, B(sz)) == 0
    # spmm argument checks (host pointers: any launch would fail)
    x = np.zeros((8, 512), np.uint16)
    y = np.zeros((8, 256), np.uint16)
    xa, ya = x.ctypes.data, y.ctypes.data
    assert L.usw_union_spmm(None, xa, ya, 1, 8, 0, None, 0, None) == -1
    assert L.usw_union_spmm(B(f), None, ya, 1, 8, 0, None, 0, None) == -1
    assert L.usw_union_spmm(B(f), xa, None, 1, 8, 0, None, 0, None) == -1
    assert L.usw_union_spmm(B(fmt_of(h, scales=None)), xa, ya, 1, 8, 0, None, 0, None) == -1
    assert L.usw_union_spmm(B(f), xa, ya, 2, 8, 0, None, 0, None) == -3
    assert L.usw_union_spmm(B(f), xa, ya, 1, 0, 0, None, 0, None) == -4
    assert L.usw_union_spmm(B(f), xa + 2, ya, 1, 8, 1, None, 0, None) == -6
    assert L.usw_union_spmm(B(f), xa, ya + 4, 1, 8, 1, None, 0, None) == -6
    assert L.usw_union_spmm(B(fmt_of(h, values=h.values.ctypes.data + 2)), xa, ya, 1, 8, 1, None, 0, None) == -6
    assert L.usw_union_spmm(B(fmt_of(h, reserved=1)), xa, ya, 1, 8, 0, None, 0, None) == -2
    assert L.usw_union_spmm(B(f), xa, ya, 1, 8, 2, None, 0, None) == -7
    small = np.zeros(16, np.uint8)
    assert L.usw_union_spmm(B(f), xa, ya, 1, 8, 2, small.ctypes.data, 16, None) == -7
    # encode argument checks
    pl = ctypes.c_int64()
    assert L.usw_union_encode_query(None, None, 256, 512, 64, 64, 2, 2, 2, B(pl), None, None, None, None, None) == -1
    assert L.usw_union_encode_query(W.ctypes.data, None, 256, 512, 64, 48, 2, 2, 2, B(pl),
                                    None, None, None, None, None) == -2
    # 4 x 8 areas: 32 union bits per LT, not whole 64-bit words
    assert L.usw_union_encode_query(W.ctypes.data, None, 256, 512, 16, 32, 4, 4, 2, B(pl),
                                    None, None, None, None, None) == -2
    assert L.usw_union_encode_query(W.ctypes.data, None, 256, 512, 16, 32, 2, 2, 2, B(pl),
                                    None, None, None, None, None) == 0
    assert L.usw_union_encode_query(W.ctypes.data, None, 256, 512, 64, 64, 2, 2, 9, B(pl),
                                    None, None, None, None, None) == -3
    vals = np.zeros(4, np.uint8)
    bm_out, off_out = h.bitmaps.copy(), h.offsets.copy()     # kept alive across the calls
    assert L.usw_union_encode(W.ctypes.data, None, 256, 512, 64, 64, 2, 2, 1, bm_out.ctypes.data,
                              off_out.ctypes.data, vals.ctypes.data, 4, None) == -10
    assert L.usw_union_encode(W.ctypes.data, None, 256, 512, 64, 64, 2, 2, 2, bm_out.ctypes.data,
                              off_out.ctypes.data, vals.ctypes.data, 4, None) == -1
