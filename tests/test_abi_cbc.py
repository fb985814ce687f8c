"""CPU tests of the Tiled-CBC entry points of the C-ABI library: the host
encoder writes exactly the oracle's bytes, the validator catches corruption,
and every argument error returns before anything is launched.  No kernel is
launched here."""
import ctypes

import numpy as np
import pytest

import unstructured_sparse_weight_amd as usw
import workloads as wl
from oracle import tiled_cbc as oc

B = ctypes.byref


def assert_same_cbc(h, o):
    assert h.nnz == o.nnz and h.nnz_padded == o.nnz_padded
    assert np.array_equal(h.bitmaps, o.bitmaps)
    assert np.array_equal(h.tile_offsets, o.tile_offsets)
    assert np.array_equal(h.colinfo, o.colinfo)
    assert np.array_equal(h.values[: h.nnz_padded], o.values)
    assert not h.values[h.nnz_padded:].any()


@pytest.mark.parametrize("shape", [(256, 16), (512, 96), (768, 48), (256, 1024)])
@pytest.mark.parametrize("density", [0.0, 0.05, 0.5, 1.0])
def test_cbc_encoder_matches_oracle(shape, density):
    M, K = shape
    rng = np.random.default_rng(int(density * 100) + M + K)
    W = wl.weight_normal(M, K, rng)
    W[rng.random((M, K)) < 0.05] = np.float16(-0.0)
    mask = wl.mask_bernoulli(M, K, density, rng)
    h = usw.cbc_encode_host(W, mask)
    assert_same_cbc(h, oc.encode_cbc(W, mask))
    usw.cbc_validate(h)


def test_cbc_encoder_null_mask_matches_oracle():
    rng = np.random.default_rng(5)
    W = wl.weight_normal(256, 64, rng)
    W[rng.random(W.shape) < 0.5] = np.float16(0.0)
    W[0, 0] = np.float16(-0.0)
    W[3, 7] = np.float16(np.nan)
    assert_same_cbc(usw.cbc_encode_host(W, None), oc.encode_cbc(W, None))


def test_cbc_encoder_full_size():
    """The FFN-up layer (20480 x 5120, magnitude 50%), bit for bit."""
    W, mask, _ = wl.config_case(2, 20480, 5120, 1, 0.5, layer_id=2)
    h = usw.cbc_encode_host(W, mask)
    assert_same_cbc(h, oc.encode_cbc(W, mask))
    usw.cbc_validate(h)


def fmt_of(h, **over):
    f = h.fmt()
    for k, v in over.items():
        setattr(f, k, v)
    return f


def test_cbc_validate_detects_corruption():
    rng = np.random.default_rng(6)
    W = wl.weight_normal(512, 64, rng)
    mask = wl.mask_bernoulli(512, 64, 0.4, rng)
    h = usw.cbc_encode_host(W, mask)
    L = usw.lib()
    for mutate in ("offset", "last", "count", "colstart", "word"):
        off, ci, bm = h.tile_offsets.copy(), h.colinfo.copy(), h.bitmaps.copy()
        if mutate == "offset":
            off[2] += 8
        elif mutate == "last":
            off[-1] += 8
        elif mutate == "count":
            ci[5] += 1
        elif mutate == "colstart":
            ci[5] += 8 << 16
        else:
            bm[9] ^= np.uint64(1 << 17)
        f = fmt_of(h, tile_offsets=off.ctypes.data, colinfo=ci.ctypes.data, bitmaps=bm.ctypes.data)
        assert L.usw_cbc_validate(B(f)) == -8, mutate


@pytest.mark.host_pointers
def test_cbc_argument_errors_return_before_launch():
    L = usw.lib()
    rng = np.random.default_rng(7)
    W = wl.weight_normal(512, 256, rng)
    mask = wl.mask_bernoulli(512, 256, 0.5, rng)
    h = usw.cbc_encode_host(W, mask)
    f = h.fmt()
    sz, cz = ctypes.c_size_t(), ctypes.c_size_t()
    # workspace: 2 strips of counters (256 B) plus splits * M fp32; factor clamped to K / 16
    assert L.usw_cbc_spmspv_workspace(B(f), 3, B(sz), B(cz)) == 0 and sz.value == 256 + 3 * 512 * 4
    assert cz.value == 256
    assert L.usw_cbc_spmspv_workspace(B(f), 99, B(sz), B(cz)) == 0 and sz.value == 256 + 16 * 512 * 4
    assert L.usw_cbc_spmspv_workspace(B(f), 1, B(sz), B(cz)) == 0 and sz.value == 0 and cz.value == 0
    assert L.usw_cbc_spmspv_workspace(None, 0, B(sz), None) == -1
    assert L.usw_cbc_spmspv_workspace(B(f), 0, None, None) == -1
    assert L.usw_cbc_spmspv_workspace(B(fmt_of(h, M=500)), 0, B(sz), None) == -2
    assert L.usw_cbc_spmspv_workspace(B(fmt_of(h, val_type=7)), 0, B(sz), None) == -3
    assert L.usw_cbc_spmspv_workspace(B(fmt_of(h, val_type=2)), 0, B(sz), None) == -5
    assert L.usw_cbc_spmspv_workspace(B(fmt_of(h, tile_k=32)), 0, B(sz), None) == -5
    x = np.zeros(256, np.uint16)
    y = np.zeros(512, np.uint16)
    xa, ya = x.ctypes.data, y.ctypes.data
    assert L.usw_cbc_spmspv(None, xa, ya, 1, 0.0, 1, None, 0, None) == -1
    assert L.usw_cbc_spmspv(B(f), None, ya, 1, 0.0, 1, None, 0, None) == -1
    assert L.usw_cbc_spmspv(B(f), xa, None, 1, 0.0, 1, None, 0, None) == -1
    assert L.usw_cbc_spmspv(B(f), xa, ya, 2, 0.0, 1, None, 0, None) == -3
    assert L.usw_cbc_spmspv(B(f), xa, ya, 1, -1.0, 1, None, 0, None) == -5
    assert L.usw_cbc_spmspv(B(f), xa, ya, 1, float("nan"), 1, None, 0, None) == -5
    assert L.usw_cbc_spmspv(B(f), xa + 2, ya, 1, 0.0, 1, None, 0, None) == -6
    assert L.usw_cbc_spmspv(B(fmt_of(h, values=h.values.ctypes.data + 2)), xa, ya, 1, 0.0, 1, None, 0, None) == -6
    assert L.usw_cbc_spmspv(B(fmt_of(h, reserved=1)), xa, ya, 1, 0.0, 1, None, 0, None) == -2
    assert L.usw_cbc_spmspv(B(f), xa, ya, 1, 0.0, 2, None, 0, None) == -7
    small = np.zeros(16, np.uint8)
    assert L.usw_cbc_spmspv(B(f), xa, ya, 1, 0.0, 2, small.ctypes.data, 16, None) == -7
    nnz, npad = ctypes.c_int64(), ctypes.c_int64()
    assert L.usw_cbc_encode_query(None, None, 512, 256, B(nnz), B(npad), None, None, None, None) == -1
    assert L.usw_cbc_encode_query(W.ctypes.data, None, 500, 256, B(nnz), B(npad), None, None, None, None) == -2
    assert L.usw_cbc_encode_query(W.ctypes.data, None, 512, 250, B(nnz), B(npad), None, None, None, None) == -2
    vals = np.zeros(4, np.uint16)
    bm_out, to_out, ci_out = h.bitmaps.copy(), h.tile_offsets.copy(), h.colinfo.copy()   # kept alive
    assert L.usw_cbc_encode(W.ctypes.data, None, 512, 256, bm_out.ctypes.data,
                            to_out.ctypes.data, ci_out.ctypes.data,
                            vals.ctypes.data, 8) == -10
