"""Property tests (hypothesis) of the host encoders against the oracle:
random M and K as multiples of the tile, masks at density 0, 1 and random,
kept exact zeros and -0.0 included.  For every drawn case the C++ encoder's
buffers equal the oracle's byte for byte and the oracle decodes them back to
W (mask applied); TCA-BME (fp16, INT4), IE-BME (fp16, INT4, 2-bit; plain and
reordered LTs) and Tiled-CBC.  No kernel is launched."""
import numpy as np
import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

import unstructured_sparse_weight_amd as usw  # noqa: E402
from oracle import ie_bme as ou  # noqa: E402
from oracle import tca_bme as ob  # noqa: E402
from oracle import tiled_cbc as oc  # noqa: E402

SETTINGS = settings(max_examples=25, deadline=None, suppress_health_check=[HealthCheck.too_slow])
VT = {"f16": ob.VAL_F16, "i4": ob.VAL_I4, "i2": ob.VAL_I2}


@st.composite
def weights_and_mask(draw, tile_m, tile_k, max_m=4, max_k=4):
    M = tile_m * draw(st.integers(1, max_m))
    K = tile_k * draw(st.integers(1, max_k))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    kind = draw(st.sampled_from(["empty", "full", "random"]))
    rng = np.random.default_rng(seed)
    W = (rng.normal(0.0, 1.0, size=(M, K))).astype(np.float16)
    W[rng.random((M, K)) < 0.1] = np.float16(0.0)
    W[rng.random((M, K)) < 0.1] = np.float16(-0.0)
    if kind == "empty":
        mask = np.zeros((M, K), bool)
    elif kind == "full":
        mask = np.ones((M, K), bool)
    else:
        mask = rng.random((M, K)) < draw(st.floats(0.0, 1.0))
    return W, mask, seed


def same_bytes(h, o, values_logical):
    assert np.array_equal(h.bitmaps, o.bitmaps)
    assert np.array_equal(h.offsets, o.offsets)
    vb = o.values.view(np.uint8).reshape(-1)
    assert values_logical == vb.size
    assert np.array_equal(h.values[:values_logical], vb)
    assert not h.values[values_logical:].any()
    if o.scales is not None:
        assert np.array_equal(h.scales, o.scales.view(np.uint16))


@SETTINGS
@given(case=weights_and_mask(16, 16), gt=st.sampled_from([(16, 16), (32, 16), (16, 32), (64, 64)]),
       dtype=st.sampled_from(["f16", "i4"]))
def test_tca_bme_encoder_property(case, gt, dtype):
    W, mask, _ = case
    M, K = W.shape
    if M % gt[0] or K % gt[1]:
        gt = (16, 16)
    h = usw.encode_host(W, mask, gt, dtype)
    o = (ob.encode if dtype == "f16" else ob.encode_i4)(W, mask, *gt)
    assert h.nnz == o.nnz == int(mask.sum())
    same_bytes(h, o, h.values_bytes)
    usw.validate(h)
    if dtype == "f16":
        assert np.array_equal(ob.decode(o).view(np.uint16), np.where(mask, W, np.float16(0)).view(np.uint16))
    else:
        assert np.array_equal(ob.decode_i4(o)[0], ob.quantize_rows_i4(W, mask)[1])


@SETTINGS
@given(case=weights_and_mask(16, 64), dtype=st.sampled_from(["f16", "i4", "i2"]),
       layout=st.sampled_from([((16, 64), (2, 2)), ((16, 64), (4, 1)), ((16, 32), (1, 2))]),
       reorder=st.booleans())
def test_union_encoder_property(case, dtype, layout, reorder):
    W, mask, seed = case
    lt, areas = layout
    M, K = W.shape
    if K % lt[1]:
        lt = (lt[0], 32)
    nlt = (M // lt[0]) * (K // lt[1])
    perms = None
    if reorder:
        rng = np.random.default_rng(seed + 1)
        perms = np.array([rng.permutation(lt[0]) for _ in range(nlt)], dtype=np.int32)
    h = usw.union_encode_host(W, mask, lt, areas, dtype, perm=perms)
    if perms is None:
        o = ou.encode_union(W, mask, lt[0], lt[1], *areas, VT[dtype])
    else:
        o = ou.encode_union_reordered(W, mask, perms, lt[0], lt[1], *areas, VT[dtype])
        assert np.array_equal(h.rowmap, o.rowmap.reshape(-1))
    assert h.payload == o.payload
    same_bytes(h, o, h.values_bytes)
    usw.union_validate(h)
    dec = ou.decode_union(o)
    if dtype == "f16":
        assert np.array_equal(dec, np.where(mask, W, np.float16(0)).view(np.uint16))
    elif dtype == "i4":
        assert np.array_equal(dec, ob.quantize_rows_i4(W, mask)[1])
    else:
        assert np.array_equal(dec, ob.quantize_rows_i2(W, mask)[1])


@SETTINGS
@given(case=weights_and_mask(256, 16, max_m=2, max_k=3))
def test_cbc_encoder_property(case):
    W, mask, _ = case
    h = usw.cbc_encode_host(W, mask)
    o = oc.encode_cbc(W, mask)
    assert h.nnz == o.nnz and h.nnz_padded == o.nnz_padded
    assert np.array_equal(h.bitmaps, o.bitmaps)
    assert np.array_equal(h.tile_offsets, o.tile_offsets)
    assert np.array_equal(h.colinfo, o.colinfo)
    assert np.array_equal(h.values[:o.nnz_padded], o.values.view(np.uint16))
    usw.cbc_validate(h)
    assert np.array_equal(oc.decode_cbc(o), np.where(mask, W, np.float16(0)).view(np.uint16))
