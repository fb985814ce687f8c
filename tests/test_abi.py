"""CPU tests of the C-ABI library: it loads, exports every declared symbol,
rejects bad arguments before launching anything, and its host encoder writes
exactly the oracle's bytes.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import unstructured_sparse_weight_amd as usw
from unstructured_sparse_weight_amd import _lib
import workloads as wl
from oracle import tca_bme as ob

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    txt = open(os.path.join(ROOT, "include", "usw.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(usw_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = usw.lib()
    syms = header_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(L, s), s
    assert set(syms) == set(_lib.EXPORTED)
    assert L.usw_abi_version() == 1
    assert L.usw_status_str(0) == b"ok"
    for code in range(-10, 0):
        assert L.usw_status_str(code) not in (b"ok", b"unknown status")


def assert_same_encoding(h, o):
    assert h.nnz == o.nnz
    assert np.array_equal(h.bitmaps, o.bitmaps)
    assert np.array_equal(h.offsets, o.offsets)
    vb = o.values.view(np.uint8).reshape(-1)
    assert h.values_bytes == vb.size
    assert np.array_equal(h.values[: h.values_bytes], vb)
    assert not h.values[h.values_bytes:].any()          # padding is zero
    assert h.values.size % 16 == 0 and h.values.size >= max(16, vb.size)
    if o.scales is not None:
        assert np.array_equal(h.scales, o.scales.view(np.uint16))


@pytest.mark.parametrize("gt", [(64, 64), (32, 64), (16, 16), (64, 32)])
@pytest.mark.parametrize("density", [0.0, 0.5, 1.0])
@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_encoder_matches_oracle_small(gt, density, dtype):
    rng = np.random.default_rng(int(density * 10) + gt[0] + 7 * gt[1])
    M, K = 128, 192
    W = wl.weight_normal(M, K, rng)
    W[rng.random((M, K)) < 0.05] = np.float16(0.0)
    W[rng.random((M, K)) < 0.05] = np.float16(-0.0)
    mask = wl.mask_bernoulli(M, K, density, rng)
    h = usw.encode_host(W, mask, gt, dtype)
    o = (ob.encode if dtype == "f16" else ob.encode_i4)(W, mask, *gt)
    assert_same_encoding(h, o)
    usw.validate(h)


def test_encoder_null_mask_matches_oracle():
    rng = np.random.default_rng(4)
    W = wl.weight_normal(64, 128, rng)
    W[rng.random(W.shape) < 0.4] = np.float16(0.0)
    W[0, 0] = np.float16(-0.0)
    W[0, 1] = np.float16(np.nan)
    h = usw.encode_host(W, None)
    o = ob.encode(W, None)
    assert_same_encoding(h, o)


def test_int4_encoder_non_finite_weights_match_oracle():
    """Kept NaN and infinities in INT4 mode: scales and codes as the oracle's
    reading (NaN row scale with zero codes; infinite scale, codes 0)."""
    rng = np.random.default_rng(4)
    W = wl.weight_normal(64, 128, rng)
    W[rng.random(W.shape) < 0.4] = np.float16(0.0)
    W[0, 1] = np.float16(np.nan)
    W[1, 5] = np.float16(np.inf)
    W[2, 7] = np.float16(-np.inf)
    W[3, 9] = np.float16(np.nan)
    h = usw.encode_host(W, None, (64, 64), "i4")
    o = ob.encode_i4(W, None)
    assert_same_encoding(h, o)
    assert h.scales[0] == 0x7E00 and h.scales[1] == 0x7C00


@pytest.mark.parametrize("config_id", [1, 2, 3, 4, 5])
def test_encoder_matches_oracle_configs(config_id):
    """Bit-exact buffers on every workload (full-size shapes for the first
    layer of each; the tiny workload at its only size)."""
    if config_id == 1:
        W, mask, _ = wl.config_case(1, 256, 256, 8, 0.5)
    elif config_id == 2:
        W, mask, _ = wl.config_case(2, 5120, 5120, 16, 0.5, layer_id=1)      # attn-out
    elif config_id == 3:
        W, mask, _ = wl.config_case(3, 20480, 5120, 16, 0.3, layer_id=3)
    elif config_id == 4:
        W, mask, _ = wl.config_case(4, 4096, 11008, 512, 0.5, layer_id=1)
    else:
        W, mask, _ = wl.config_case(5, 20480, 5120, 2, 0.5)
    dtype = "i4" if config_id == 5 else "f16"
    h = usw.encode_host(W, mask, (64, 64), dtype)
    o = (ob.encode if dtype == "f16" else ob.encode_i4)(W, mask)
    assert_same_encoding(h, o)
    usw.validate(h)


def test_int4_scale_rounding_matches_numpy():
    """The library's fp64 -> fp16 rounding of the row scales against numpy's
    correctly rounded conversion, including subnormal and tie cases."""
    rng = np.random.default_rng(8)
    M, K = 256, 16
    W = np.zeros((M, K), dtype=np.float16)
    amax = np.concatenate([
        rng.uniform(1e-7, 1e-4, 64),                  # scales in the fp16 subnormal range
        rng.uniform(0.01, 60000.0, 64),
        np.float16(np.arange(1, 65)) * np.float16(2.0 ** -14),
        (np.arange(64) + 0.5) * 7 * 2.0 ** -24,       # amax/7 exactly between subnormals
    ])
    W[:, 0] = amax.astype(np.float16)
    W[:, 1] = -W[:, 0] / np.float16(3)
    mask = np.zeros((M, K), bool)
    mask[:, :2] = True
    h = usw.encode_host(W, mask, (16, 16), "i4")
    o = ob.encode_i4(W, mask, 16, 16)
    assert np.array_equal(h.scales, o.scales.view(np.uint16))
    assert_same_encoding(h, o)


def fmt_of(h, **over):
    f = h.fmt()
    for k, v in over.items():
        setattr(f, k, v)
    return f


def test_validate_detects_corruption():
    W, mask, _ = wl.config_case(1, 256, 256, 8, 0.5)
    h = usw.encode_host(W, mask)
    usw.validate(h)
    L = usw.lib()
    for mutate in ("bump", "decrease", "last", "first", "bitmap"):
        off = h.offsets.copy()
        bm = h.bitmaps.copy()
        if mutate == "bump":
            off[5] += 1
        elif mutate == "decrease":
            off[6] = off[5] - 1 if off[5] > 0 else 0
            off[5] += 3
        elif mutate == "last":
            off[-1] += 2
        elif mutate == "first":
            off[0] = 1
        else:
            bm[70] ^= np.uint64(1 << 9)
        f = fmt_of(h, offsets=off.ctypes.data, bitmaps=bm.ctypes.data)
        assert L.usw_validate(ctypes.byref(f)) == -8, mutate


@pytest.mark.host_pointers
def test_argument_errors_return_before_launch():
    """Every argument error is reported without touching a GPU (these calls
    pass host pointers and would fail loudly if anything were launched)."""
    L = usw.lib()
    W, mask, X = wl.config_case(1, 256, 256, 8, 0.5)
    h = usw.encode_host(W, mask)
    f = h.fmt()
    B = ctypes.byref
    sz = ctypes.c_size_t()
    # workspace queries
    assert L.usw_spmm_workspace(B(f), 8, B(sz)) == 0
    assert L.usw_spmm_workspace(B(f), 0, B(sz)) == -4
    assert L.usw_spmm_workspace(None, 8, B(sz)) == -1
    assert L.usw_spmm_workspace(B(f), 8, None) == -1
    assert L.usw_spmm_workspace(B(fmt_of(h, M=250)), 8, B(sz)) == -2
    assert L.usw_spmm_workspace(B(fmt_of(h, val_type=7)), 8, B(sz)) == -3
    assert L.usw_spmm_workspace(B(fmt_of(h, gt_m=32, M=256)), 8, B(sz)) == -5
    # INT4 with more than 32 tokens runs in 32-token decode passes
    assert L.usw_spmm_workspace(B(fmt_of(h, val_type=2, scales=h.bitmaps.ctypes.data)), 33, B(sz)) == 0
    # forced split-K needs 256 B of strip counters plus splits * 16 * M fp32
    # partial sums (N <= 16); the factor is clamped to K/256 (tiny: 1, none)
    assert L.usw_spmm_workspace_ex(B(f), 8, 1, B(sz)) == 0 and sz.value == 0
    assert L.usw_spmm_workspace_ex(B(f), 8, 2, B(sz)) == 0 and sz.value == 0
    Ww = wl.weight_normal(64, 512, np.random.default_rng(3))
    hw = usw.encode_host(Ww, None)
    fw = hw.fmt()
    assert L.usw_spmm_workspace_ex(B(fw), 8, 2, B(sz)) == 0 and sz.value == 256 + 2 * 16 * 64 * 4
    assert L.usw_spmm_workspace_ex(B(fw), 20, 9, B(sz)) == 0 and sz.value == 256 + 2 * 32 * 64 * 4
    # spmm argument checks (host pointers: any launch would fail)
    x = np.zeros((8, 256), np.uint16)
    y = np.zeros((8, 256), np.uint16)
    xa = x.ctypes.data
    ya = y.ctypes.data
    assert L.usw_spmm(B(f), None, ya, 1, 8, None, 0, None) == -1
    assert L.usw_spmm(B(f), xa, None, 1, 8, None, 0, None) == -1
    assert L.usw_spmm(B(f), xa, ya, 2, 8, None, 0, None) == -3
    assert L.usw_spmm(B(f), xa, ya, 1, 0, None, 0, None) == -4
    assert L.usw_spmm(B(f), xa, ya, 1, -3, None, 0, None) == -4
    assert L.usw_spmm(B(f), xa + 2, ya, 1, 8, None, 0, None) == -6
    assert L.usw_spmm(B(f), xa, ya + 4, 1, 8, None, 0, None) == -6
    assert L.usw_spmm(B(fmt_of(h, values=h.values.ctypes.data + 2)), xa, ya, 1, 8, None, 0, None) == -6
    assert L.usw_spmm(B(fmt_of(h, reserved=1)), xa, ya, 1, 8, None, 0, None) == -2
    assert L.usw_spmm(B(fmt_of(h, K=200)), xa, ya, 1, 8, None, 0, None) == -2
    xw = np.zeros((8, 512), np.uint16)
    assert L.usw_spmm_ex(B(fw), xw.ctypes.data, ya, 1, 8, 2, None, 0, None) == -7
    small = np.zeros(16, np.uint8)
    assert L.usw_spmm_ex(B(fw), xw.ctypes.data, ya, 1, 8, 2, small.ctypes.data, 16, None) == -7
    # streaming-read probe: argument errors, and nothing to read, return
    # before any launch
    assert L.usw_probe_read(None, 1024, ya, None) == -1
    assert L.usw_probe_read(xa, 1024, None, None) == -1
    assert L.usw_probe_read(xa + 4, 1024, ya, None) == -6
    assert L.usw_probe_read(xa, 15, ya, None) == 0
    # encode argument checks
    nnz = ctypes.c_int64()
    assert L.usw_encode_query(None, None, 256, 256, 64, 64, 1, B(nnz), None, None, None, None, None) == -1
    assert L.usw_encode_query(W.ctypes.data, None, 256, 256, 64, 48, 1, B(nnz), None, None, None, None, None) == -2
    assert L.usw_encode_query(W.ctypes.data, None, 256, 256, 64, 64, 9, B(nnz), None, None, None, None, None) == -3
    vals = np.zeros(4, np.uint8)
    bm_out, off_out = h.bitmaps.copy(), h.offsets.copy()     # kept alive across the calls
    assert L.usw_encode(W.ctypes.data, None, 256, 256, 64, 64, 1, bm_out.ctypes.data,
                        off_out.ctypes.data, vals.ctypes.data, 4, None) == -10
    assert L.usw_encode(W.ctypes.data, None, 256, 256, 64, 64, 2, bm_out.ctypes.data,
                        off_out.ctypes.data, vals.ctypes.data, 4, None) == -1


@pytest.mark.host_pointers
def test_noalloc_argument_errors_return_before_launch():
    """usw_spmm_noalloc reports argument errors, and partial sums that do not
    fit its 16 MiB scratch, before it touches the GPU (host pointers here)."""
    L = usw.lib()
    W, mask, X = wl.config_case(1, 256, 256, 8, 0.5)
    h = usw.encode_host(W, mask)
    f = h.fmt()
    B = ctypes.byref
    x = np.zeros((8, 256), np.uint16)
    y = np.zeros((8, 256), np.uint16)
    xa, ya = x.ctypes.data, y.ctypes.data
    assert L.usw_spmm_noalloc(None, xa, ya, 1, 8, 0, None) == -1
    assert L.usw_spmm_noalloc(B(f), None, ya, 1, 8, 0, None) == -1
    assert L.usw_spmm_noalloc(B(f), xa, None, 1, 8, 0, None) == -1
    assert L.usw_spmm_noalloc(B(f), xa, ya, 2, 8, 0, None) == -3
    assert L.usw_spmm_noalloc(B(f), xa, ya, 1, 0, 0, None) == -4
    assert L.usw_spmm_noalloc(B(f), xa + 2, ya, 1, 8, 0, None) == -6
    assert L.usw_spmm_noalloc(B(fmt_of(h, K=200)), xa, ya, 1, 8, 0, None) == -2
    assert L.usw_spmm_noalloc(B(fmt_of(h, gt_m=32)), xa, ya, 1, 8, 0, None) == -5
    # 16 splits of 32 tokens x 16384 rows of fp32 partial sums (32 MiB) do
    # not fit the scratch: WORKSPACE, checked before any HIP call.
    big = fmt_of(h, M=16384, K=4096, nnz=16384 * 2048)
    sz = ctypes.c_size_t()
    assert L.usw_spmm_workspace_ex(B(big), 32, 16, B(sz)) == 0 and sz.value > 16 << 20
    assert L.usw_spmm_noalloc(B(big), xa, ya, 1, 32, 16, None) == -7


@pytest.mark.host_pointers
def test_device_encoder_argument_errors_return_before_launch():
    """usw_encode_device_index / _values report every argument error before
    any launch (host pointers here: a launch would fail)."""
    L = usw.lib()
    W = np.zeros((256, 256), np.uint16)
    m = np.zeros((256, 256), np.uint8)
    bm = np.zeros(1024, np.uint64)
    off = np.zeros(64, np.uint32)
    sc = np.zeros(256, np.uint16)
    vals = np.zeros(4096, np.uint8)
    w, mp, b, o, s, v = (a.ctypes.data for a in (W, m, bm, off, sc, vals))
    idx = L.usw_encode_device_index
    assert idx(None, mp, 256, 256, 64, 64, 1, b, o, None, None) == -1
    assert idx(w, mp, 256, 256, 64, 64, 1, None, o, None, None) == -1
    assert idx(w, mp, 256, 256, 64, 64, 1, b, None, None, None) == -1
    assert idx(w, mp, 256, 256, 64, 64, 2, b, o, None, None) == -1        # I4 needs scales
    assert idx(w, mp, 256, 250, 64, 64, 1, b, o, None, None) == -2
    assert idx(w, mp, 256, 256, 64, 48, 1, b, o, None, None) == -2
    assert idx(w, mp, 65536, 65536, 64, 64, 1, b, o, None, None) == -2    # M*K >= 2^32
    assert idx(w, mp, 256, 256, 64, 64, 5, b, o, None, None) == -3
    assert idx(w, mp, 256, 256, 128, 64, 1, b, o, None, None) == -5       # 128 BitmapTiles per GroupTile
    assert idx(w + 2, mp, 256, 256, 64, 64, 1, b, o, None, None) == -6
    assert idx(w, mp + 4, 256, 256, 64, 64, 1, b, o, None, None) == -6
    assert idx(w, mp, 256, 256, 64, 64, 1, b + 4, o, None, None) == -6
    assert idx(w, mp, 256, 256, 64, 64, 2, b, o, s + 1, None) == -6
    val = L.usw_encode_device_values
    assert val(None, 256, 256, 64, 64, 1, b, o, None, 10, v, 4096, None) == -1
    assert val(w, 256, 256, 64, 64, 1, b, o, None, 10, None, 4096, None) == -1
    assert val(w, 256, 256, 64, 64, 2, b, o, None, 10, v, 4096, None) == -1
    assert val(w, 256, 256, 64, 64, 9, b, o, None, 10, v, 4096, None) == -3
    assert val(w, 256, 256, 128, 64, 1, b, o, None, 10, v, 4096, None) == -5
    assert val(w, 256, 256, 64, 64, 1, b, o, None, -1, v, 4096, None) == -10
    assert val(w, 256, 256, 64, 64, 1, b, o, None, 256 * 256 + 1, v, 1 << 20, None) == -10
    assert val(w, 256, 256, 64, 64, 1, b, o, None, 2049, v, 4096, None) == -10   # 2*2049 > 4096
    assert val(w, 256, 256, 64, 64, 2, b, o, s, 8193, v, 4096, None) == -10      # ceil(8193/2) > 4096
    assert val(w, 256, 256, 64, 64, 1, b, o, None, 10, v + 1, 4096, None) == -6
    assert val(w, 256, 256, 64, 64, 1, b, o, None, 10, v + 8, 4096, None) == -6


@pytest.mark.host_pointers
def test_device_union_encoder_argument_errors_return_before_launch():
    L = usw.lib()
    W = np.zeros((128, 128), np.uint16)
    m = np.zeros((128, 128), np.uint8)
    bm = np.zeros(256, np.uint64)
    off = np.zeros(16, np.uint32)
    sc = np.zeros(128, np.uint16)
    vals = np.zeros(4096, np.uint8)
    w, mp, b, o, s, v = (a.ctypes.data for a in (W, m, bm, off, sc, vals))
    idx = L.usw_union_encode_device_index
    assert idx(None, mp, 128, 128, 64, 64, 2, 2, 2, b, o, s, None) == -1
    assert idx(w, mp, 128, 128, 64, 64, 2, 2, 2, b, o, None, None) == -1
    assert idx(w, mp, 128, 120, 64, 64, 2, 2, 2, b, o, s, None) == -2
    assert idx(w, mp, 128, 128, 64, 64, 2, 2, 7, b, o, s, None) == -3
    assert idx(w, mp, 128, 128, 64, 64, 2, 2, 1, b, o, s, None) == -5         # fp16 payload
    assert idx(w, mp, 128, 128, 128, 64, 2, 2, 2, b, o, s, None) == -5        # 8192-element LT
    assert idx(w, mp, 128, 128, 64, 64, 1, 16, 2, b, o, s, None) == -5       # area rows of 4
    assert idx(w + 8, mp, 128, 128, 64, 64, 2, 2, 2, b, o, s, None) == -6
    val = L.usw_union_encode_device_values
    assert val(w, mp, 128, 128, 64, 64, 2, 2, 2, b, o, s, 10, None, 4096, None) == -1
    assert val(w, mp, 128, 128, 64, 64, 2, 2, 2, b, o, s, -1, v, 4096, None) == -10
    assert val(w, mp, 128, 128, 64, 64, 2, 2, 2, b, o, s, 8193, v, 4096, None) == -10
    assert val(w, mp, 128, 128, 64, 64, 2, 2, 2, b, o, s, 10, v + 8, 4096, None) == -6
    # 2-bit payload: four codes per byte
    assert val(w, mp, 128, 128, 64, 64, 2, 2, 3, b, o, s, 4096, v, 1023, None) == -10
    assert val(w, mp, 128, 128, 64, 64, 2, 2, 2, b, o, s, 4096, v, 2047, None) == -10
    assert val(w, mp, 128, 128, 64, 64, 2, 2, 3, b, o, s, 10, v + 8, 4096, None) == -6


@pytest.mark.host_pointers
def test_device_cbc_encoder_argument_errors_return_before_launch():
    L = usw.lib()
    W = np.zeros((256, 32), np.uint16)
    m = np.zeros((256, 32), np.uint8)
    bm = np.zeros(128, np.uint64)
    off = np.zeros(4, np.uint32)
    ci = np.zeros(32, np.uint32)
    vals = np.zeros(8192, np.uint16)
    w, mp, b, o, c, v = (a.ctypes.data for a in (W, m, bm, off, ci, vals))
    idx = L.usw_cbc_encode_device_index
    assert idx(None, mp, 256, 32, b, o, c, None) == -1
    assert idx(w, mp, 256, 32, b, o, None, None) == -1
    assert idx(w, mp, 250, 32, b, o, c, None) == -2
    assert idx(w, mp, 256, 24, b, o, c, None) == -2
    assert idx(w, mp + 8, 256, 32, b, o, c, None) == -6
    assert idx(w + 8, mp, 256, 32, b, o, c, None) == -6
    val = L.usw_cbc_encode_device_values
    assert val(w, 256, 32, b, o, c, 10, None, 16384, None) == -1
    assert val(w, 256, 32, b, o, c, -1, v, 16384, None) == -10
    assert val(w, 256, 32, b, o, c, 8193, v, 16384, None) == -10
    assert val(w, 256, 32, b, o, c, 10, v + 8, 16384, None) == -6


def test_python_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.lib()
