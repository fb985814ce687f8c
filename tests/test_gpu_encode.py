"""GPU parity of the on-device encoders, called through the C ABI: TCA-BME
(usw_encode_device_index / _values), IE-BME union-mask INT4
(usw_union_encode_device_*) and Tiled-CBC (usw_cbc_encode_device_*).  Every
buffer must equal the CPU oracle's encoding, and the host encoder's, byte
for byte."""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import tca_bme as ob

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)

import unstructured_sparse_weight_amd as usw  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev_encode(W, mask, gt=(64, 64), dtype="f16"):
    Wt = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    mt = torch.from_numpy(np.ascontiguousarray(mask)).to(DEV) if mask is not None else None
    enc = usw.encode_device(Wt, mt, gt, dtype)
    torch.cuda.synchronize()
    return enc


def host_arrays(enc):
    """The device encoding's buffers as host numpy arrays."""
    sc = enc.scales.cpu().numpy().view(np.uint16) if enc.scales is not None else None
    return (enc.bitmaps.cpu().numpy().view(np.uint64), enc.offsets.cpu().numpy().view(np.uint32),
            enc.values.cpu().numpy(), sc)


def assert_matches_oracle(enc, o):
    bm, off, vals, sc = host_arrays(enc)
    assert enc.nnz == o.nnz
    assert np.array_equal(bm, o.bitmaps)
    assert np.array_equal(off, o.offsets)
    vb = o.values.view(np.uint8).reshape(-1)
    assert vals.size % 16 == 0 and vals.size >= max(16, vb.size)
    assert np.array_equal(vals[: vb.size], vb)
    assert not vals[vb.size:].any()
    if o.scales is not None:
        assert np.array_equal(sc, o.scales.view(np.uint16))


def assert_matches_host(enc, h):
    bm, off, vals, sc = host_arrays(enc)
    assert enc.nnz == h.nnz
    assert np.array_equal(bm, h.bitmaps)
    assert np.array_equal(off, h.offsets)
    assert np.array_equal(vals, h.values)
    if h.scales is not None:
        assert np.array_equal(sc, h.scales)


@pytest.mark.parametrize("gt", [(64, 64), (32, 64), (16, 16), (64, 32), (16, 64)])
@pytest.mark.parametrize("density", [0.0, 0.03, 0.5, 1.0])
@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_device_encoder_matches_oracle(gt, density, dtype):
    rng = np.random.default_rng(int(density * 100) + gt[0] + 7 * gt[1] + (dtype == "i4"))
    M, K = 128, 192
    W = wl.weight_normal(M, K, rng)
    W[rng.random((M, K)) < 0.05] = np.float16(0.0)
    W[rng.random((M, K)) < 0.05] = np.float16(-0.0)
    mask = wl.mask_bernoulli(M, K, density, rng)
    say(f"[encode] gt={gt} density={density} dtype={dtype}")
    enc = dev_encode(W, mask, gt, dtype)
    o = (ob.encode if dtype == "f16" else ob.encode_i4)(W, mask, *gt)
    assert_matches_oracle(enc, o)


@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_null_mask_keeps_ieee_nonzeros(dtype):
    """No mask: +0 and -0 dropped, NaN and infinities kept (NaN is skipped by
    the INT4 row maximum; an infinite row maximum gives an infinite scale)."""
    rng = np.random.default_rng(4)
    W = wl.weight_normal(64, 128, rng)
    W[rng.random(W.shape) < 0.4] = np.float16(0.0)
    W[0, 0] = np.float16(-0.0)
    W[0, 1] = np.float16(np.nan)
    W[1, 5] = np.float16(np.inf)
    W[2, 7] = np.float16(-np.inf)
    W[3, 9] = np.float16(np.nan)
    say(f"[encode] null mask dtype={dtype}")
    enc = dev_encode(W, None, (64, 64), dtype)
    o = (ob.encode if dtype == "f16" else ob.encode_i4)(W, None)
    assert_matches_oracle(enc, o)
    assert_matches_host(enc, usw.encode_host(W, None, (64, 64), dtype))


@pytest.mark.parametrize("dtype", ["f16", "i4"])
def test_kept_zeros_are_stored(dtype):
    """The mask is authoritative: a kept +0 or -0 sets its bit and is stored."""
    rng = np.random.default_rng(5)
    W = wl.weight_normal(64, 64, rng)
    W[::3, ::5] = np.float16(0.0)
    W[1::3, ::7] = np.float16(-0.0)
    W[10, :] = np.float16(0.0)          # a row that keeps only zeros: scale 0, codes 0
    mask = np.ones((64, 64), bool)
    say(f"[encode] kept zeros dtype={dtype}")
    enc = dev_encode(W, mask, (64, 64), dtype)
    o = (ob.encode if dtype == "f16" else ob.encode_i4)(W, mask)
    assert_matches_oracle(enc, o)


def test_int4_scale_rounding_and_ties():
    """Row scales across the fp16 subnormal range and at exact midpoints,
    and codes at exact .5 quotients (round half to even)."""
    rng = np.random.default_rng(8)
    M, K = 320, 16
    W = np.zeros((M, K), dtype=np.float16)
    amax = np.concatenate([
        rng.uniform(1e-7, 1e-4, 64),
        rng.uniform(0.01, 60000.0, 64),
        np.float16(np.arange(1, 65)) * np.float16(2.0 ** -14),
        (np.arange(64) + 0.5) * 7 * 2.0 ** -24,
        np.full(64, 7.0),                              # scale exactly 1
    ])
    W[:, 0] = amax.astype(np.float16)
    W[:, 1] = -W[:, 0] / np.float16(3)
    W[256:, 2:12] = np.float16([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, -3.5, 6.5, -7.5])
    mask = np.zeros((M, K), bool)
    mask[:, :2] = True
    mask[256:, 2:12] = True
    say("[encode] int4 scale rounding")
    enc = dev_encode(W, mask, (16, 16), "i4")
    o = ob.encode_i4(W, mask, 16, 16)
    assert_matches_oracle(enc, o)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_int4_odd_runs_across_empty_group_tiles(seed):
    """GroupTiles with odd kept counts separated by empty ones: a packed byte
    whose high nibble is the first code of the next non-empty GroupTile."""
    rng = np.random.default_rng(100 + seed)
    M, K = 256, 256
    W = wl.weight_normal(M, K, rng)
    mask = np.zeros((M, K), bool)
    for gi in range(M // 16):
        for gj in range(K // 16):
            c = rng.choice([0, 0, 0, 1, 3, 5, 255, 256])
            pos = rng.choice(256, size=c, replace=False)
            mask[gi * 16 + pos // 16, gj * 16 + pos % 16] = True
    say(f"[encode] odd runs seed={seed}")
    enc = dev_encode(W, mask, (16, 16), "i4")
    o = ob.encode_i4(W, mask, 16, 16)
    off = o.offsets.astype(np.int64)
    ends = off[1:-1]
    assert ((ends % 2 == 1) & (off[2:] == ends) & (ends < o.nnz)).any()   # the case is exercised
    assert_matches_oracle(enc, o)


def test_all_pruned_gives_empty_values():
    rng = np.random.default_rng(9)
    W = wl.weight_normal(128, 128, rng)
    mask = np.zeros((128, 128), bool)
    for dtype in ("f16", "i4"):
        enc = dev_encode(W, mask, (64, 64), dtype)
        assert enc.nnz == 0
        assert_matches_oracle(enc, (ob.encode if dtype == "f16" else ob.encode_i4)(W, mask))


def test_values_writes_stay_below_logical_size():
    """usw_encode_device_values with an nnz smaller than offsets[NGT]: the
    kernel writes nothing at or past the logical size of that nnz."""
    import ctypes
    rng = np.random.default_rng(10)
    W = wl.weight_normal(128, 128, rng)
    mask = wl.mask_bernoulli(128, 128, 0.5, rng)
    enc = dev_encode(W, mask, (64, 64), "f16")
    small = enc.nnz // 3
    buf = torch.full((4 * enc.nnz + 64,), 0xAB, dtype=torch.uint8, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    Wt = torch.from_numpy(W).to(DEV)
    usw.check(usw.lib().usw_encode_device_values(Wt.data_ptr(), 128, 128, 64, 64, usw.USW_VAL_F16,
                                                 enc.bitmaps.data_ptr(), enc.offsets.data_ptr(), None, small,
                                                 buf.data_ptr(), 2 * small, st), "usw_encode_device_values")
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    full = enc.values.cpu().numpy()
    assert np.array_equal(b[: 2 * small], full[: 2 * small])
    assert (b[2 * small:] == 0xAB).all()


def test_device_encoding_runs_spmm_like_host_encoding():
    W, mask, X = wl.config_case(1, 256, 256, 8, 0.5)
    ed = dev_encode(W, mask)
    eh = usw.encode(W, mask, device=DEV)
    x = torch.from_numpy(X).to(DEV)
    yd = usw.spmm(ed, x)
    yh = usw.spmm(eh, x)
    torch.cuda.synchronize()
    assert torch.equal(yd, yh)


@pytest.mark.parametrize("case", ["ffn_up_f16", "ffn_up_i4", "attn_out_null_mask"])
def test_full_size_matches_host_encoder(case):
    """FFN-up 20480 x 5120 (fp16 at 70% sparsity, INT4 at 50%) and
    attention-output 5120 x 5120 without a mask: byte-identical to the host
    encoder (itself pinned to the oracle on these shapes)."""
    if case == "ffn_up_f16":
        W, mask, _ = wl.config_case(3, 20480, 5120, 16, 0.3, layer_id=3)
        dtype = "f16"
    elif case == "ffn_up_i4":
        W, mask, _ = wl.config_case(5, 20480, 5120, 2, 0.5)
        dtype = "i4"
    else:
        W, mask, _ = wl.config_case(2, 5120, 5120, 16, 0.5, layer_id=1)
        W = np.where(mask, W, np.float16(0.0)).astype(np.float16)
        mask = None
        dtype = "f16"
    say(f"[encode] full size {case}")
    enc = dev_encode(W, mask, (64, 64), dtype)
    assert_matches_host(enc, usw.encode_host(W, mask, (64, 64), dtype))


# ---------------------------------------------------------------------------
# IE-BME union-mask encoder on the device (usw_union_encode_device_*)
# ---------------------------------------------------------------------------

from oracle import ie_bme as ou  # noqa: E402


def dev_union_encode(W, mask, lt=(64, 64), areas=(2, 2), dtype="i4"):
    Wt = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    mt = torch.from_numpy(np.ascontiguousarray(mask)).to(DEV) if mask is not None else None
    enc = usw.union_encode_device(Wt, mt, lt, areas, dtype)
    torch.cuda.synchronize()
    return enc


def assert_union_matches_oracle(enc, o):
    assert enc.payload == o.payload
    assert np.array_equal(enc.bitmaps.cpu().numpy().view(np.uint64)[: o.bitmaps.size], o.bitmaps)
    assert np.array_equal(enc.offsets.cpu().numpy().view(np.uint32), o.offsets)
    vals = enc.values.cpu().numpy()
    vb = o.values.view(np.uint8).reshape(-1)
    assert vals.size % 16 == 0 and vals.size >= max(16, vb.size)
    assert np.array_equal(vals[: vb.size], vb)
    assert not vals[vb.size:].any()
    assert np.array_equal(enc.scales.cpu().numpy().view(np.uint16), o.scales.view(np.uint16))


@pytest.mark.parametrize("lt,areas", [((64, 64), (2, 2)), ((32, 64), (2, 2)), ((64, 64), (1, 1)),
                                      ((16, 64), (2, 2)), ((64, 32), (2, 1)), ((64, 64), (4, 2))])
@pytest.mark.parametrize("density", [0.0, 0.05, 0.5, 1.0])
@pytest.mark.parametrize("dtype", ["i4", "i2"])
def test_device_union_encoder_matches_oracle(lt, areas, density, dtype):
    rng = np.random.default_rng(int(density * 100) + lt[0] + 3 * lt[1] + 11 * areas[0] + areas[1])
    M, K = 128, 256
    W = wl.weight_normal(M, K, rng)
    W[rng.random((M, K)) < 0.05] = np.float16(0.0)
    mask = wl.mask_bernoulli(M, K, density, rng)
    say(f"[union encode] lt={lt} areas={areas} density={density} {dtype}")
    enc = dev_union_encode(W, mask, lt, areas, dtype)
    vt = ob.VAL_I4 if dtype == "i4" else ob.VAL_I2
    assert_union_matches_oracle(enc, ou.encode_union(W, mask, lt[0], lt[1], areas[0], areas[1], vt))


def test_device_union_null_mask_and_non_finite():
    rng = np.random.default_rng(21)
    W = wl.weight_normal(128, 128, rng)
    W[rng.random(W.shape) < 0.6] = np.float16(0.0)
    W[0, 1] = np.float16(np.nan)
    W[5, 9] = np.float16(np.inf)
    W[70, 3] = np.float16(-0.0)
    say("[union encode] null mask, NaN/Inf")
    enc = dev_union_encode(W, None)
    assert_union_matches_oracle(enc, ou.encode_union(W, None, 64, 64, 2, 2, ob.VAL_I4))


@pytest.mark.parametrize("seed", [0, 1])
def test_device_union_odd_runs_across_empty_lts(seed):
    """LTs whose payload ends on an odd code next to empty LTs, and active
    groups whose area-0 weight is pruned (a first code of 0)."""
    rng = np.random.default_rng(300 + seed)
    M, K = 256, 256
    W = wl.weight_normal(M, K, rng)
    mask = np.zeros((M, K), bool)
    for ti in range(M // 16):
        for tj in range(K // 64):
            c = rng.choice([0, 0, 1, 3, 7])
            pos = rng.choice(16 * 64, size=c, replace=False)
            mask[ti * 16 + pos // 64, tj * 64 + pos % 64] = True
    say(f"[union encode] odd runs seed={seed}")
    enc = dev_union_encode(W, mask, (16, 64), (1, 1))
    o = ou.encode_union(W, mask, 16, 64, 1, 1, ob.VAL_I4)
    off = o.offsets.astype(np.int64)
    ends = off[1:-1]
    assert ((ends % 2 == 1) & (off[2:] == ends) & (ends < o.payload)).any()
    assert_union_matches_oracle(enc, o)
    enc2 = dev_union_encode(W, mask, (16, 64), (2, 2))        # Q = 4: runs of even length
    assert_union_matches_oracle(enc2, ou.encode_union(W, mask, 16, 64, 2, 2, ob.VAL_I4))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_device_union_2bit_runs_across_empty_lts(seed):
    """2-bit payload: four codes per byte, so a byte can hold the end of one
    LT's run and the first codes of up to three following LTs (runs of one
    to three codes next to empty LTs, Q = 1), and active groups whose
    weight is pruned."""
    rng = np.random.default_rng(400 + seed)
    M, K = 256, 512
    W = wl.weight_normal(M, K, rng)
    mask = np.zeros((M, K), bool)
    for ti in range(M // 16):
        for tj in range(K // 64):
            c = rng.choice([0, 0, 1, 1, 2, 3, 5])
            pos = rng.choice(16 * 64, size=c, replace=False)
            mask[ti * 16 + pos // 64, tj * 64 + pos % 64] = True
    say(f"[union encode] 2-bit short runs seed={seed}")
    o = ou.encode_union(W, mask, 16, 64, 1, 1, ob.VAL_I2)
    off = o.offsets.astype(np.int64)
    runs = np.diff(off)
    assert ((runs > 0) & (runs < 4) & (off[1:] % 4 != 0)).any()       # bytes shared across LTs
    assert_union_matches_oracle(dev_union_encode(W, mask, (16, 64), (1, 1), "i2"), o)
    # Q = 2 and Q = 8 grids: runs of even lengths and multiples of 8
    for areas in [(2, 1), (4, 2)]:
        assert_union_matches_oracle(dev_union_encode(W, mask, (16, 64), areas, "i2"),
                                    ou.encode_union(W, mask, 16, 64, areas[0], areas[1], ob.VAL_I2))


def test_device_union_full_size_2bit_matches_host_and_runs_spmm():
    """FFN-up 20480 x 5120 with a 2-bit payload at 50%: byte-identical to
    the host union encoder, and both encodings give the same product bits."""
    W, mask, X = wl.config_case(5, 20480, 5120, 2, 0.5)
    say("[union encode] full size FFN-up, 2-bit")
    enc = dev_union_encode(W, mask, (64, 64), (2, 2), "i2")
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i2")
    assert enc.payload == h.payload
    assert np.array_equal(enc.bitmaps.cpu().numpy().view(np.uint64), h.bitmaps)
    assert np.array_equal(enc.offsets.cpu().numpy().view(np.uint32), h.offsets)
    assert np.array_equal(enc.values.cpu().numpy(), h.values)
    assert np.array_equal(enc.scales.cpu().numpy().view(np.uint16), h.scales)
    x = torch.from_numpy(X).to(DEV)
    yd = usw.union_spmm(enc, x)
    yh = usw.union_spmm(usw.union_to_device(h, DEV), x)
    torch.cuda.synchronize()
    assert torch.equal(yd, yh)


def test_device_union_full_size_matches_host_and_runs_spmm():
    """FFN-up 20480 x 5120 INT4 at 50%: byte-identical to the host union
    encoder, and the union SpMM of both encodings gives the same bits."""
    W, mask, X = wl.config_case(5, 20480, 5120, 2, 0.5)
    say("[union encode] full size FFN-up")
    enc = dev_union_encode(W, mask)
    h = usw.union_encode_host(W, mask, (64, 64), (2, 2), "i4")
    assert enc.payload == h.payload
    assert np.array_equal(enc.bitmaps.cpu().numpy().view(np.uint64), h.bitmaps)
    assert np.array_equal(enc.offsets.cpu().numpy().view(np.uint32), h.offsets)
    assert np.array_equal(enc.values.cpu().numpy(), h.values)
    assert np.array_equal(enc.scales.cpu().numpy().view(np.uint16), h.scales)
    x = torch.from_numpy(X).to(DEV)
    yd = usw.union_spmm(enc, x)
    yh = usw.union_spmm(usw.union_to_device(h, DEV), x)
    torch.cuda.synchronize()
    assert torch.equal(yd, yh)


def test_device_encoder_replays_from_a_hip_graph():
    """Both TCA-BME device-encoder calls launch kernels only (no allocation,
    no memset), so they can be captured: three replays, with eager work and
    synchronisation in between, each give the eager encoding's bytes."""
    import ctypes
    W, mask, _ = wl.config_case(1, 256, 256, 8, 0.5)
    Wt = torch.from_numpy(W).to(DEV)
    mt = torch.from_numpy(mask.view(np.uint8)).to(DEV)
    ref = usw.encode_device(Wt, mt, (64, 64), "i4")
    torch.cuda.synchronize()
    bm = torch.zeros_like(ref.bitmaps)
    off = torch.zeros_like(ref.offsets)
    sc = torch.zeros_like(ref.scales)
    vals = torch.zeros_like(ref.values)
    L = usw.lib()
    cap = torch.cuda.Stream(DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        sp = ctypes.c_void_p(cap.cuda_stream)
        assert L.usw_encode_device_index(Wt.data_ptr(), mt.data_ptr(), 256, 256, 64, 64, usw.USW_VAL_I4,
                                         bm.data_ptr(), off.data_ptr(), sc.data_ptr(), sp) == 0
        assert L.usw_encode_device_values(Wt.data_ptr(), 256, 256, 64, 64, usw.USW_VAL_I4, bm.data_ptr(),
                                          off.data_ptr(), sc.data_ptr(), ref.nnz, vals.data_ptr(), vals.numel(),
                                          sp) == 0
    for i in range(3):
        for tns in (bm, off, sc):
            tns.fill_(-1)
        vals.fill_(0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        say(f"[encode] graph replay {i}")
        assert torch.equal(bm, ref.bitmaps) and torch.equal(off, ref.offsets)
        assert torch.equal(sc, ref.scales) and torch.equal(vals, ref.values)


# ---------------------------------------------------------------------------
# Tiled-CBC encoder on the device (usw_cbc_encode_device_*)
# ---------------------------------------------------------------------------

from oracle import tiled_cbc as oc  # noqa: E402


def assert_cbc_matches_oracle(enc, o):
    assert enc.nnz == o.nnz and enc.nnz_padded == o.nnz_padded
    assert np.array_equal(enc.bitmaps.cpu().numpy().view(np.uint64)[: o.bitmaps.size], o.bitmaps)
    assert np.array_equal(enc.tile_offsets.cpu().numpy().view(np.uint32), o.tile_offsets)
    assert np.array_equal(enc.colinfo.cpu().numpy().view(np.uint32)[: o.colinfo.size], o.colinfo)
    vals = enc.values.cpu().numpy().view(np.uint16)
    assert np.array_equal(vals[: o.nnz_padded], o.values.view(np.uint16)[: o.nnz_padded])
    assert not vals[o.nnz_padded:].any()


def dev_cbc_encode(W, mask):
    Wt = torch.from_numpy(np.ascontiguousarray(W)).to(DEV)
    mt = torch.from_numpy(np.ascontiguousarray(mask)).to(DEV) if mask is not None else None
    enc = usw.cbc_encode_device(Wt, mt)
    torch.cuda.synchronize()
    return enc


@pytest.mark.parametrize("shape", [(256, 16), (512, 64), (768, 96)])
@pytest.mark.parametrize("density", [0.0, 0.03, 0.5, 1.0])
def test_device_cbc_encoder_matches_oracle(shape, density):
    rng = np.random.default_rng(int(density * 100) + shape[0] + shape[1])
    W = wl.weight_normal(*shape, rng)
    W[rng.random(shape) < 0.05] = np.float16(-0.0)
    mask = wl.mask_bernoulli(*shape, density, rng)
    say(f"[cbc encode] shape={shape} density={density}")
    assert_cbc_matches_oracle(dev_cbc_encode(W, mask), oc.encode_cbc(W, mask))


def test_device_cbc_null_mask_and_full_size():
    rng = np.random.default_rng(31)
    W = wl.weight_normal(512, 128, rng)
    W[rng.random(W.shape) < 0.5] = np.float16(0.0)
    W[3, 4] = np.float16(np.nan)
    say("[cbc encode] null mask")
    assert_cbc_matches_oracle(dev_cbc_encode(W, None), oc.encode_cbc(W, None))
    W, mask, X = wl.config_case(2, 20480, 5120, 1, 0.5, layer_id=2)
    say("[cbc encode] full size FFN-up")
    enc = dev_cbc_encode(W, mask)
    h = usw.cbc_encode_host(W, mask)
    assert enc.nnz == h.nnz and enc.nnz_padded == h.nnz_padded
    for a, b in ((enc.bitmaps, h.bitmaps), (enc.tile_offsets, h.tile_offsets), (enc.colinfo, h.colinfo)):
        assert np.array_equal(a.cpu().numpy().view(b.dtype), b)
    assert np.array_equal(enc.values.cpu().numpy().view(np.uint16)[: h.values.size], h.values)
    x = torch.from_numpy(X[0]).to(DEV)
    yd = usw.cbc_spmspv(enc, x, 0.5)
    yh = usw.cbc_spmspv(usw.cbc_to_device(h, DEV), x, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(yd, yh)
