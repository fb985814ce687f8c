"""CPU oracle for the bitmap-encoded sparse-weight SpMM Y = W.X.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The GPU library never imports,
links or calls it, and this module imports nothing from the GPU library.

What it computes, and where each step comes from:

* The format is TCA-BME as described in the blog "SpInfer: How bitmaps make
  sparse LLMs actually fast", section "How TCA-BME addresses the indexing
  overhead": one bit per element, 64 elements (an 8x8 BitmapTile) per 64-bit
  word, 2x2 BitmapTiles form a 16x16 TCTile, TCTiles form a GroupTile; a
  Bitmap array, a Values array holding only the kept elements packed in
  GroupTile -> TCTile -> BitmapTile order, and GroupTile offsets; storage
  4(NGT+1) + 8 NBT + 2 NNZ bytes (the storage equation of that section).
* A value is found by masked popcount (same blog, section "Shared Memory
  Bitmap Decoding (SMBD)"): its index among the packed values is the number of
  set bits below its position; a clear bit means the element is zero.
* The product is the plain definition: Y[n][m] = sum_k W_sp[m][k] * X[n][k]
  with W_sp = W (elementwise) M, the static-pruning equation of "Unified
  Static-Dynamic Pruning for Efficient LLM Inference", section 2.2.  It is
  accumulated in fp64, where every fp16 x fp16 product is exact.

Readings where the pages are silent (all frozen here and listed with the
design notes): bit p of a BitmapTile word is position p of the tile taken
row-major (p = 8*row + col, least significant bit first); the 2x2
BitmapTiles of a TCTile, the TCTiles of a GroupTile and the GroupTiles of the
matrix are each taken row-major; GroupTile offsets are uint32 element counts
with offsets[0] = 0 and offsets[NGT] = NNZ; values are not padded; the mask is
authoritative (a kept exact zero sets its bit and stores its bit pattern).
These tile orders are conventions the pages do not fix ("parity unpinned" by
the pages beyond self-consistency: two independent encoders, round trip).

INT4 values (per-row symmetric, range [-8, 7], fp16 scale): for each row,
amax = max |w| over kept entries, scale = fp16(amax / 7) rounded to nearest
even (0 when amax is 0), q = clamp(round_half_even(w / scale), -8, 7) in fp64
(q = 0 when scale is 0).  Element 2i of the packed value stream is the low
nibble of byte i, element 2i+1 the high nibble (two's complement); a trailing
high nibble is 0.  Dequantised weight = q * scale, exact in fp64.

2-bit values (the W2 payload of UnionSparse's W2A4 kernel-level analysis,
read as weight-only like INT4; the pages give no rule): the same per-row rule
with b = 2, i.e. range [-2, 1] and scale = fp16(amax / (2^(b-1) - 1)) =
fp16(amax), q = clamp(round_half_even(w / scale), -2, 1).  Four codes per
byte, element 4i in bits 0-1 of byte i up to element 4i+3 in bits 6-7 (two's
complement), trailing bits 0.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

VAL_F16 = 1
VAL_I4 = 2
VAL_I2 = 3


# --------------------------------------------------------------------------
# Masked popcount (SMBD section of the SpInfer blog)
# --------------------------------------------------------------------------

def popcount(x: int) -> int:
    """Number of set bits of a non-negative Python integer."""
    return bin(int(x)).count("1")


def masked_popcount(bitmap: int, position: int) -> int:
    """Count of set bits strictly below ``position``: the value's index.

    The blog builds the mask (1 << position) - 1, ANDs it with the bitmap and
    counts the surviving bits; that count is the offset into Values.
    """
    return popcount(int(bitmap) & ((1 << int(position)) - 1))


# --------------------------------------------------------------------------
# Geometry
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Geometry:
    M: int
    K: int
    gt_m: int
    gt_k: int

    def __post_init__(self):
        if self.gt_m <= 0 or self.gt_k <= 0 or self.gt_m % 16 or self.gt_k % 16:
            raise ValueError("GroupTile sides must be positive multiples of 16 (whole TCTiles)")
        if self.M <= 0 or self.K <= 0 or self.M % self.gt_m or self.K % self.gt_k:
            raise ValueError("M and K must be positive multiples of the GroupTile sides")

    @property
    def Gr(self) -> int:
        return self.M // self.gt_m

    @property
    def Gc(self) -> int:
        return self.K // self.gt_k

    @property
    def ngt(self) -> int:
        return self.Gr * self.Gc

    @property
    def Tr(self) -> int:
        return self.gt_m // 16

    @property
    def Tc(self) -> int:
        return self.gt_k // 16

    @property
    def bt_per_gt(self) -> int:
        return self.Tr * self.Tc * 4

    @property
    def nbt(self) -> int:
        return self.M * self.K // 64


@dataclass
class Encoded:
    """Host copy of an encoded matrix (numpy arrays, exact lengths)."""
    M: int
    K: int
    gt_m: int
    gt_k: int
    val_type: int
    nnz: int
    bitmaps: np.ndarray                 # uint64 [NBT]
    offsets: np.ndarray                 # uint32 [NGT + 1]
    values: np.ndarray                  # float16 [NNZ] or uint8 [ceil(NNZ/2)]
    scales: Optional[np.ndarray] = field(default=None)   # float16 [M] (INT4 only)

    @property
    def geom(self) -> Geometry:
        return Geometry(self.M, self.K, self.gt_m, self.gt_k)


# --------------------------------------------------------------------------
# Storage accounting (TCA-BME storage equation; CR from the same blog's
# "The problem with being sparse" and SPDP section 3.1, eq. (1); CI from
# SPDP eq. (2); PMR from the UnionSparse motivation section)
# --------------------------------------------------------------------------

def storage_bytes(ngt: int, nbt: int, nnz: int, value_bytes: float = 2.0) -> float:
    """4 B per GroupTile offset (NGT + 1 of them), 8 B per BitmapTile, B_w per value."""
    return 4 * (ngt + 1) + 8 * nbt + value_bytes * nnz


def compression_ratio(M: int, K: int, stor: float) -> float:
    """Dense fp16 bytes (2 M K) over the compressed bytes."""
    return 2.0 * M * K / stor


def compute_intensity(M: int, N: int, cr: float) -> float:
    """CI = M N / (M / CR + N), up to the constant factors the pages drop."""
    return M * N / (M / cr + N)


def payload_metadata_ratio(nnz: int, ngt: int, nbt: int, value_bytes: float = 2.0) -> float:
    """Payload bytes B_w * NNZ over index metadata bytes (bitmaps + offsets)."""
    return value_bytes * nnz / (8 * nbt + 4 * (ngt + 1))


# --------------------------------------------------------------------------
# Encoders
# --------------------------------------------------------------------------

def _check_inputs(W: np.ndarray, mask: Optional[np.ndarray]):
    if W.ndim != 2:
        raise ValueError("W must be 2-D [M][K]")
    if W.dtype != np.float16:
        raise TypeError("W must be float16")
    if mask is None:
        # Without a mask an element is kept when it is nonzero in IEEE terms
        # (+0 and -0 dropped, NaN kept).
        mask = W != 0
        mask |= np.isnan(W)
    if mask.shape != W.shape:
        raise ValueError("mask shape must match W")
    return mask.astype(bool, copy=False)


def encode_loop(W: np.ndarray, mask: Optional[np.ndarray], gt_m: int = 64, gt_k: int = 64) -> Encoded:
    """Literal nested-loop encoder (small matrices only).

    GroupTiles in row-major order; inside each, TCTiles row-major; inside
    each TCTile the 2x2 BitmapTiles row-major; inside each BitmapTile the 64
    positions row-major with position p on bit p.
    """
    mask = _check_inputs(W, mask)
    g = Geometry(W.shape[0], W.shape[1], gt_m, gt_k)
    bitmaps = np.zeros(g.nbt, dtype=np.uint64)
    offsets = np.zeros(g.ngt + 1, dtype=np.uint32)
    values = []
    wbits = W.view(np.uint16)
    idx = 0
    for gid in range(g.ngt):
        gi, gj = divmod(gid, g.Gc)
        offsets[gid] = idx
        for t in range(g.Tr * g.Tc):
            ti, tj = divmod(t, g.Tc)
            for b in range(4):
                bi, bj = divmod(b, 2)
                r0 = gi * gt_m + 16 * ti + 8 * bi
                c0 = gj * gt_k + 16 * tj + 8 * bj
                bm = 0
                for p in range(64):
                    r, c = divmod(p, 8)
                    if mask[r0 + r, c0 + c]:
                        bm |= 1 << p
                        values.append(int(wbits[r0 + r, c0 + c]))
                        idx += 1
                bitmaps[gid * g.bt_per_gt + 4 * t + b] = np.uint64(bm)
    offsets[g.ngt] = idx
    vals = np.array(values, dtype=np.uint16).view(np.float16)
    return Encoded(g.M, g.K, gt_m, gt_k, VAL_F16, idx, bitmaps, offsets, vals)


def tile_order(A: np.ndarray, gt_m: int, gt_k: int) -> np.ndarray:
    """Rearrange [M][K] into [NBT][64] in storage order.

    Row index = gi*gt_m + 16*ti + 8*bi + r, column = gj*gt_k + 16*tj + 8*bj + c;
    the result is ordered (gi, gj, ti, tj, bi, bj) over BitmapTiles and
    (r, c) over the 64 positions, i.e. GroupTile -> TCTile -> BitmapTile ->
    position, all row-major.
    """
    M, K = A.shape
    Gr, Gc, Tr, Tc = M // gt_m, K // gt_k, gt_m // 16, gt_k // 16
    t = A.reshape(Gr, Tr, 2, 8, Gc, Tc, 2, 8)
    return t.transpose(0, 4, 1, 5, 2, 6, 3, 7).reshape(-1, 64)


def untile_order(T: np.ndarray, M: int, K: int, gt_m: int, gt_k: int) -> np.ndarray:
    """Inverse of :func:`tile_order`."""
    Gr, Gc, Tr, Tc = M // gt_m, K // gt_k, gt_m // 16, gt_k // 16
    t = T.reshape(Gr, Gc, Tr, Tc, 2, 2, 8, 8)
    return t.transpose(0, 2, 4, 6, 1, 3, 5, 7).reshape(M, K)


def _bitmaps_from_bits(bits: np.ndarray) -> np.ndarray:
    """[NBT][64] bool -> uint64 words with position p on bit p (LSB first)."""
    packed = np.packbits(bits, axis=1, bitorder="little")        # 8 bytes per row
    return packed.reshape(-1).view("<u8").astype(np.uint64)


def _bits_from_bitmaps(bitmaps: np.ndarray) -> np.ndarray:
    return np.unpackbits(bitmaps.astype("<u8").view(np.uint8).reshape(-1, 8), axis=1,
                         bitorder="little").astype(bool)


def encode(W: np.ndarray, mask: Optional[np.ndarray], gt_m: int = 64, gt_k: int = 64) -> Encoded:
    """Vectorised encoder, same definition as :func:`encode_loop`."""
    mask = _check_inputs(W, mask)
    g = Geometry(W.shape[0], W.shape[1], gt_m, gt_k)
    bits = tile_order(mask, gt_m, gt_k)
    vals = tile_order(W, gt_m, gt_k)[bits]
    per_gt = bits.reshape(g.ngt, -1).sum(axis=1, dtype=np.int64)
    offsets = np.zeros(g.ngt + 1, dtype=np.int64)
    np.cumsum(per_gt, out=offsets[1:])
    nnz = int(offsets[-1])
    if nnz >= 2 ** 32:
        raise ValueError("NNZ does not fit the 32-bit offsets")
    return Encoded(g.M, g.K, gt_m, gt_k, VAL_F16, nnz, _bitmaps_from_bits(bits),
                   offsets.astype(np.uint32), np.ascontiguousarray(vals))


# --------------------------------------------------------------------------
# Decoders
# --------------------------------------------------------------------------

def check_offsets(enc: Encoded) -> None:
    """Offsets invariants: start at 0, non-decreasing, end at NNZ, and each
    GroupTile's span equals the popcount of its bitmaps."""
    g = enc.geom
    off = enc.offsets.astype(np.int64)
    if off.shape != (g.ngt + 1,):
        raise ValueError("offsets must have NGT + 1 entries")
    if off[0] != 0 or off[-1] != enc.nnz:
        raise ValueError("offsets must start at 0 and end at NNZ")
    if np.any(np.diff(off) < 0):
        raise ValueError("offsets must be non-decreasing")
    counts = _bits_from_bitmaps(enc.bitmaps).reshape(g.ngt, -1).sum(axis=1)
    if not np.array_equal(counts, np.diff(off)):
        raise ValueError("GroupTile offsets disagree with bitmap popcounts")


def decode_loop(enc: Encoded) -> np.ndarray:
    """Dense fp16 [M][K] from an fp16 encoding, by per-position masked popcount.

    Each BitmapTile's first value sits at its GroupTile's offset plus the
    popcounts of the earlier BitmapTiles of that GroupTile; position p then
    reads Values[base + masked_popcount(bitmap, p)] when its bit is set.
    """
    g = enc.geom
    out = np.zeros((g.M, g.K), dtype=np.uint16)
    vbits = enc.values.view(np.uint16)
    for gid in range(g.ngt):
        gi, gj = divmod(gid, g.Gc)
        base = int(enc.offsets[gid])
        for t in range(g.Tr * g.Tc):
            ti, tj = divmod(t, g.Tc)
            for b in range(4):
                bi, bj = divmod(b, 2)
                bm = int(enc.bitmaps[gid * g.bt_per_gt + 4 * t + b])
                r0 = gi * g.gt_m + 16 * ti + 8 * bi
                c0 = gj * g.gt_k + 16 * tj + 8 * bj
                for p in range(64):
                    if (bm >> p) & 1:
                        r, c = divmod(p, 8)
                        out[r0 + r, c0 + c] = vbits[base + masked_popcount(bm, p)]
                base += popcount(bm)
        if base != int(enc.offsets[gid + 1]):
            raise ValueError(f"GroupTile {gid}: bitmap popcount disagrees with offsets")
    return out.view(np.float16)


def decode(enc: Encoded) -> np.ndarray:
    """Vectorised fp16 decoder (scatter the packed values onto the set bits)."""
    check_offsets(enc)
    g = enc.geom
    bits = _bits_from_bitmaps(enc.bitmaps)
    tiles = np.zeros(bits.shape, dtype=np.float16)
    tiles[bits] = enc.values
    return untile_order(tiles, g.M, g.K, g.gt_m, g.gt_k)


# --------------------------------------------------------------------------
# INT4 values
# --------------------------------------------------------------------------

def fp16_rne(x) -> np.ndarray:
    """fp64 -> fp16, round to nearest even (numpy's direct conversion)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def quantize_rows_int(W: np.ndarray, mask: np.ndarray, bits: int):
    """Per-row symmetric b-bit quantisation over the kept entries: scale =
    fp16(amax / (2^(b-1) - 1)), q = clamp(rint(w / scale), -2^(b-1),
    2^(b-1) - 1) in fp64.

    Returns (scales fp16 [M], q int8 [M][K]) with q = 0 outside the mask.
    """
    qmax = (1 << (bits - 1)) - 1
    Wd = W.astype(np.float64)
    absk = np.where(mask, np.abs(Wd), 0.0)
    amax = absk.max(axis=1) if W.shape[1] else np.zeros(W.shape[0])
    scales = fp16_rne(amax / float(qmax))
    s64 = scales.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(Wd / s64[:, None])
    # Zero scale (nothing but zeros kept), NaN scale (a kept NaN makes the
    # row maximum NaN) and a NaN quotient (inf / inf) all give code 0.
    q = np.where((s64[:, None] > 0) & ~np.isnan(q), q, 0.0)
    q = np.clip(q, -qmax - 1, qmax)
    q = np.where(mask, q, 0.0).astype(np.int8)
    return scales, q


def quantize_rows_i4(W: np.ndarray, mask: np.ndarray):
    """Per-row symmetric INT4 quantisation over the kept entries (b = 4:
    scale amax / 7, codes in [-8, 7])."""
    return quantize_rows_int(W, mask, 4)


def quantize_rows_i2(W: np.ndarray, mask: np.ndarray):
    """Per-row symmetric 2-bit quantisation over the kept entries (b = 2:
    scale amax / 1, codes in [-2, 1])."""
    return quantize_rows_int(W, mask, 2)


def pack_crumbs(q: np.ndarray) -> np.ndarray:
    """Two's-complement 2-bit codes, element 4i + j in bits 2j, 2j+1 of byte i."""
    u = (q.astype(np.int16) & 0x3).astype(np.uint8)
    pad = (-u.size) % 4
    if pad:
        u = np.concatenate([u, np.zeros(pad, dtype=np.uint8)])
    u = u.reshape(-1, 4)
    return (u[:, 0] | (u[:, 1] << 2) | (u[:, 2] << 4) | (u[:, 3] << 6)).astype(np.uint8)


def unpack_crumbs(packed: np.ndarray, n: int) -> np.ndarray:
    u = np.empty(4 * packed.size, dtype=np.int8)
    for j in range(4):
        u[j::4] = ((packed >> (2 * j)) & 0x3).astype(np.int8)
    u = u[:n]
    return np.where(u >= 2, u - 4, u).astype(np.int8)


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, element 2i low and 2i+1 high in byte i."""
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    if u.size % 2:
        u = np.concatenate([u, np.zeros(1, dtype=np.uint8)])
    return (u[0::2] | (u[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray, n: int) -> np.ndarray:
    lo = (packed & 0xF).astype(np.int8)
    hi = (packed >> 4).astype(np.int8)
    u = np.empty(2 * packed.size, dtype=np.int8)
    u[0::2] = lo
    u[1::2] = hi
    u = u[:n]
    return np.where(u >= 8, u - 16, u).astype(np.int8)


def encode_i4(W: np.ndarray, mask: Optional[np.ndarray], gt_m: int = 64, gt_k: int = 64) -> Encoded:
    """INT4 encoding: quantise per row, then the same bitmaps/offsets/order."""
    mask = _check_inputs(W, mask)
    scales, q = quantize_rows_i4(W, mask)
    g = Geometry(W.shape[0], W.shape[1], gt_m, gt_k)
    bits = tile_order(mask, gt_m, gt_k)
    qseq = tile_order(q, gt_m, gt_k)[bits]
    per_gt = bits.reshape(g.ngt, -1).sum(axis=1, dtype=np.int64)
    offsets = np.zeros(g.ngt + 1, dtype=np.int64)
    np.cumsum(per_gt, out=offsets[1:])
    nnz = int(offsets[-1])
    return Encoded(g.M, g.K, gt_m, gt_k, VAL_I4, nnz, _bitmaps_from_bits(bits),
                   offsets.astype(np.uint32), pack_nibbles(qseq), scales)


def decode_i4(enc: Encoded):
    """(q int8 [M][K], W_deq fp64 [M][K]) from an INT4 encoding."""
    check_offsets(enc)
    g = enc.geom
    bits = _bits_from_bitmaps(enc.bitmaps)
    tiles = np.zeros(bits.shape, dtype=np.int8)
    tiles[bits] = unpack_nibbles(enc.values, enc.nnz)
    q = untile_order(tiles, g.M, g.K, g.gt_m, g.gt_k)
    return q, q.astype(np.float64) * enc.scales.astype(np.float64)[:, None]


def dense_weight(enc: Encoded) -> np.ndarray:
    """fp64 dense weight the encoding stands for."""
    if enc.val_type == VAL_F16:
        return decode(enc).astype(np.float64)
    return decode_i4(enc)[1]


# --------------------------------------------------------------------------
# The product and the acceptance test
# --------------------------------------------------------------------------

def spmm_fp64(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Y [N][M] = X [N][K] times W^T, all in fp64 (fp16 products are exact)."""
    return np.asarray(X, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T


def abs_bound(W: np.ndarray, X: np.ndarray) -> np.ndarray:
    """Bnd[n][m] = sum_k |W[m][k]| |X[n][k]|, the scale of rounding error."""
    return np.abs(np.asarray(X, dtype=np.float64)) @ np.abs(np.asarray(W, dtype=np.float64)).T


def spmm(enc: Encoded, X: np.ndarray) -> np.ndarray:
    """Decode, then the fp64 product."""
    return spmm_fp64(dense_weight(enc), X)


REL_L2_TOL = 1e-3
ABS_BOUND_FACTOR = 2e-3


def compare(Y: np.ndarray, Yref: np.ndarray, Bnd: np.ndarray):
    """Acceptance test for an fp32-accumulated result against the fp64 oracle.

    Passes when ||Y - Yref||_2 <= 1e-3 ||Yref||_2 (Y exactly zero when Yref is)
    and |Y - Yref| <= 2e-3 * Bnd elementwise.  Returns (ok, rel_l2, worst) with
    worst = max |Y - Yref| / (2e-3 * Bnd) over entries with Bnd > 0.
    """
    Y = np.asarray(Y, dtype=np.float64)
    Yref = np.asarray(Yref, dtype=np.float64)
    if Y.shape != Yref.shape:
        return False, float("inf"), float("inf")
    if not np.all(np.isfinite(Y)):
        return False, float("inf"), float("inf")
    err = np.abs(Y - Yref)
    nref = float(np.linalg.norm(Yref))
    rel = float(np.linalg.norm(Y - Yref)) / nref if nref > 0 else (0.0 if not err.any() else float("inf"))
    lim = ABS_BOUND_FACTOR * Bnd
    ok_elem = bool(np.all(err <= lim))
    pos = lim > 0
    worst = float(np.max(err[pos] / lim[pos])) if pos.any() else 0.0
    ok = ok_elem and rel <= REL_L2_TOL
    return ok, rel, worst
