"""CPU oracle for the IE-BME union-mask low-bit format and its SpMM.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The GPU library never imports,
links or calls it, and this module imports nothing from the GPU library.

What it computes, and where each step comes from ("UnionSparse: An
Index-Efficient Sparsity Framework for Low-Bit Sparse LLM Inference on Edge",
section on IE-BME and section on LSPD):

* Area partitioning.  A local tile (LT) W_t of H_L x K_L weights is cut into
  an R_A x C_A grid of areas of (H_L/R_A) x (K_L/C_A) each, Q = R_A C_A.
  Position (i, j) of every area together forms one logical grouped position.
* Shared union mask.  B_t(i, j) is 1 when at least one of the Q values of the
  group is kept, so one bit describes Q payload values.
* Storage.  Union Bitmaps: B_t scanned row-major, packed into 64-bit words,
  least significant bit first (the section's Fig. 7 shows the leftmost bit of
  a displayed row as the LSB), words of all LTs concatenated.  Union Value
  Offsets: o_t is the prefix sum of Q P_t over the preceding LTs, P_t the
  number of set union bits of LT t.  Compressed Values: an active position
  gets the compact rank r = number of active positions before it in
  row-major order; the value of area q is stored at o_t + q P_t + r (the Q
  streams of an LT one after the other).  A group whose union bit is set
  stores all Q values, zeros of individual areas included; a clear bit
  stores nothing.
* LSPD.  A logical row is cut into segments of G bits; a segment's payload
  base is o_t plus the active bits before it, and its k-th active bit reads
  index base + k in every area stream.
* The product is the plain definition Y[n][m] = sum_k W_sp[m][k] X[n][k]
  accumulated in fp64 (tca_bme.spmm_fp64).

Readings where the pages are silent (frozen here and listed with the design
notes): LTs are taken row-major over the matrix; area q = a_r * C_A + a_c
(row-major over the area grid); the group of position (i, j) is
W_t[a_r H_L/R_A + i][a_c K_L/C_A + j]; offsets are uint32 payload-element
counts; the mask is authoritative for the union (a kept exact zero makes its
group active and stores its bit pattern; a pruned position of an active group
stores zero).  INT4 payload uses the per-row rule and nibble packing of
tca_bme (element 2i in the low nibble of byte i), 2-bit payload (the W2 of
the section's W2A4 kernel-level analysis) the same per-row rule with b = 2
and four codes per byte (tca_bme); activations stay fp16 (the format
concerns the weights).  H_L K_L / Q must be a multiple of 64 so that
each LT owns whole words.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Tuple

import numpy as np

from .tca_bme import (VAL_F16, VAL_I2, VAL_I4, _check_inputs, masked_popcount, pack_crumbs, pack_nibbles, popcount,
                      quantize_rows_i2, quantize_rows_i4, spmm_fp64, unpack_crumbs, unpack_nibbles)


# --------------------------------------------------------------------------
# Geometry
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class UnionGeometry:
    M: int
    K: int
    h_l: int      # LT rows
    k_l: int      # LT columns
    r_a: int      # area rows per LT
    c_a: int      # area columns per LT

    def __post_init__(self):
        if min(self.M, self.K, self.h_l, self.k_l, self.r_a, self.c_a) <= 0:
            raise ValueError("sizes must be positive")
        if self.M % self.h_l or self.K % self.k_l:
            raise ValueError("M and K must be multiples of the LT shape")
        if self.h_l % self.r_a or self.k_l % self.c_a:
            raise ValueError("the LT shape must be a multiple of the area grid")
        if (self.am * self.ak) % 64:
            raise ValueError("an LT's union mask must fill whole 64-bit words")

    @property
    def Q(self) -> int:
        return self.r_a * self.c_a

    @property
    def am(self) -> int:
        return self.h_l // self.r_a

    @property
    def ak(self) -> int:
        return self.k_l // self.c_a

    @property
    def lt_rows(self) -> int:
        return self.M // self.h_l

    @property
    def lt_cols(self) -> int:
        return self.K // self.k_l

    @property
    def nlt(self) -> int:
        return self.lt_rows * self.lt_cols

    @property
    def words_per_lt(self) -> int:
        return self.am * self.ak // 64

    @property
    def nwords(self) -> int:
        return self.nlt * self.words_per_lt


@dataclass
class UnionEncoded:
    geom: UnionGeometry
    val_type: int
    payload: int               # stored payload elements, = offsets[NLT]
    bitmaps: np.ndarray        # uint64 [NWORDS]
    offsets: np.ndarray        # uint32 [NLT + 1]
    values: np.ndarray         # F16: uint16 [payload]; I4: uint8 [ceil(payload / 2)]; I2: uint8 [ceil(payload / 4)]
    scales: Optional[np.ndarray] = None   # I4, I2: fp16 [M], per original row
    # Reordered LTs only: uint8 [NLT][H_L]; rowmap[t][r] is the stored row of
    # LT t that holds the LT's original row r.  None: rows in natural order.
    rowmap: Optional[np.ndarray] = None


def union_storage_bytes(nlt: int, nwords: int, payload: int, value_bits: int = 4) -> float:
    """Offsets (4 B per LT plus one), union words (8 B each) and payload bytes."""
    return 4.0 * (nlt + 1) + 8.0 * nwords + payload * value_bits / 8.0


# --------------------------------------------------------------------------
# Encoding
# --------------------------------------------------------------------------

def _payload_source(W: np.ndarray, mask: np.ndarray, val_type: int):
    """Per-element payload (uint16 fp16 bits or int8 q) and the scales."""
    if val_type == VAL_F16:
        return np.where(mask, W.astype(np.float16).view(np.uint16), np.uint16(0)).astype(np.uint16), None
    if val_type == VAL_I4:
        scales, q = quantize_rows_i4(W, mask)
        return q, scales
    if val_type == VAL_I2:
        scales, q = quantize_rows_i2(W, mask)
        return q, scales
    raise ValueError("unknown value type")


def _finish(g: UnionGeometry, val_type: int, bits: np.ndarray, payload_seq: np.ndarray,
            offsets: np.ndarray, scales) -> UnionEncoded:
    words = np.packbits(bits.reshape(-1, 64).astype(np.uint8), axis=1, bitorder="little")
    bitmaps = words.view("<u8").reshape(-1).astype(np.uint64)
    if val_type == VAL_F16:
        values = payload_seq.astype(np.uint16)
    elif val_type == VAL_I4:
        values = pack_nibbles(payload_seq.astype(np.int8))
    else:
        values = pack_crumbs(payload_seq.astype(np.int8))
    return UnionEncoded(g, val_type, int(offsets[-1]), bitmaps, offsets.astype(np.uint32), values, scales)


def encode_union_loop(W: np.ndarray, mask: Optional[np.ndarray], h_l: int = 64, k_l: int = 64,
                      r_a: int = 2, c_a: int = 2, val_type: int = VAL_I4) -> UnionEncoded:
    """IE-BME encoding written as the section builds it, one LT at a time.

    For each LT (row-major): form the union mask over the Q area-aligned
    groups, give every active position its compact rank, append the Q area
    streams in area order, and advance the offset by Q P_t.
    """
    mask = _check_inputs(W, mask)
    g = UnionGeometry(W.shape[0], W.shape[1], h_l, k_l, r_a, c_a)
    src, scales = _payload_source(W, mask, val_type)
    bits: List[bool] = []
    seq: List[int] = []
    offsets = [0]
    for ti in range(g.lt_rows):
        for tj in range(g.lt_cols):
            r0, c0 = ti * h_l, tj * k_l
            active: List[Tuple[int, int]] = []
            for i in range(g.am):
                for j in range(g.ak):
                    on = any(mask[r0 + ar * g.am + i, c0 + ac * g.ak + j]
                             for ar in range(r_a) for ac in range(c_a))
                    bits.append(on)
                    if on:
                        active.append((i, j))
            for q in range(g.Q):
                ar, ac = divmod(q, c_a)
                for (i, j) in active:          # rank = place in this list
                    seq.append(int(src[r0 + ar * g.am + i, c0 + ac * g.ak + j]))
            offsets.append(offsets[-1] + g.Q * len(active))
    if offsets[-1] >= 1 << 32:
        raise ValueError("payload does not fit 32-bit offsets")
    dtype = np.uint16 if val_type == VAL_F16 else np.int8
    return _finish(g, val_type, np.array(bits, dtype=bool), np.array(seq, dtype=dtype),
                   np.array(offsets, dtype=np.int64), scales)


def area_view(A: np.ndarray, g: UnionGeometry) -> np.ndarray:
    """[NLT][Q][am * ak]: each LT's areas, LT row-major, area q = a_r C_A + a_c."""
    T = A.reshape(g.lt_rows, g.r_a, g.am, g.lt_cols, g.c_a, g.ak)
    T = T.transpose(0, 3, 1, 4, 2, 5)          # ti, tj, a_r, a_c, i, j
    return T.reshape(g.nlt, g.Q, g.am * g.ak)


def area_unview(T: np.ndarray, g: UnionGeometry) -> np.ndarray:
    A = T.reshape(g.lt_rows, g.lt_cols, g.r_a, g.c_a, g.am, g.ak).transpose(0, 2, 4, 1, 3, 5)
    return A.reshape(g.M, g.K)


def encode_union(W: np.ndarray, mask: Optional[np.ndarray], h_l: int = 64, k_l: int = 64,
                 r_a: int = 2, c_a: int = 2, val_type: int = VAL_I4) -> UnionEncoded:
    """Vectorised IE-BME encoding (an independent route to the same bytes)."""
    mask = _check_inputs(W, mask)
    g = UnionGeometry(W.shape[0], W.shape[1], h_l, k_l, r_a, c_a)
    src, scales = _payload_source(W, mask, val_type)
    return _construct(g, val_type, src, mask, scales)


def _construct(g: UnionGeometry, val_type: int, src: np.ndarray, mask: np.ndarray, scales) -> UnionEncoded:
    """Union words, offsets and area streams of a payload source and mask."""
    areas_m = area_view(mask, g)
    union = areas_m.any(axis=1)                               # [NLT][am*ak]
    areas_v = area_view(src, g)                               # [NLT][Q][am*ak]
    seq = areas_v[np.broadcast_to(union[:, None, :], areas_v.shape)]   # order: LT, area, rank
    per_lt = g.Q * union.sum(axis=1, dtype=np.int64)
    offsets = np.zeros(g.nlt + 1, dtype=np.int64)
    np.cumsum(per_lt, out=offsets[1:])
    if offsets[-1] >= 1 << 32:
        raise ValueError("payload does not fit 32-bit offsets")
    return _finish(g, val_type, union.reshape(-1), seq, offsets, scales)


# --------------------------------------------------------------------------
# Reordered LTs (the section on bitmap-aware row reordering)
# --------------------------------------------------------------------------
#
# Reordering permutes the rows of each LT before compression; it changes
# neither the number nor the values of the surviving weights, only where
# their rows sit inside the LT.  So quantisation (one scale per row of W)
# happens on the original rows, and the IE-BME construction then runs on
# every LT with its rows rearranged: stored row s of LT t holds original LT
# row perms[t][s] (the order usw_union_reorder and row_reorder return).  The
# encoding keeps, per LT, the inverse map (original row -> stored row) so
# that a reader can put each row's products back where they belong.

def permute_lt_rows(A: np.ndarray, perms: np.ndarray, h_l: int, k_l: int) -> np.ndarray:
    """A with the rows of every LT rearranged: stored row s of LT t is the
    LT's original row perms[t][s]."""
    M, K = A.shape
    lc = K // k_l
    out = np.empty_like(A)
    for t in range(perms.shape[0]):
        ti, tj = divmod(t, lc)
        rows = ti * h_l + np.asarray(perms[t], dtype=np.int64)
        out[ti * h_l:(ti + 1) * h_l, tj * k_l:(tj + 1) * k_l] = A[rows, tj * k_l:(tj + 1) * k_l]
    return out


def inverse_rowmap(perms: np.ndarray, h_l: int) -> np.ndarray:
    """rowmap[t][r] = the s with perms[t][s] = r (each row a permutation)."""
    perms = np.asarray(perms, dtype=np.int64)
    rowmap = np.empty(perms.shape, dtype=np.uint8)
    for t in range(perms.shape[0]):
        if sorted(perms[t].tolist()) != list(range(h_l)):
            raise ValueError("each LT's row order must be a permutation of its rows")
        rowmap[t, perms[t]] = np.arange(h_l, dtype=np.uint8)
    return rowmap


def encode_union_reordered(W: np.ndarray, mask: Optional[np.ndarray], perms: np.ndarray, h_l: int = 16,
                           k_l: int = 64, r_a: int = 2, c_a: int = 2, val_type: int = VAL_I4) -> UnionEncoded:
    """IE-BME encoding of W after each LT's rows are rearranged by perms
    ([NLT][H_L]); INT4 scales and codes come from the original rows."""
    mask = _check_inputs(W, mask)
    g = UnionGeometry(W.shape[0], W.shape[1], h_l, k_l, r_a, c_a)
    perms = np.asarray(perms)
    if perms.shape != (g.nlt, h_l):
        raise ValueError("one row order per LT")
    if h_l > 256:
        raise ValueError("row maps hold one byte per row")
    rowmap = inverse_rowmap(perms, h_l)
    src, scales = _payload_source(W, mask, val_type)
    enc = _construct(g, val_type, permute_lt_rows(src, perms, h_l, k_l), permute_lt_rows(mask, perms, h_l, k_l),
                     scales)
    enc.rowmap = rowmap
    return enc


def _unpermute(enc: UnionEncoded, A: np.ndarray) -> np.ndarray:
    """Per-element array in stored row order -> original row order."""
    if enc.rowmap is None:
        return A
    g = enc.geom
    out = np.empty_like(A)
    for t in range(g.nlt):
        ti, tj = divmod(t, g.lt_cols)
        r0, c0 = ti * g.h_l, tj * g.k_l
        for r in range(g.h_l):
            out[r0 + r, c0:c0 + g.k_l] = A[r0 + int(enc.rowmap[t][r]), c0:c0 + g.k_l]
    return out


# --------------------------------------------------------------------------
# Decoding
# --------------------------------------------------------------------------

def _payload_values(enc: UnionEncoded) -> np.ndarray:
    if enc.val_type == VAL_F16:
        return enc.values.astype(np.uint16)
    if enc.val_type == VAL_I4:
        return unpack_nibbles(enc.values, enc.payload)
    return unpack_crumbs(enc.values, enc.payload)


def check_union(enc: UnionEncoded) -> None:
    """Offsets start at 0, advance by Q P_t per LT and end at the payload."""
    g = enc.geom
    off = enc.offsets.astype(np.int64)
    if off.shape != (g.nlt + 1,) or off[0] != 0 or off[-1] != enc.payload:
        raise ValueError("offsets do not frame the payload")
    counts = np.array([sum(popcount(int(w)) for w in enc.bitmaps[t * g.words_per_lt:(t + 1) * g.words_per_lt])
                       for t in range(g.nlt)], dtype=np.int64)
    if not np.array_equal(np.diff(off), g.Q * counts):
        raise ValueError("an LT's payload span is not Q times its union popcount")


def union_rank(words: np.ndarray, p: int) -> int:
    """Compact rank of logical position p of an LT: active bits before it."""
    w, b = divmod(p, 64)
    return sum(popcount(int(x)) for x in words[:w]) + masked_popcount(int(words[w]), b)


def decode_union_loop(enc: UnionEncoded) -> np.ndarray:
    """Per-element payload [M][K] (fp16 bits or int8 q) from the streams.

    Every position of every LT reads its union bit; an active one reads its
    rank by masked popcount and takes area q's value at o_t + q P_t + rank.
    """
    check_union(enc)
    g = enc.geom
    vals = _payload_values(enc)
    out = np.zeros((g.M, g.K), dtype=vals.dtype)
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
                    rank = union_rank(words, p)
                    for q in range(g.Q):
                        ar, ac = divmod(q, g.c_a)
                        out[ti * g.h_l + ar * g.am + i, tj * g.k_l + ac * g.ak + j] = vals[o_t + q * P_t + rank]
            t += 1
    return _unpermute(enc, out)


def decode_union(enc: UnionEncoded) -> np.ndarray:
    """Vectorised decode (same result as decode_union_loop)."""
    check_union(enc)
    g = enc.geom
    bits = np.unpackbits(enc.bitmaps.astype("<u8").view(np.uint8), bitorder="little").astype(bool)
    union = bits.reshape(g.nlt, g.am * g.ak)
    vals = _payload_values(enc)
    T = np.zeros((g.nlt, g.Q, g.am * g.ak), dtype=vals.dtype)
    T[np.broadcast_to(union[:, None, :], T.shape)] = vals
    return _unpermute(enc, area_unview(T, g))


def dense_weight_union(enc: UnionEncoded) -> np.ndarray:
    """fp64 dense weight the encoding stands for."""
    P = decode_union(enc)
    if enc.val_type == VAL_F16:
        return P.view(np.float16).astype(np.float64)
    return P.astype(np.float64) * enc.scales.astype(np.float64)[:, None]


def spmm_union(enc: UnionEncoded, X: np.ndarray) -> np.ndarray:
    """Decode, then the fp64 product Y [N][M] = X W^T."""
    return spmm_fp64(dense_weight_union(enc), X)


# --------------------------------------------------------------------------
# LSPD: bitmap-guided offsets and area gathering for one segment
# --------------------------------------------------------------------------

def lspd_segment(enc: UnionEncoded, t: int, row: int, seg: int, G: int):
    """The section's per-thread work for logical row ``row``, segment ``seg``.

    The segment covers union columns [seg G, seg G + G).  Its payload base is
    o_t plus the active bits before its first column; its k-th active bit
    reads index base + k of each area stream.  Returns a list of
    (column, [value of area 0, ..., area Q-1]); inactive columns are omitted
    (they are zeros in the fragment).
    """
    g = enc.geom
    words = enc.bitmaps[t * g.words_per_lt:(t + 1) * g.words_per_lt]
    o_t = int(enc.offsets[t])
    P_t = (int(enc.offsets[t + 1]) - o_t) // g.Q
    vals = _payload_values(enc)
    start = row * g.ak + seg * G
    base = union_rank(words, start)
    out = []
    k = 0
    for c in range(G):
        p = start + c
        if (int(words[p // 64]) >> (p % 64)) & 1:
            out.append((seg * G + c, [vals[o_t + q * P_t + base + k] for q in range(g.Q)]))
            k += 1
    return out
