"""CPU oracle for the Tiled-CBC format and the dynamically pruned spMspV.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  The GPU library never imports,
links or calls it, and this module imports nothing from the GPU library.

What it computes, and where each step comes from ("Unified Static-Dynamic
Pruning for Efficient LLM Inference", section 4.1 Tiled-CBC, section 4.2
decode phase, section 2.2 pruning):

* Tiled-CBC.  The matrix is cut into GTiles of TILE_M x TILE_K (256 x 16,
  the sizes of section 4.2.3), stored row-major.  A GTile is TILE_K column
  tiles of TILE_M x 1, each described by TILE_M / 64 64-bit bitmap words (bit
  i of word j <-> row 64 j + i of the column, least significant bit first).
  Values hold the kept weights column by column (tile-column order), rows
  top to bottom.  TileOffset[t] is the element index of GTile t's first
  value; ColInfo packs, per column, its starting offset inside the tile in
  the upper 16 bits and its kept count in the lower 16 bits.  Storage
  (section 4.1's equation): 4 (NGT + 1) + 4 NGT TILE_K + 8 NBM + 2 NNZ bytes.
  Each column's run is padded with zeros to a multiple of 8 values (16
  bytes), as section 4.2.3 does for its 16-byte copies; NNZ in the equation
  then counts the padded runs.
* Dynamic pruning (section 2.2, W_dp(x) = W (.) M(x); section 4.2: columns
  whose activation fails a magnitude test are skipped).  Column k is active
  when |x_k| >= tau, both in fp32 (x is fp16, exact in fp32).  The product
  is the plain definition y[m] = sum_k W_sp[m][k] x_k [|x_k| >= tau],
  accumulated in fp64, i.e. the static product with the inactive entries of
  x set to zero.

Readings where the pages are silent (frozen here and listed with the design
notes): the bitmap word and bit order above; padding runs hold +0.0;
ColInfo offsets count elements including padding; tau is inclusive (>=);
only N = 1 (the section's spMspV); the mask is authoritative as in tca_bme.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .tca_bme import _check_inputs, masked_popcount, popcount, spmm_fp64

TILE_M = 256
TILE_K = 16
PAD = 8


@dataclass(frozen=True)
class CbcGeometry:
    M: int
    K: int
    tile_m: int = TILE_M
    tile_k: int = TILE_K

    def __post_init__(self):
        if min(self.M, self.K, self.tile_m, self.tile_k) <= 0:
            raise ValueError("sizes must be positive")
        if self.M % self.tile_m or self.K % self.tile_k or self.tile_m % 64:
            raise ValueError("M, K must be multiples of the GTile; TILE_M a multiple of 64")

    @property
    def gr(self) -> int:
        return self.M // self.tile_m

    @property
    def gc(self) -> int:
        return self.K // self.tile_k

    @property
    def ngt(self) -> int:
        return self.gr * self.gc

    @property
    def wpc(self) -> int:           # bitmap words per column tile
        return self.tile_m // 64

    @property
    def nbm(self) -> int:           # bitmap words in the matrix
        return self.M * self.K // 64


@dataclass
class CbcEncoded:
    geom: CbcGeometry
    nnz: int                  # kept weights
    nnz_padded: int           # stored values = tile_offsets[NGT]
    bitmaps: np.ndarray       # uint64 [NGT * TILE_K * wpc]
    tile_offsets: np.ndarray  # uint32 [NGT + 1]
    colinfo: np.ndarray       # uint32 [NGT * TILE_K]
    values: np.ndarray        # uint16 fp16 bits [nnz_padded]


def storage_bytes_cbc(ngt: int, tile_k: int, nbm: int, nnz: int) -> int:
    """Section 4.1's storage equation."""
    return 4 * (ngt + 1) + 4 * (ngt * tile_k) + 8 * nbm + 2 * nnz


def pad_run(n: int, pad: int = PAD) -> int:
    return (n + pad - 1) // pad * pad


def encode_cbc_loop(W: np.ndarray, mask: Optional[np.ndarray], tile_m: int = TILE_M,
                    tile_k: int = TILE_K) -> CbcEncoded:
    """Tiled-CBC written as the section describes it, one GTile at a time:
    for each column tile, its bitmap words, its kept values in row order
    (padded to 8), and its ColInfo entry."""
    mask = _check_inputs(W, mask)
    g = CbcGeometry(W.shape[0], W.shape[1], tile_m, tile_k)
    bits = W.view(np.uint16)
    bitmaps, colinfo, values, offs = [], [], [], [0]
    nnz = 0
    for ti in range(g.gr):
        for tj in range(g.gc):
            start = len(values)
            for c in range(tile_k):
                col = tj * tile_k + c
                run_start = len(values) - start
                words = [0] * g.wpc
                n = 0
                for r in range(tile_m):
                    if mask[ti * tile_m + r, col]:
                        words[r // 64] |= 1 << (r % 64)
                        values.append(int(bits[ti * tile_m + r, col]))
                        n += 1
                values.extend([0] * (pad_run(n) - n))
                nnz += n
                bitmaps.extend(words)
                colinfo.append((run_start << 16) | n)
            offs.append(len(values))
    if offs[-1] >= 1 << 32:
        raise ValueError("values do not fit 32-bit offsets")
    return CbcEncoded(g, nnz, offs[-1], np.array(bitmaps, dtype=np.uint64), np.array(offs, dtype=np.uint32),
                      np.array(colinfo, dtype=np.uint32), np.array(values, dtype=np.uint16))


def _tile_columns(A: np.ndarray, g: CbcGeometry) -> np.ndarray:
    """[NGT][TILE_K][TILE_M]: GTiles row-major, then columns, then rows."""
    T = A.reshape(g.gr, g.tile_m, g.gc, g.tile_k).transpose(0, 2, 3, 1)
    return T.reshape(g.ngt, g.tile_k, g.tile_m)


def encode_cbc(W: np.ndarray, mask: Optional[np.ndarray], tile_m: int = TILE_M,
               tile_k: int = TILE_K) -> CbcEncoded:
    """Vectorised Tiled-CBC encoding (an independent route to the same bytes)."""
    mask = _check_inputs(W, mask)
    g = CbcGeometry(W.shape[0], W.shape[1], tile_m, tile_k)
    mt = _tile_columns(mask, g)                                  # [NGT][TK][TM]
    vt = _tile_columns(W.view(np.uint16), g)
    counts = mt.sum(axis=2, dtype=np.int64)                      # [NGT][TK]
    padded = (counts + PAD - 1) // PAD * PAD
    # Padded slots: the first `padded` rows of a column, kept values first.
    order = np.argsort(~mt, axis=2, kind="stable")               # kept rows first, in row order
    sorted_vals = np.take_along_axis(np.where(mt, vt, 0), order, axis=2)
    slot = np.arange(tile_m)[None, None, :] < padded[:, :, None]
    values = sorted_vals[slot].astype(np.uint16)
    run_start = np.zeros_like(padded)
    run_start[:, 1:] = np.cumsum(padded, axis=1)[:, :-1]
    colinfo = ((run_start << 16) | counts).astype(np.uint32).reshape(-1)
    offs = np.zeros(g.ngt + 1, dtype=np.int64)
    np.cumsum(padded.sum(axis=1), out=offs[1:])
    if offs[-1] >= 1 << 32:
        raise ValueError("values do not fit 32-bit offsets")
    wbits = mt.reshape(g.ngt, tile_k, g.wpc, 64)
    words = np.packbits(wbits.astype(np.uint8), axis=3, bitorder="little").view("<u8")
    return CbcEncoded(g, int(counts.sum()), int(offs[-1]), words.reshape(-1).astype(np.uint64),
                      offs.astype(np.uint32), colinfo, values)


def check_cbc(enc: CbcEncoded) -> None:
    """Offsets, ColInfo and bitmaps agree."""
    g = enc.geom
    off = enc.tile_offsets.astype(np.int64)
    if off[0] != 0 or off[-1] != enc.nnz_padded or np.any(np.diff(off) < 0):
        raise ValueError("tile offsets do not frame the values")
    for t in range(g.ngt):
        run = 0
        for c in range(g.tile_k):
            ci = int(enc.colinfo[t * g.tile_k + c])
            n = sum(popcount(int(w)) for w in enc.bitmaps[(t * g.tile_k + c) * g.wpc:(t * g.tile_k + c + 1) * g.wpc])
            if ci >> 16 != run or ci & 0xFFFF != n:
                raise ValueError("ColInfo disagrees with the bitmaps")
            run += pad_run(n)
        if run != off[t + 1] - off[t]:
            raise ValueError("a GTile's span disagrees with its columns")


def decode_cbc_loop(enc: CbcEncoded) -> np.ndarray:
    """fp16 bits [M][K]: each kept position reads its column's run at its
    rank, the kept positions above it in the column (masked popcount of its
    word plus the popcounts of the column's earlier words)."""
    check_cbc(enc)
    g = enc.geom
    out = np.zeros((g.M, g.K), dtype=np.uint16)
    for t in range(g.ngt):
        ti, tj = divmod(t, g.gc)
        base = int(enc.tile_offsets[t])
        for c in range(g.tile_k):
            ci = int(enc.colinfo[t * g.tile_k + c])
            words = enc.bitmaps[(t * g.tile_k + c) * g.wpc:(t * g.tile_k + c + 1) * g.wpc]
            before = 0
            for j in range(g.wpc):
                w = int(words[j])
                for i in range(64):
                    if (w >> i) & 1:
                        rank = before + masked_popcount(w, i)
                        out[ti * g.tile_m + 64 * j + i, tj * g.tile_k + c] = enc.values[base + (ci >> 16) + rank]
                before += popcount(w)
    return out


def decode_cbc(enc: CbcEncoded) -> np.ndarray:
    """Vectorised decode (same result as decode_cbc_loop)."""
    check_cbc(enc)
    g = enc.geom
    bits = np.unpackbits(enc.bitmaps.astype("<u8").view(np.uint8), bitorder="little").astype(bool)
    mt = bits.reshape(g.ngt, g.tile_k, g.tile_m)
    counts = mt.sum(axis=2)
    padded = (counts + PAD - 1) // PAD * PAD
    slot = np.arange(g.tile_m)[None, None, :] < padded[:, :, None]
    runs = np.zeros((g.ngt, g.tile_k, g.tile_m), dtype=np.uint16)
    runs[slot] = enc.values
    # The kept rows of a column, in order, take the first `count` slots of its run.
    vt = np.zeros_like(runs)
    rank = np.cumsum(mt, axis=2) - 1
    src = np.take_along_axis(runs, np.where(mt, rank, 0), axis=2)
    vt[mt] = src[mt]
    A = vt.reshape(g.gr, g.gc, g.tile_k, g.tile_m).transpose(0, 3, 1, 2)
    return A.reshape(g.M, g.K)


def dp_active(x: np.ndarray, tau: float) -> np.ndarray:
    """Active columns: |x_k| >= tau, compared in fp32."""
    return np.abs(np.asarray(x, dtype=np.float16).astype(np.float32)) >= np.float32(tau)


def spmspv(enc: CbcEncoded, x: np.ndarray, tau: float) -> np.ndarray:
    """y [M] = W_sp x with the inactive entries of x skipped, in fp64."""
    x = np.asarray(x, dtype=np.float16).reshape(-1)
    Wd = decode_cbc(enc).view(np.float16).astype(np.float64)
    xd = np.where(dp_active(x, tau), x.astype(np.float64), 0.0)
    return spmm_fp64(Wd, xd[None, :])[0]


def spmspv_bound(enc: CbcEncoded, x: np.ndarray, tau: float) -> np.ndarray:
    """sum_k |W_sp[m][k]| |x_k| over active k: the scale of rounding error."""
    x = np.asarray(x, dtype=np.float16).reshape(-1)
    Wd = decode_cbc(enc).view(np.float16).astype(np.float64)
    xd = np.where(dp_active(x, tau), np.abs(x.astype(np.float64)), 0.0)
    return np.abs(Wd) @ xd


def ci_spdp(M: int, N: int, cr: float, s: float) -> float:
    """Equation (3) of section 3.2.3: M N / (M / CR (1 - s) + N)."""
    return M * N / (M / cr * (1.0 - s) + N)
