"""Bitmap-encoded unstructured-sparse weight SpMM for AMD MI355X (gfx950).

Thin Python binding over libusw.so (include/usw.h).  Every step of the SpMM
runs in the library's HIP kernels; this module only marshals arguments,
using PyTorch for device memory and the current stream.

    enc = encode(W, mask)                 # host C++ encoder -> device tensors
    y = spmm(enc, x)                      # x [N][K] fp16 on the GPU -> y [N][M]

Format: TCA-BME (blog "SpInfer: How bitmaps make sparse LLMs actually fast",
section "How TCA-BME addresses the indexing overhead"); see include/usw.h for
the exact bit and tile orders.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np

from ._lib import (USW_OUT_F16, USW_OUT_F32, USW_VAL_F16, USW_VAL_I2, USW_VAL_I4, EXPORTED, UswCbcFmt, UswError,  # noqa: F401
                   UswFmt, UswUnionFmt, check, lib)

__all__ = ["HostEncoding", "Encoding", "encode_host", "encode", "to_device", "validate", "spmm",
           "spmm_workspace_bytes", "spmm_counter_bytes", "UnionHostEncoding", "UnionEncoding",
           "union_encode_host", "union_encode", "union_to_device", "union_validate", "union_spmm",
           "union_workspace_bytes", "CbcHostEncoding", "CbcEncoding", "cbc_encode_host", "cbc_encode",
           "cbc_to_device", "cbc_validate", "cbc_spmspv", "cbc_workspace_bytes", "save", "load", "UswError", "lib"]

_VAL = {"f16": USW_VAL_F16, "i4": USW_VAL_I4, "i2": USW_VAL_I2}


@dataclass
class HostEncoding:
    """Encoded matrix in host memory (numpy), as written by usw_encode."""
    M: int
    K: int
    gt_m: int
    gt_k: int
    val_type: int
    nnz: int
    bitmaps: np.ndarray          # uint64 [NBT]
    offsets: np.ndarray          # uint32 [NGT+1]
    values: np.ndarray           # uint8, padded allocation (values_alloc bytes)
    values_bytes: int            # logical byte count
    scales: Optional[np.ndarray]  # uint16 fp16 bits [M] (INT4) or None

    def fmt(self) -> UswFmt:
        return UswFmt(self.M, self.K, self.gt_m, self.gt_k, self.val_type, 0, self.nnz,
                      self.bitmaps.ctypes.data, self.offsets.ctypes.data, self.values.ctypes.data,
                      self.scales.ctypes.data if self.scales is not None else None)


@dataclass
class Encoding:
    """Encoded matrix on a GPU (torch tensors) plus its usw_fmt view."""
    M: int
    K: int
    gt_m: int
    gt_k: int
    val_type: int
    nnz: int
    bitmaps: "object"
    offsets: "object"
    values: "object"
    scales: "object"

    def fmt(self) -> UswFmt:
        return UswFmt(self.M, self.K, self.gt_m, self.gt_k, self.val_type, 0, self.nnz,
                      self.bitmaps.data_ptr(), self.offsets.data_ptr(), self.values.data_ptr(),
                      self.scales.data_ptr() if self.scales is not None else None)

    @property
    def device(self):
        return self.bitmaps.device


@dataclass
class UnionHostEncoding:
    """IE-BME encoding in host memory (numpy), as written by usw_union_encode."""
    M: int
    K: int
    lt_m: int
    lt_k: int
    r_a: int
    c_a: int
    val_type: int
    payload: int
    bitmaps: np.ndarray           # uint64 [NLT * NW]
    offsets: np.ndarray           # uint32 [NLT+1]
    values: np.ndarray            # uint8, padded allocation
    values_bytes: int             # logical byte count
    scales: Optional[np.ndarray]  # uint16 fp16 bits [M] (INT4) or None
    rowmap: Optional[np.ndarray] = None   # uint8 [NLT * lt_m] for reordered LTs, else None

    def fmt(self) -> UswUnionFmt:
        return UswUnionFmt(self.M, self.K, self.lt_m, self.lt_k, self.r_a, self.c_a, self.val_type, 0, self.payload,
                           self.bitmaps.ctypes.data, self.offsets.ctypes.data, self.values.ctypes.data,
                           self.scales.ctypes.data if self.scales is not None else None,
                           self.rowmap.ctypes.data if self.rowmap is not None else None)


@dataclass
class UnionEncoding:
    """IE-BME encoding on a GPU (torch tensors) plus its usw_union_fmt view."""
    M: int
    K: int
    lt_m: int
    lt_k: int
    r_a: int
    c_a: int
    val_type: int
    payload: int
    bitmaps: "object"
    offsets: "object"
    values: "object"
    scales: "object"
    rowmap: "object" = None

    def fmt(self) -> UswUnionFmt:
        return UswUnionFmt(self.M, self.K, self.lt_m, self.lt_k, self.r_a, self.c_a, self.val_type, 0, self.payload,
                           self.bitmaps.data_ptr(), self.offsets.data_ptr(), self.values.data_ptr(),
                           self.scales.data_ptr() if self.scales is not None else None,
                           self.rowmap.data_ptr() if self.rowmap is not None else None)


@dataclass
class CbcHostEncoding:
    """Tiled-CBC encoding in host memory (numpy), as written by usw_cbc_encode."""
    M: int
    K: int
    nnz: int
    nnz_padded: int
    bitmaps: np.ndarray        # uint64 [NGT * 64]
    tile_offsets: np.ndarray   # uint32 [NGT+1]
    colinfo: np.ndarray        # uint32 [NGT * 16]
    values: np.ndarray         # uint16 fp16 bits [nnz_padded]

    def fmt(self) -> UswCbcFmt:
        return UswCbcFmt(self.M, self.K, 256, 16, USW_VAL_F16, 0, self.nnz_padded, self.bitmaps.ctypes.data,
                         self.tile_offsets.ctypes.data, self.colinfo.ctypes.data, self.values.ctypes.data)


@dataclass
class CbcEncoding:
    """Tiled-CBC encoding on a GPU (torch tensors) plus its usw_cbc_fmt view."""
    M: int
    K: int
    nnz: int
    nnz_padded: int
    bitmaps: "object"
    tile_offsets: "object"
    colinfo: "object"
    values: "object"

    def fmt(self) -> UswCbcFmt:
        return UswCbcFmt(self.M, self.K, 256, 16, USW_VAL_F16, 0, self.nnz_padded, self.bitmaps.data_ptr(),
                         self.tile_offsets.data_ptr(), self.colinfo.data_ptr(), self.values.data_ptr())


def _as_numpy_f16(W) -> np.ndarray:
    if hasattr(W, "detach"):
        W = W.detach().cpu().numpy()
    W = np.ascontiguousarray(W)
    if W.dtype != np.float16:
        raise TypeError("W must be float16")
    return W


def encode_host(W, mask=None, gt=(64, 64), dtype: str = "f16") -> HostEncoding:
    """Run usw_encode on host arrays. ``mask`` None keeps the IEEE nonzeros."""
    W = _as_numpy_f16(W)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    M, K = W.shape
    if mask is not None:
        if hasattr(mask, "detach"):
            mask = mask.detach().cpu().numpy()
        mask = np.ascontiguousarray(mask.astype(np.uint8, copy=False))
        if mask.shape != W.shape:
            raise ValueError("mask shape must match W")
    vt = _VAL[dtype]
    L = lib()
    nnz = ctypes.c_int64()
    sz = [ctypes.c_size_t() for _ in range(5)]
    wp = W.ctypes.data
    mp = mask.ctypes.data if mask is not None else None
    check(L.usw_encode_query(wp, mp, M, K, gt[0], gt[1], vt, ctypes.byref(nnz), *[ctypes.byref(s) for s in sz]),
          "usw_encode_query")
    b_bm, b_off, b_val, b_alloc, b_sc = (s.value for s in sz)
    bitmaps = np.empty(b_bm // 8, dtype=np.uint64)
    offsets = np.empty(b_off // 4, dtype=np.uint32)
    values = np.empty(b_alloc, dtype=np.uint8)
    scales = np.empty(M, dtype=np.uint16) if vt == USW_VAL_I4 else None
    check(L.usw_encode(wp, mp, M, K, gt[0], gt[1], vt, bitmaps.ctypes.data, offsets.ctypes.data,
                       values.ctypes.data, b_alloc, scales.ctypes.data if scales is not None else None),
          "usw_encode")
    return HostEncoding(M, K, gt[0], gt[1], vt, nnz.value, bitmaps, offsets, values, b_val, scales)


def _as_mask(mask, shape):
    if mask is None:
        return None
    if hasattr(mask, "detach"):
        mask = mask.detach().cpu().numpy()
    mask = np.ascontiguousarray(mask.astype(np.uint8, copy=False))
    if mask.shape != shape:
        raise ValueError("mask shape must match W")
    return mask


def union_encode_host(W, mask=None, lt=(64, 64), areas=(2, 2), dtype: str = "i4", perm=None) -> UnionHostEncoding:
    """Run usw_union_encode on host arrays (IE-BME union-mask format).

    ``perm`` (int32 [NLT][lt_m], e.g. from ``union_reorder``) rearranges each
    LT's rows before compression (usw_union_encode_reordered); the encoding
    then carries the rowmap the product kernel needs."""
    W = _as_numpy_f16(W)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    M, K = W.shape
    mask = _as_mask(mask, W.shape)
    vt = _VAL[dtype]
    L = lib()
    if perm is not None:
        return _union_encode_reordered_host(W, mask, lt, areas, vt, perm)
    payload = ctypes.c_int64()
    sz = [ctypes.c_size_t() for _ in range(5)]
    wp = W.ctypes.data
    mp = mask.ctypes.data if mask is not None else None
    check(L.usw_union_encode_query(wp, mp, M, K, lt[0], lt[1], areas[0], areas[1], vt, ctypes.byref(payload),
                                   *[ctypes.byref(s) for s in sz]), "usw_union_encode_query")
    b_bm, b_off, b_val, b_alloc, _ = (s.value for s in sz)
    bitmaps = np.empty(b_bm // 8, dtype=np.uint64)
    offsets = np.empty(b_off // 4, dtype=np.uint32)
    values = np.empty(b_alloc, dtype=np.uint8)
    scales = np.empty(M, dtype=np.uint16) if vt != USW_VAL_F16 else None
    check(L.usw_union_encode(wp, mp, M, K, lt[0], lt[1], areas[0], areas[1], vt, bitmaps.ctypes.data,
                             offsets.ctypes.data, values.ctypes.data, b_alloc,
                             scales.ctypes.data if scales is not None else None), "usw_union_encode")
    return UnionHostEncoding(M, K, lt[0], lt[1], areas[0], areas[1], vt, payload.value, bitmaps, offsets, values,
                             b_val, scales)


def _union_encode_reordered_host(W, mask, lt, areas, vt, perm) -> UnionHostEncoding:
    M, K = W.shape
    perm = np.ascontiguousarray(np.asarray(perm, dtype=np.int32))
    if lt[0] <= 0 or lt[1] <= 0 or perm.size != (M // lt[0]) * (K // lt[1]) * lt[0]:
        raise ValueError("perm must hold one row order of lt_m rows per LT")
    L = lib()
    payload = ctypes.c_int64()
    b_val, b_alloc = ctypes.c_size_t(), ctypes.c_size_t()
    wp = W.ctypes.data
    mp = mask.ctypes.data if mask is not None else None
    args = (M, K, lt[0], lt[1], areas[0], areas[1], vt)
    check(L.usw_union_encode_reordered_query(wp, mp, *args, perm.ctypes.data, ctypes.byref(payload),
                                             ctypes.byref(b_val), ctypes.byref(b_alloc)),
          "usw_union_encode_reordered_query")
    sz = [ctypes.c_size_t() for _ in range(5)]
    check(L.usw_union_encode_query(wp, mp, *args, None, *[ctypes.byref(x) for x in sz]), "usw_union_encode_query")
    b_bm, b_off = sz[0].value, sz[1].value
    bitmaps = np.empty(b_bm // 8, dtype=np.uint64)
    offsets = np.empty(b_off // 4, dtype=np.uint32)
    values = np.empty(b_alloc.value, dtype=np.uint8)
    scales = np.empty(M, dtype=np.uint16) if vt != USW_VAL_F16 else None
    rowmap = np.empty(perm.size, dtype=np.uint8)
    check(L.usw_union_encode_reordered(wp, mp, *args, perm.ctypes.data, bitmaps.ctypes.data, offsets.ctypes.data,
                                       values.ctypes.data, b_alloc.value,
                                       scales.ctypes.data if scales is not None else None, rowmap.ctypes.data),
          "usw_union_encode_reordered")
    return UnionHostEncoding(M, K, lt[0], lt[1], areas[0], areas[1], vt, payload.value, bitmaps, offsets, values,
                             b_val.value, scales, rowmap)


def union_encode_device(W, mask=None, lt=(64, 64), areas=(2, 2), dtype: str = "i4") -> UnionEncoding:
    """IE-BME encoding (INT4, or 2-bit with dtype="i2") of a weight already
    on the GPU (usw_union_encode_device_index, then
    usw_union_encode_device_values) on torch's current stream; the same
    bytes as ``union_encode(W, mask, lt, areas, dtype)``.  Reading the
    payload size between the calls synchronises the stream."""
    if dtype not in ("i4", "i2"):
        raise ValueError("the device IE-BME encoder writes INT4 or 2-bit payloads")
    vt = _VAL[dtype]
    import torch
    if not (torch.is_tensor(W) and W.is_cuda and W.dtype == torch.float16 and W.dim() == 2):
        raise TypeError("W must be a 2-D float16 CUDA tensor")
    W = W.contiguous()
    M, K = W.shape
    if mask is not None:
        if not torch.is_tensor(mask) or mask.shape != W.shape or mask.device != W.device:
            raise ValueError("mask must be a tensor of W's shape on W's device")
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        elif mask.dtype != torch.uint8:
            mask = (mask != 0).view(torch.uint8)
        mask = mask.contiguous()
    if lt[0] <= 0 or lt[1] <= 0 or M % lt[0] or K % lt[1] or lt[0] % areas[0] or lt[1] % areas[1]:
        raise ValueError("M, K must be multiples of the LT shape, and the LT of the area grid")
    nlt = (M // lt[0]) * (K // lt[1])
    nw = (lt[0] // areas[0]) * (lt[1] // areas[1]) // 64
    dev = W.device
    bitmaps = torch.empty(max(nlt * nw, 1), dtype=torch.int64, device=dev)
    offsets = torch.empty(nlt + 1, dtype=torch.int32, device=dev)
    scales = torch.empty(M, dtype=torch.int16, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    L = lib()
    mp = mask.data_ptr() if mask is not None else None
    args = (M, K, lt[0], lt[1], areas[0], areas[1], vt)
    check(L.usw_union_encode_device_index(W.data_ptr(), mp, *args, bitmaps.data_ptr(), offsets.data_ptr(),
                                          scales.data_ptr(), st), "usw_union_encode_device_index")
    payload = int(offsets[nlt].item()) & 0xFFFFFFFF
    values = torch.empty(_values_alloc_bytes(vt, payload), dtype=torch.uint8, device=dev)
    check(L.usw_union_encode_device_values(W.data_ptr(), mp, *args, bitmaps.data_ptr(), offsets.data_ptr(),
                                           scales.data_ptr(), payload, values.data_ptr(), values.numel(), st),
          "usw_union_encode_device_values")
    return UnionEncoding(M, K, lt[0], lt[1], areas[0], areas[1], vt, payload, bitmaps, offsets, values, scales)


def union_reorder(W, mask=None, lt=(16, 64), areas=(2, 2)):
    """Bitmap-aware row reordering of every LT (usw_union_reorder).

    Returns (perm int32 [NLT][lt_m] of LT-local rows, active union entries
    per LT before, after).  ``mask`` None keeps the IEEE nonzeros of W.
    """
    W = _as_numpy_f16(W)
    M, K = W.shape
    mask = _as_mask(mask, W.shape)
    nlt = (M // lt[0]) * (K // lt[1]) if lt[0] > 0 and lt[1] > 0 else 0
    perm = np.zeros((max(nlt, 1), max(lt[0], 1)), dtype=np.int32)
    before = np.zeros(max(nlt, 1), dtype=np.int32)
    after = np.zeros(max(nlt, 1), dtype=np.int32)
    check(lib().usw_union_reorder(W.ctypes.data, mask.ctypes.data if mask is not None else None, M, K, lt[0], lt[1],
                                  areas[0], areas[1], perm.ctypes.data, before.ctypes.data, after.ctypes.data),
          "usw_union_reorder")
    return perm[:nlt], before[:nlt], after[:nlt]


def apply_row_permutation(W, perm, lt_m: int, lt_k: int):
    """W with every LT's rows permuted as usw_union_reorder returned them."""
    W = np.asarray(W)
    M, K = W.shape
    out = np.empty_like(W)
    lc = K // lt_k
    for t in range(perm.shape[0]):
        ti, tj = divmod(t, lc)
        rows = ti * lt_m + perm[t]
        out[ti * lt_m:(ti + 1) * lt_m, tj * lt_k:(tj + 1) * lt_k] = W[rows, tj * lt_k:(tj + 1) * lt_k]
    return out


def union_validate(enc: UnionHostEncoding) -> None:
    """usw_union_validate on a host encoding (raises UswError when corrupt)."""
    f = enc.fmt()
    check(lib().usw_union_validate(ctypes.byref(f)), "usw_union_validate")


def union_to_device(enc: UnionHostEncoding, device="cuda") -> UnionEncoding:
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
    return UnionEncoding(enc.M, enc.K, enc.lt_m, enc.lt_k, enc.r_a, enc.c_a, enc.val_type, enc.payload,
                         t(enc.bitmaps.view(np.int64)), t(enc.offsets.view(np.int32)), t(enc.values),
                         t(enc.scales.view(np.int16)) if enc.scales is not None else None,
                         t(enc.rowmap) if enc.rowmap is not None else None)


def union_encode(W, mask=None, lt=(64, 64), areas=(2, 2), dtype: str = "i4", device="cuda",
                 perm=None) -> UnionEncoding:
    """Encode on the host (usw_union_encode, or usw_union_encode_reordered
    with ``perm``) and copy the buffers to ``device``."""
    return union_to_device(union_encode_host(W, mask, lt, areas, dtype, perm), device)


def union_workspace_bytes(enc: UnionEncoding, N: int, splits: int = 0):
    """(workspace bytes, counter bytes) of usw_union_spmm."""
    f = enc.fmt()
    b = ctypes.c_size_t()
    c = ctypes.c_size_t()
    check(lib().usw_union_spmm_workspace(ctypes.byref(f), int(N), int(splits), ctypes.byref(b)),
          "usw_union_spmm_workspace")
    check(lib().usw_union_spmm_counter_bytes(ctypes.byref(f), int(N), int(splits), ctypes.byref(c)),
          "usw_union_spmm_counter_bytes")
    return b.value, c.value


def union_spmm(enc: UnionEncoding, x, y=None, out_dtype=None, splits: int = 0, stream=None):
    """Y [N][M] = W_sp . X from an IE-BME encoding (usw_union_spmm)."""
    import torch
    if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != enc.K:
        raise ValueError("x must be [N][K] float16")
    if not x.is_contiguous():
        x = x.contiguous()
    N = x.shape[0]
    st = stream if stream is not None else torch.cuda.current_stream(x.device)
    if y is None:
        with torch.cuda.stream(st):
            y = torch.empty((N, enc.M), dtype=out_dtype or torch.float16, device=x.device)
    if y.shape != (N, enc.M) or not y.is_contiguous():
        raise ValueError("y must be a contiguous [N][M] tensor")
    yt = {torch.float16: USW_OUT_F16, torch.float32: USW_OUT_F32}.get(y.dtype)
    if yt is None:
        raise ValueError("y must be float16 or float32")
    f = enc.fmt()
    nbytes, cbytes = union_workspace_bytes(enc, N, splits)
    ws = _workspace(st, nbytes, cbytes) if nbytes else None
    check(lib().usw_union_spmm(ctypes.byref(f), x.data_ptr(), y.data_ptr(), yt, N, int(splits),
                               ws.data_ptr() if ws is not None else None, nbytes, ctypes.c_void_p(st.cuda_stream)),
          "usw_union_spmm")
    return y


def cbc_encode_host(W, mask=None) -> CbcHostEncoding:
    """Run usw_cbc_encode on host arrays (Tiled-CBC, 256x16 GTiles, fp16 values)."""
    W = _as_numpy_f16(W)
    if W.ndim != 2:
        raise ValueError("W must be 2-D")
    M, K = W.shape
    mask = _as_mask(mask, W.shape)
    L = lib()
    nnz, npad = ctypes.c_int64(), ctypes.c_int64()
    sz = [ctypes.c_size_t() for _ in range(4)]
    wp = W.ctypes.data
    mp = mask.ctypes.data if mask is not None else None
    check(L.usw_cbc_encode_query(wp, mp, M, K, ctypes.byref(nnz), ctypes.byref(npad), *[ctypes.byref(s) for s in sz]),
          "usw_cbc_encode_query")
    b_bm, b_off, b_ci, b_val = (s.value for s in sz)
    bitmaps = np.empty(b_bm // 8, dtype=np.uint64)
    offs = np.empty(b_off // 4, dtype=np.uint32)
    colinfo = np.empty(b_ci // 4, dtype=np.uint32)
    values = np.empty(max(b_val // 2, 8), dtype=np.uint16)
    check(L.usw_cbc_encode(wp, mp, M, K, bitmaps.ctypes.data, offs.ctypes.data, colinfo.ctypes.data,
                           values.ctypes.data, values.nbytes), "usw_cbc_encode")
    return CbcHostEncoding(M, K, nnz.value, npad.value, bitmaps, offs, colinfo, values)


def cbc_validate(enc: CbcHostEncoding) -> None:
    """usw_cbc_validate on a host encoding (raises UswError when corrupt)."""
    f = enc.fmt()
    check(lib().usw_cbc_validate(ctypes.byref(f)), "usw_cbc_validate")


def cbc_to_device(enc: CbcHostEncoding, device="cuda") -> CbcEncoding:
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
    return CbcEncoding(enc.M, enc.K, enc.nnz, enc.nnz_padded, t(enc.bitmaps.view(np.int64)),
                       t(enc.tile_offsets.view(np.int32)), t(enc.colinfo.view(np.int32)), t(enc.values.view(np.int16)))


def cbc_encode_device(W, mask=None) -> CbcEncoding:
    """Tiled-CBC encoding of a weight already on the GPU
    (usw_cbc_encode_device_index, then usw_cbc_encode_device_values) on
    torch's current stream; the same bytes as ``cbc_encode(W, mask)``.
    Reading the padded size between the calls synchronises the stream."""
    import torch
    if not (torch.is_tensor(W) and W.is_cuda and W.dtype == torch.float16 and W.dim() == 2):
        raise TypeError("W must be a 2-D float16 CUDA tensor")
    W = W.contiguous()
    M, K = W.shape
    if mask is not None:
        if not torch.is_tensor(mask) or mask.shape != W.shape or mask.device != W.device:
            raise ValueError("mask must be a tensor of W's shape on W's device")
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        elif mask.dtype != torch.uint8:
            mask = (mask != 0).view(torch.uint8)
        mask = mask.contiguous()
    if M % 256 or K % 16:
        raise ValueError("M and K must be multiples of 256 and 16")
    ngt = (M // 256) * (K // 16)
    dev = W.device
    bitmaps = torch.empty(max(ngt * 64, 1), dtype=torch.int64, device=dev)
    offs = torch.empty(ngt + 1, dtype=torch.int32, device=dev)
    colinfo = torch.empty(max(ngt * 16, 1), dtype=torch.int32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    L = lib()
    check(L.usw_cbc_encode_device_index(W.data_ptr(), mask.data_ptr() if mask is not None else None, M, K,
                                        bitmaps.data_ptr(), offs.data_ptr(), colinfo.data_ptr(), st),
          "usw_cbc_encode_device_index")
    npad = int(offs[ngt].item()) & 0xFFFFFFFF
    values = torch.empty(max(npad, 8), dtype=torch.int16, device=dev)
    check(L.usw_cbc_encode_device_values(W.data_ptr(), M, K, bitmaps.data_ptr(), offs.data_ptr(), colinfo.data_ptr(),
                                         npad, values.data_ptr(), values.numel() * 2, st),
          "usw_cbc_encode_device_values")
    nnz = int((colinfo.cpu().numpy().view(np.uint32) & 0xFFFF).sum()) if ngt else 0
    return CbcEncoding(M, K, nnz, npad, bitmaps, offs, colinfo, values)


def cbc_encode(W, mask=None, device="cuda") -> CbcEncoding:
    """Encode on the host (usw_cbc_encode) and copy the buffers to ``device``."""
    return cbc_to_device(cbc_encode_host(W, mask), device)


def cbc_workspace_bytes(enc: CbcEncoding, splits: int = 0):
    """(workspace bytes, counter bytes) of usw_cbc_spmspv."""
    f = enc.fmt()
    b, c = ctypes.c_size_t(), ctypes.c_size_t()
    check(lib().usw_cbc_spmspv_workspace(ctypes.byref(f), int(splits), ctypes.byref(b), ctypes.byref(c)),
          "usw_cbc_spmspv_workspace")
    return b.value, c.value


def cbc_spmspv(enc: CbcEncoding, x, tau: float = 0.0, y=None, out_dtype=None, splits: int = 0, stream=None):
    """y [M] = W_sp x over the columns with |x_k| >= tau (usw_cbc_spmspv)."""
    import torch
    if x.dtype != torch.float16 or x.numel() != enc.K:
        raise ValueError("x must hold K float16 values")
    x = x.reshape(-1).contiguous()
    st = stream if stream is not None else torch.cuda.current_stream(x.device)
    if y is None:
        with torch.cuda.stream(st):
            y = torch.empty(enc.M, dtype=out_dtype or torch.float16, device=x.device)
    if y.numel() != enc.M or not y.is_contiguous():
        raise ValueError("y must be a contiguous tensor of M values")
    yt = {torch.float16: USW_OUT_F16, torch.float32: USW_OUT_F32}.get(y.dtype)
    if yt is None:
        raise ValueError("y must be float16 or float32")
    f = enc.fmt()
    nbytes, cbytes = cbc_workspace_bytes(enc, splits)
    ws = _workspace(st, nbytes, cbytes) if nbytes else None
    check(lib().usw_cbc_spmspv(ctypes.byref(f), x.data_ptr(), y.data_ptr(), yt, float(tau), int(splits),
                               ws.data_ptr() if ws is not None else None, nbytes, ctypes.c_void_p(st.cuda_stream)),
          "usw_cbc_spmspv")
    return y


def validate(enc: HostEncoding) -> None:
    """usw_validate on a host encoding (raises UswError when corrupt)."""
    f = enc.fmt()
    check(lib().usw_validate(ctypes.byref(f)), "usw_validate")


def to_device(enc: HostEncoding, device="cuda") -> Encoding:
    import torch
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)  # noqa: E731
    return Encoding(enc.M, enc.K, enc.gt_m, enc.gt_k, enc.val_type, enc.nnz,
                    t(enc.bitmaps.view(np.int64)), t(enc.offsets.view(np.int32)), t(enc.values),
                    t(enc.scales.view(np.int16)) if enc.scales is not None else None)


def encode(W, mask=None, gt=(64, 64), dtype: str = "f16", device="cuda") -> Encoding:
    """Encode on the host (usw_encode) and copy the buffers to ``device``."""
    return to_device(encode_host(W, mask, gt, dtype), device)


def _values_alloc_bytes(val_type: int, nnz: int) -> int:
    """Values allocation usw_spmm expects: the logical size rounded down to a
    multiple of 16, plus 16 (as usw_encode_query reports it)."""
    logical = 2 * nnz if val_type == USW_VAL_F16 else (nnz + 1) // 2 if val_type == USW_VAL_I4 else (nnz + 3) // 4
    return (logical & ~15) + 16


def encode_device(W, mask=None, gt=(64, 64), dtype: str = "f16") -> Encoding:
    """Encode a weight that is already on the GPU (usw_encode_device_index,
    then usw_encode_device_values) on torch's current stream.

    ``W`` is a contiguous [M][K] float16 CUDA tensor; ``mask`` None keeps the
    IEEE nonzeros, else a [M][K] bool or uint8 tensor on the same device.
    The result has the same bytes as ``encode(W, mask, gt, dtype)``.  Reading
    NNZ between the two calls synchronises the stream.
    """
    import torch
    if not (torch.is_tensor(W) and W.is_cuda and W.dtype == torch.float16 and W.dim() == 2):
        raise TypeError("W must be a 2-D float16 CUDA tensor")
    W = W.contiguous()
    M, K = W.shape
    if mask is not None:
        if not torch.is_tensor(mask) or mask.shape != W.shape or mask.device != W.device:
            raise ValueError("mask must be a tensor of W's shape on W's device")
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        elif mask.dtype != torch.uint8:
            mask = (mask != 0).view(torch.uint8)
        mask = mask.contiguous()
    vt = _VAL[dtype]
    dev = W.device
    if gt[0] <= 0 or gt[1] <= 0 or M % gt[0] or K % gt[1]:
        raise ValueError("M and K must be multiples of the GroupTile shape")
    ngt = (M // gt[0]) * (K // gt[1])
    bitmaps = torch.empty(M * K // 64, dtype=torch.int64, device=dev)
    offsets = torch.empty(ngt + 1, dtype=torch.int32, device=dev)
    scales = torch.empty(M, dtype=torch.int16, device=dev) if vt == USW_VAL_I4 else None
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    L = lib()
    check(L.usw_encode_device_index(W.data_ptr(), mask.data_ptr() if mask is not None else None, M, K, gt[0], gt[1],
                                    vt, bitmaps.data_ptr(), offsets.data_ptr(),
                                    scales.data_ptr() if scales is not None else None, st),
          "usw_encode_device_index")
    nnz = int(offsets[ngt].item()) & 0xFFFFFFFF
    values = torch.empty(_values_alloc_bytes(vt, nnz), dtype=torch.uint8, device=dev)
    check(L.usw_encode_device_values(W.data_ptr(), M, K, gt[0], gt[1], vt, bitmaps.data_ptr(), offsets.data_ptr(),
                                     scales.data_ptr() if scales is not None else None, nnz, values.data_ptr(),
                                     values.numel(), st),
          "usw_encode_device_values")
    return Encoding(M, K, gt[0], gt[1], vt, nnz, bitmaps, offsets, values, scales)


def spmm_workspace_bytes(enc: Encoding, N: int, splits: int = 0) -> int:
    f = enc.fmt()
    b = ctypes.c_size_t()
    check(lib().usw_spmm_workspace_ex(ctypes.byref(f), int(N), int(splits), ctypes.byref(b)), "usw_spmm_workspace")
    return b.value


_WS = {}


def spmm_counter_bytes(enc: Encoding, N: int, splits: int = 0) -> int:
    f = enc.fmt()
    b = ctypes.c_size_t()
    check(lib().usw_spmm_counter_bytes(ctypes.byref(f), int(N), int(splits), ctypes.byref(b)), "usw_spmm_counter_bytes")
    return b.value


def _workspace(stream, nbytes: int, counter_bytes: int):
    """One zero-filled workspace per (device, stream).

    Its first ``counter_bytes`` bytes must be zero when a call starts; each
    call leaves them zero, but a call with another counter size may have
    written partial sums there, so they are cleared (a small fill kernel)
    whenever the counter size changes.  The allocation and the clear are
    issued on ``stream``, the stream the call launches on, so they are
    ordered before it; calls on different streams never share a workspace.
    """
    import torch
    key = (str(stream.device), int(stream.cuda_stream))
    ent = _WS.get(key)
    with torch.cuda.stream(stream):
        if ent is None or ent[0].numel() < nbytes:
            ent = [torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=stream.device), counter_bytes]
            _WS[key] = ent
        elif ent[1] != counter_bytes:
            ent[0][:counter_bytes].zero_()
            ent[1] = counter_bytes
    return ent[0]


def spmm(enc: Encoding, x, y=None, out_dtype=None, splits: int = 0, stream=None):
    """Y [N][M] = W_sp . X for x [N][K] fp16 on enc's device (usw_spmm_ex).

    ``y`` (optional) must be a contiguous [N][M] fp16 or fp32 tensor.  The
    launch goes on ``stream`` (default: torch's current stream).
    """
    import torch
    if x.dtype != torch.float16 or x.dim() != 2 or x.shape[1] != enc.K:
        raise ValueError("x must be [N][K] float16")
    if not x.is_contiguous():
        x = x.contiguous()
    N = x.shape[0]
    st = stream if stream is not None else torch.cuda.current_stream(x.device)
    if y is None:
        with torch.cuda.stream(st):
            y = torch.empty((N, enc.M), dtype=out_dtype or torch.float16, device=x.device)
    if y.shape != (N, enc.M) or not y.is_contiguous():
        raise ValueError("y must be a contiguous [N][M] tensor")
    yt = {torch.float16: USW_OUT_F16, torch.float32: USW_OUT_F32}.get(y.dtype)
    if yt is None:
        raise ValueError("y must be float16 or float32")
    f = enc.fmt()
    nbytes = spmm_workspace_bytes(enc, N, splits)
    ws = _workspace(st, nbytes, spmm_counter_bytes(enc, N, splits)) if nbytes else None
    check(lib().usw_spmm_ex(ctypes.byref(f), x.data_ptr(), y.data_ptr(), yt, N, int(splits),
                            ws.data_ptr() if ws is not None else None, nbytes, ctypes.c_void_p(st.cuda_stream)),
          "usw_spmm")
    return y


# ---------------------------------------------------------------------------
# Offline cache of encoded weights
# ---------------------------------------------------------------------------
#
# Encoding (and for IE-BME the row-reordering search) is offline work; the
# pages keep the converted weights and load them at inference time.  save()
# writes a host encoding's buffers and shape fields to an .npz archive (no
# pickled objects); load() reads it back with pickling disabled and runs the
# library's validator on it before returning, so a truncated or edited file
# is rejected instead of reaching a kernel.

_SCALARS = {
    "tca_bme": ("M", "K", "gt_m", "gt_k", "val_type", "nnz", "values_bytes"),
    "ie_bme": ("M", "K", "lt_m", "lt_k", "r_a", "c_a", "val_type", "payload", "values_bytes"),
    "tiled_cbc": ("M", "K", "nnz", "nnz_padded"),
}
_ARRAYS = {
    "tca_bme": (("bitmaps", np.uint64), ("offsets", np.uint32), ("values", np.uint8), ("scales", np.uint16)),
    "ie_bme": (("bitmaps", np.uint64), ("offsets", np.uint32), ("values", np.uint8), ("scales", np.uint16),
               ("rowmap", np.uint8)),
    "tiled_cbc": (("bitmaps", np.uint64), ("tile_offsets", np.uint32), ("colinfo", np.uint32), ("values", np.uint16)),
}
_CLASSES = {"tca_bme": HostEncoding, "ie_bme": UnionHostEncoding, "tiled_cbc": CbcHostEncoding}
_VALIDATE = {"tca_bme": validate, "ie_bme": union_validate, "tiled_cbc": cbc_validate}


def save(path, enc) -> None:
    """Write a host encoding (HostEncoding, UnionHostEncoding or
    CbcHostEncoding) to an .npz archive."""
    kind = next((k for k, c in _CLASSES.items() if isinstance(enc, c)), None)
    if kind is None:
        raise TypeError("save takes a host encoding; copy device encodings back first")
    out = {"kind": np.array(kind)}
    for name in _SCALARS[kind]:
        out[name] = np.array(int(getattr(enc, name)), dtype=np.int64)
    for name, dt in _ARRAYS[kind]:
        a = getattr(enc, name)
        if a is not None:
            out[name] = np.ascontiguousarray(a, dtype=dt)
    np.savez(path, **out)


def load(path):
    """Read an archive written by save(); the result has passed the
    library's validator (UswError otherwise)."""
    with np.load(path, allow_pickle=False) as z:
        if "kind" not in z.files:
            raise ValueError("not an encoding archive")
        kind = str(z["kind"])
        if kind not in _CLASSES:
            raise ValueError(f"unknown encoding kind {kind!r}")
        fields = {}
        for name in _SCALARS[kind]:
            if name not in z.files or z[name].shape != ():
                raise ValueError(f"archive lacks the field {name}")
            fields[name] = int(z[name])
        for name, dt in _ARRAYS[kind]:
            if name in z.files:
                a = z[name]
                if a.dtype != dt or a.ndim != 1:
                    raise ValueError(f"field {name} must be a 1-D {np.dtype(dt).name} array")
                fields[name] = np.ascontiguousarray(a)
            elif name in ("scales", "rowmap"):
                fields[name] = None
            else:
                raise ValueError(f"archive lacks the field {name}")
    enc = _CLASSES[kind](**fields)
    _check_sizes(kind, enc)
    _VALIDATE[kind](enc)
    return enc


def _check_sizes(kind, enc) -> None:
    """Array lengths against the shape fields, before any pointer reaches
    the library (the validator trusts them)."""
    def need(a, n, name):
        if a is None or a.size < n:
            raise ValueError(f"field {name} is shorter than its shape requires")
    if kind == "tca_bme":
        if enc.gt_m <= 0 or enc.gt_k <= 0 or enc.M % enc.gt_m or enc.K % enc.gt_k or enc.gt_m % 8 or enc.gt_k % 8:
            raise ValueError("bad GroupTile shape")
        ngt = (enc.M // enc.gt_m) * (enc.K // enc.gt_k)
        need(enc.bitmaps, ngt * (enc.gt_m // 8) * (enc.gt_k // 8), "bitmaps")
        need(enc.offsets, ngt + 1, "offsets")
        need(enc.values, _values_alloc_bytes(enc.val_type, enc.nnz), "values")
        if enc.val_type != USW_VAL_F16:
            need(enc.scales, enc.M, "scales")
    elif kind == "ie_bme":
        if min(enc.lt_m, enc.lt_k, enc.r_a, enc.c_a) <= 0 or enc.M % enc.lt_m or enc.K % enc.lt_k \
                or enc.lt_m % enc.r_a or enc.lt_k % enc.c_a:
            raise ValueError("bad LT shape or area grid")
        nlt = (enc.M // enc.lt_m) * (enc.K // enc.lt_k)
        need(enc.bitmaps, nlt * (enc.lt_m // enc.r_a) * (enc.lt_k // enc.c_a) // 64, "bitmaps")
        need(enc.offsets, nlt + 1, "offsets")
        need(enc.values, _values_alloc_bytes(enc.val_type, enc.payload), "values")
        if enc.val_type != USW_VAL_F16:
            need(enc.scales, enc.M, "scales")
        if enc.rowmap is not None:
            need(enc.rowmap, nlt * enc.lt_m, "rowmap")
    else:
        if enc.M % 256 or enc.K % 16 or enc.M <= 0 or enc.K <= 0:
            raise ValueError("bad Tiled-CBC shape")
        ngt = (enc.M // 256) * (enc.K // 16)
        need(enc.bitmaps, ngt * 64, "bitmaps")
        need(enc.tile_offsets, ngt + 1, "tile_offsets")
        need(enc.colinfo, ngt * 16, "colinfo")
        need(enc.values, enc.nnz_padded, "values")
