/*
 * usw.h -- bitmap-encoded unstructured-sparse weight x dense activation SpMM
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation is Y = W_sp . X with W_sp = W (elementwise) M, the static
 * unstructured pruning of "Unified Static-Dynamic Pruning for Efficient LLM
 * Inference" (section 2.2, static-pruning equation), computed from W_sp held
 * in the TCA-BME bitmap format described in the blog "SpInfer: How bitmaps
 * make sparse LLMs actually fast" (section "How TCA-BME addresses the
 * indexing overhead"):
 *
 *   - BitmapTile: an 8x8 block of W; one uint64 word, bit p <-> position p of
 *     the block taken row-major (p = 8*row + col), least significant bit first.
 *   - TCTile: 16x16 = 2x2 BitmapTiles, stored row-major (top-left, top-right,
 *     bottom-left, bottom-right).
 *   - GroupTile: gt_m x gt_k (multiples of 16; 64x64 by default) = TCTiles
 *     stored row-major; GroupTiles of the matrix stored row-major.
 *   - bitmaps[NBT]: all BitmapTile words in that storage order (NBT = M*K/64).
 *   - values[NNZ]: the kept elements, packed with no gaps in the same order
 *     (GroupTile -> TCTile -> BitmapTile -> position).
 *   - offsets[NGT+1]: uint32 element index of each GroupTile's first value,
 *     offsets[0] = 0 and offsets[NGT] = NNZ (NGT = (M/gt_m)*(K/gt_k)).
 *   Logical storage 4*(NGT+1) + 8*NBT + 2*NNZ bytes (the blog's storage
 *   equation).  A value is located by masked popcount: its index is the
 *   GroupTile offset plus the set bits that precede it in storage order (blog
 *   section "Shared Memory Bitmap Decoding (SMBD)").
 *
 * INT4 values (USW_VAL_I4): per output row m a symmetric scale
 *   scale[m] = fp16_rne(max|w| over row m's kept entries / 7) and
 *   q = clamp(round_half_even(w / scale[m]), -8, 7), all in fp64 (q = 0 when
 *   the scale is 0); the dequantised weight is q * scale[m].  Non-finite kept
 *   weights: a NaN makes the row's scale NaN (0x7E00) and its codes 0; an
 *   infinity makes the scale infinite, and inf / inf gives code 0.  Element 2i of the
 *   packed stream is the low nibble of byte i, element 2i+1 the high nibble,
 *   two's complement; a trailing high nibble is 0.  Quantisation shrinks the
 *   payload but not the bitmap metadata ("UnionSparse", motivation section on
 *   the payload-to-metadata ratio).
 *
 * 2-bit values (USW_VAL_I2, IE-BME union format only; the W2 payload of
 *   "UnionSparse", kernel-level W2A4 analysis, weight-only like INT4): the
 *   same rule with 2 bits, scale[m] = fp16_rne(max|w| / 1) and
 *   q = clamp(round_half_even(w / scale[m]), -2, 1).  Element 4i + j of the
 *   packed stream is bits 2j, 2j+1 of byte i (two's complement); trailing
 *   bits are 0.
 *
 * Layouts of the product: X is [N][K] fp16 row-major (one row per token, the
 * transposed activation tile the pages stage), Y is [N][M] row-major, fp16
 * (rounded to nearest even from the fp32 accumulator) or fp32.
 *
 * Ownership: the caller allocates and owns every buffer.  The library keeps
 * no pointer after a call returns and never allocates or frees caller memory.
 * usw_fmt is a non-owning view.
 *
 * Errors: every entry point returns a usw_status; argument errors are
 * reported before anything is written or launched.  Device faults surface at
 * the next synchronisation of the stream, as for any HIP launch.  Nothing is
 * printed and no exception crosses this interface.  All entry points are
 * re-entrant; concurrent calls must not share output or workspace buffers.
 */
#ifndef USW_H
#define USW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define USW_ABI_VERSION 1

typedef int32_t usw_status;
#define USW_OK 0
#define USW_ERR_NULL_ARG (-1)     /* a required pointer is NULL */
#define USW_ERR_BAD_SHAPE (-2)    /* M, K not positive multiples of gt_m, gt_k; gt_* not multiples of 16 */
#define USW_ERR_BAD_DTYPE (-3)    /* unknown val_type or y_type */
#define USW_ERR_BAD_N (-4)        /* N < 1 */
#define USW_ERR_UNSUPPORTED (-5)  /* valid request with no kernel for it (e.g. a GroupTile other than 64x64) */
#define USW_ERR_MISALIGNED (-6)   /* a device pointer is not 16-byte aligned */
#define USW_ERR_WORKSPACE (-7)    /* workspace NULL or smaller than usw_spmm_workspace() reports */
#define USW_ERR_CORRUPT (-8)      /* usw_validate: offsets disagree with the bitmaps */
#define USW_ERR_HIP (-9)          /* a HIP launch or query failed */
#define USW_ERR_CAPACITY (-10)    /* an output buffer is smaller than required, or NNZ >= 2^32 */

#define USW_VAL_F16 1             /* fp16 values */
#define USW_VAL_I4 2              /* INT4 values + fp16 per-row scales */
#define USW_VAL_I2 3              /* 2-bit values + fp16 per-row scales (IE-BME union format only) */
#define USW_OUT_F16 1             /* Y in fp16 */
#define USW_OUT_F32 3             /* Y in fp32 */

/* Non-owning view of one encoded matrix.  For usw_spmm every pointer is a
 * device pointer; for usw_validate every pointer is a host pointer. */
typedef struct usw_fmt {
  int32_t M, K;             /* W is M x K */
  int32_t gt_m, gt_k;       /* GroupTile shape */
  int32_t val_type;         /* USW_VAL_F16 or USW_VAL_I4 */
  int32_t reserved;         /* must be 0 */
  int64_t nnz;              /* number of kept elements = offsets[NGT] */
  const uint64_t* bitmaps;  /* [M*K/64] */
  const uint32_t* offsets;  /* [NGT+1] */
  const void* values;       /* F16: uint16 bits [NNZ]; I4: uint8 [ceil(NNZ/2)]; see usw_encode_query for padding */
  const uint16_t* scales;   /* I4: fp16 bits [M]; F16: ignored (may be NULL) */
} usw_fmt;

/* Version of this interface (USW_ABI_VERSION). */
int32_t usw_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* usw_status_str(usw_status s);

/*
 * Sizes of an encoding, computed from the mask alone (host memory).
 *   W:    fp16 bits [M][K] row-major; read only when mask is NULL.
 *   mask: uint8 [M][K] row-major, nonzero = kept; NULL means "kept where W is
 *         nonzero in IEEE terms" (+0 and -0 dropped, NaN kept).
 * Outputs (each may be NULL if not wanted):
 *   nnz, and byte sizes of bitmaps (8*NBT), offsets (4*(NGT+1)), values
 *   (logical: 2*NNZ for F16, ceil(NNZ/2) for I4), values_alloc (the size the
 *   values buffer must have for usw_spmm: the logical size rounded down to a
 *   multiple of 16, plus 16; the kernels read whole 16-byte chunks), scales
 *   (2*M for I4, 0 for F16).
 * Errors: NULL_ARG (W and mask both NULL), BAD_SHAPE, BAD_DTYPE, CAPACITY
 * (NNZ does not fit the 32-bit offsets).
 */
usw_status usw_encode_query(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K,
                            int32_t gt_m, int32_t gt_k, int32_t val_type, int64_t* nnz,
                            size_t* bytes_bitmaps, size_t* bytes_offsets, size_t* bytes_values,
                            size_t* bytes_values_alloc, size_t* bytes_scales);

/*
 * Encode W (host memory) into caller-allocated host buffers, following the
 * TCA-BME construction above (blog section "How TCA-BME addresses the indexing
 * overhead"; INT4 rule in the header comment).  The mask is authoritative: a
 * kept exact zero sets its bit and stores its bit pattern.
 *   W:      fp16 bits [M][K] (required).
 *   mask:   uint8 [M][K] or NULL (see usw_encode_query).
 *   bitmaps [NBT], offsets [NGT+1]: outputs.
 *   values: output of values_capacity bytes (>= the logical size); bytes past
 *           the logical size up to values_capacity are zeroed.
 *   scales: output fp16 [M] for I4; ignored for F16.
 * Deterministic: the same input always gives the same bytes.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, CAPACITY.
 */
usw_status usw_encode(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t gt_m,
                      int32_t gt_k, int32_t val_type, uint64_t* bitmaps, uint32_t* offsets, void* values,
                      size_t values_capacity, uint16_t* scales);

/*
 * Check a host copy of an encoding: shape fields, offsets[0] = 0,
 * non-decreasing offsets, offsets[NGT] = nnz, and each GroupTile's offset span
 * equal to the popcount of its bitmaps.  Errors: NULL_ARG, BAD_SHAPE,
 * BAD_DTYPE, CORRUPT.
 */
usw_status usw_validate(const usw_fmt* host_fmt);

/*
 * On-device TCA-BME encoder, for a W already in GPU memory (the same
 * construction and the same bytes as usw_encode; blog section "How TCA-BME
 * addresses the indexing overhead").  Two calls, because the caller sizes
 * the values buffer from NNZ in between:
 *
 * usw_encode_device_index: bitmaps, GroupTile offsets and, for I4, the
 * per-row scales.
 *   W:       device fp16 bits [M][K] row-major, 16-byte aligned (required).
 *   mask:    device uint8 [M][K] row-major, 8-byte aligned, or NULL (kept
 *            where W is nonzero in IEEE terms, as usw_encode_query).
 *   bitmaps: device output [NBT]; offsets: device output [NGT+1], 4-byte
 *            aligned, ending in offsets[NGT] = NNZ; scales: device output
 *            fp16 [M] for I4 (ignored for F16).
 *   stream:  a hipStream_t (NULL = the default stream); the call only
 *            enqueues work.  Read offsets[NGT] after the stream reaches it.
 * Errors: NULL_ARG, BAD_SHAPE (as usw_encode, and M*K >= 2^32), BAD_DTYPE,
 * UNSUPPORTED (a GroupTile of more than 64 BitmapTiles, i.e. gt_m*gt_k >
 * 4096), MISALIGNED, HIP.
 */
usw_status usw_encode_device_index(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t gt_m,
                                   int32_t gt_k, int32_t val_type, uint64_t* bitmaps, uint32_t* offsets,
                                   uint16_t* scales, void* stream);

/*
 * usw_encode_device_values: the values of the encoding, from W and the
 * bitmaps, offsets and scales that usw_encode_device_index wrote (mask not
 * needed: the bitmaps carry it).
 *   nnz:    offsets[NGT] as read back by the caller.
 *   values: device output of values_capacity bytes, 16-byte aligned; at least
 *           the logical size (2*NNZ for F16, ceil(NNZ/2) for I4), with the
 *           size usw_encode_query calls values_alloc for use by usw_spmm.
 *           Bytes past the logical size are zeroed.
 * Writes stay below the logical size even when nnz disagrees with offsets.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, UNSUPPORTED, CAPACITY (nnz
 * negative or above M*K, or values_capacity below the logical size),
 * MISALIGNED, HIP.
 */
usw_status usw_encode_device_values(const uint16_t* W, int32_t M, int32_t K, int32_t gt_m, int32_t gt_k,
                                    int32_t val_type, const uint64_t* bitmaps, const uint32_t* offsets,
                                    const uint16_t* scales, int64_t nnz, void* values, size_t values_capacity,
                                    void* stream);

/*
 * Workspace bytes usw_spmm needs for this matrix and N (0 when none).  The
 * workspace starts with 32-bit counters (usw_spmm_counter_bytes of them,
 * one per output tile) followed by the fp32 partial sums of the workgroups
 * that share an output tile; for the 512-token prefill kernel (N > 256) a
 * copy of X in the order of its matrix-core fragments follows (N rounded up
 * to 512, times K, fp16), written by the call itself before the product.
 * The counter bytes must be zero when a call starts: allocate
 * the workspace zero-filled; every call leaves its counter bytes zero again.
 * A workspace last used by a call with a different counter size (another M,
 * or N on the other side of 32, or another prefill token tiling) may hold
 * partial sums there: zero the new call's counter bytes before it.
 * Errors: as usw_spmm's argument checks.
 */
usw_status usw_spmm_workspace(const usw_fmt* fmt, int32_t N, size_t* bytes);

/*
 * Y = W_sp . X on the GPU, for W_sp given by fmt (device pointers).
 *   X:  device fp16 bits [N][K] row-major, 16-byte aligned.
 *   Y:  device [N][M] row-major, fp16 (y_type USW_OUT_F16) or fp32
 *       (USW_OUT_F32), 16-byte aligned; fully overwritten.
 *   ws: device workspace of ws_bytes >= usw_spmm_workspace(fmt, N); may be
 *       NULL when that size is 0.  Its first usw_spmm_counter_bytes(fmt, N,
 *       0) bytes are the per-tile counters and must be zero when the call
 *       starts (the call leaves them zero again); the bytes after them need
 *       not be initialised.  A workspace whose counters are not zero gives
 *       wrong Y without an error.  Calls that may run at the same time (on
 *       different streams) need separate workspaces.
 *   stream: a hipStream_t (NULL = the default stream).  The call only
 *       enqueues work; it returns before the kernels finish.
 * Accumulation is fp32 (each product of two fp16 values is exact in fp32);
 * the result is deterministic: the same inputs give the same bits.
 * Kernels: fp16 values with N <= 128 take the decode kernels, in passes of
 * up to 64 tokens (one pass for N <= 64), N > 128 the prefill (MFMA)
 * kernels (tiles of 256 tokens up to N = 256, of 512 above); INT4 values
 * take the INT4 decode kernel, in passes of up to 64 tokens, for any N.
 * The 512-token prefill kernel returns UNSUPPORTED when N rounded up to 512,
 * times K, reaches 2^36.
 * The values buffer must hold the padded size usw_encode_query reports.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, BAD_N, UNSUPPORTED, MISALIGNED,
 * WORKSPACE, HIP.
 */
usw_status usw_spmm(const usw_fmt* fmt, const uint16_t* X, void* Y, int32_t y_type, int32_t N, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * As usw_spmm_workspace / usw_spmm, with the split-K factor chosen by the
 * caller: splits = workgroups that share one output tile (a 64-row strip of
 * GroupTiles, with all N columns for the decode kernel, or 256 / 512 of them
 * for the prefill kernel), each summing a contiguous range of GroupTile
 * columns.  With a factor above 1 each workgroup writes fp32 partial sums to
 * the workspace and the last workgroup of a tile to finish adds them in
 * split order, so results do not depend on scheduling.  The factor is
 * clamped to [ceil(K / (64 * 4 * 63)), max(1, K / 256)] for the decode
 * kernels (lower bound ceil(K / (64 * 63)) for fp16 values at most 55%
 * dense with N <= 16, whose workgroups stream their whole range together)
 * and to [ceil(K / 65536), K / 64] for the prefill kernel.
 * splits = 0 is the automatic choice of usw_spmm: for the prefill kernel
 * with N > 256 and K <= 65536 that is a stream-K split, in which each
 * workgroup (one per compute unit, or fewer for small problems) runs the
 * same number of GroupTile columns -- whole tiles and an even share of the
 * columns of the tiles left over -- and the tiles shared by several
 * workgroups are summed in a fixed order as above.
 * Same errors as usw_spmm.  Meant for tuning and tests.
 */
usw_status usw_spmm_workspace_ex(const usw_fmt* fmt, int32_t N, int32_t splits, size_t* bytes);

/*
 * Bytes at the start of the workspace of usw_spmm_ex(fmt, N, splits) that
 * hold its per-tile counters and must be zero when the call starts (0 when
 * the call needs no workspace).  Same errors as usw_spmm_workspace_ex.
 */
usw_status usw_spmm_counter_bytes(const usw_fmt* fmt, int32_t N, int32_t splits, size_t* bytes);
usw_status usw_spmm_ex(const usw_fmt* fmt, const uint16_t* X, void* Y, int32_t y_type, int32_t N, int32_t splits,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * usw_spmm_ex without a caller workspace and without any allocation, for
 * callers that cannot allocate device memory around the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same fmt, X, Y, y_type, N, splits and stream conventions and the same
 * kernels and results as usw_spmm_ex.  The split-K counters and partial
 * sums live in a library-owned device array of 16 MiB per GPU (16 KiB of
 * counters, the rest partial sums), created with the library's code object
 * on each GPU it runs on and kept until the process ends.  Each call first
 * clears the counters it uses with a small kernel on the stream, then
 * launches the product; it never calls hipMalloc or hipFree.  splits = 0 is
 * usw_spmm's automatic factor, or 1 when that factor's partial sums do not
 * fit the array (e.g. the prefill kernel's stream-K split).  With splits 0
 * or 1, N > 256 takes the 256-token prefill kernel (no workspace at one
 * split) when the 512-token kernel's copy of X does not fit the array.
 * Every call on one GPU shares that GPU's array: calls that may overlap in
 * time on one GPU (on different streams) race and give wrong Y; order them
 * on one stream, or use usw_spmm_ex with separate workspaces.
 * Errors: as usw_spmm_ex, plus WORKSPACE when the call's counters or
 * partial sums (usw_spmm_counter_bytes, usw_spmm_workspace_ex) exceed the
 * array, UNSUPPORTED for a device index of 64 or more, HIP when the array's
 * address cannot be taken on the current device.
 */
usw_status usw_spmm_noalloc(const usw_fmt* fmt, const uint16_t* X, void* Y, int32_t y_type, int32_t N,
                            int32_t splits, void* stream);

/*
 * ---------------------------------------------------------------------------
 * IE-BME union-mask low-bit format ("UnionSparse: An Index-Efficient Sparsity
 * Framework for Low-Bit Sparse LLM Inference on Edge", section on IE-BME; the
 * gather follows its LSPD section).
 *
 *   - Local tile (LT): lt_m x lt_k weights; LTs of the matrix stored
 *     row-major.  An LT is cut into an r_a x c_a grid of areas of
 *     (lt_m/r_a) x (lt_k/c_a), Q = r_a * c_a; area q = a_r * c_a + a_c.
 *   - Union mask: bit (i, j) of an LT is set when any of the Q weights
 *     W[a_r lt_m/r_a + i][a_c lt_k/c_a + j] of the LT is kept.  It is scanned
 *     row-major and packed into uint64 words, least significant bit first;
 *     (lt_m/r_a) (lt_k/c_a) must be a multiple of 64, so each LT owns
 *     NW = lt_m lt_k / (64 Q) whole words.  bitmaps[NLT * NW].
 *   - offsets[NLT+1]: uint32 payload-element index of each LT's payload,
 *     offsets[t+1] = offsets[t] + Q * P_t with P_t the LT's set union bits.
 *   - values: per LT, Q streams of P_t elements one after the other; the
 *     element of area q at the active position of compact rank r (active
 *     positions before it, row-major) is values[offsets[t] + q P_t + r].  A
 *     pruned weight of an active group is stored as 0.  INT4 elements are
 *     packed and quantised as above (per-row scales over the kept weights).
 * The mask is authoritative, as for usw_encode.  Activations stay fp16.
 * ---------------------------------------------------------------------------
 */

/* Non-owning view of one IE-BME encoding (device pointers for usw_union_spmm,
 * host pointers for usw_union_validate). */
typedef struct usw_union_fmt {
  int32_t M, K;             /* W is M x K */
  int32_t lt_m, lt_k;       /* LT shape */
  int32_t r_a, c_a;         /* area grid of an LT */
  int32_t val_type;         /* USW_VAL_I4 or USW_VAL_I2 (USW_VAL_F16 for host-side use only) */
  int32_t reserved;         /* must be 0 */
  int64_t payload;          /* stored payload elements = offsets[NLT] */
  const uint64_t* bitmaps;  /* [NLT * NW] */
  const uint32_t* offsets;  /* [NLT+1] */
  const void* values;       /* I4: uint8 [ceil(payload/2)], I2: [ceil(payload/4)], padded as
                               usw_union_encode_query says */
  const uint16_t* scales;   /* I4, I2: fp16 bits [M], one per row of W */
  const uint8_t* rowmap;    /* reordered LTs: [NLT * lt_m], entry t * lt_m + r = the stored row of LT t
                               that holds the LT's row r of W (usw_union_encode_reordered); NULL: every
                               LT stores its rows in order */
} usw_union_fmt;

/*
 * Sizes of an IE-BME encoding from the mask alone (host memory); arguments as
 * usw_encode_query plus the LT shape and area grid.  payload = sum of Q P_t.
 * values_alloc is the logical size rounded down to 16 bytes, plus 16.
 * Errors: NULL_ARG, BAD_SHAPE (M, K not multiples of lt_m, lt_k; lt_m, lt_k
 * not multiples of r_a, c_a; an area position count not a multiple of 64),
 * BAD_DTYPE, CAPACITY (payload >= 2^32).
 */
usw_status usw_union_encode_query(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                                  int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type, int64_t* payload,
                                  size_t* bytes_bitmaps, size_t* bytes_offsets, size_t* bytes_values,
                                  size_t* bytes_values_alloc, size_t* bytes_scales);

/*
 * Encode W (host memory) into caller-allocated host buffers following the
 * IE-BME construction above.  Buffers as usw_encode; values_capacity bytes
 * of values are written (zero past the logical size).  Deterministic.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, CAPACITY.
 */
usw_status usw_union_encode(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                            int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type, uint64_t* bitmaps,
                            uint32_t* offsets, void* values, size_t values_capacity, uint16_t* scales);

/*
 * Check a host copy of an IE-BME encoding: shape fields, offsets[0] = 0,
 * offsets[NLT] = payload, each LT's span equal to Q times the popcount of
 * its union words, and (when present) each LT's rowmap a permutation of its
 * rows.  Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, CORRUPT.
 */
usw_status usw_union_validate(const usw_union_fmt* host_fmt);

/*
 * IE-BME encoding of W with the rows of every LT rearranged before
 * compression, as bitmap-aware row reordering prescribes ("UnionSparse",
 * section on bitmap-aware row reordering: Objective, Practical Effect): the
 * values of the surviving weights do not change, only which row of its LT
 * each sits in.
 *   perm:   host int32 [NLT * lt_m]; stored row s of LT t holds the LT's row
 *           perm[t * lt_m + s] of W (the order usw_union_reorder returns).
 *           Each LT's entries must be a permutation of 0 .. lt_m - 1.
 * The union words, offsets and area streams are those of usw_union_encode
 * applied to each LT with its rows so arranged.  INT4 scales and codes come
 * from the rows of W (quantisation precedes reordering), scales[m] for row m.
 *   rowmap: host output uint8 [NLT * lt_m], the inverse of perm per LT
 *           (rowmap[t * lt_m + perm[t * lt_m + s]] = s), for usw_union_fmt.
 * The query returns the payload and the value bytes (logical, padded); the
 * other buffers have usw_union_encode_query's sizes.  Other arguments as
 * usw_union_encode.  Errors: NULL_ARG (also perm or rowmap NULL), BAD_SHAPE
 * (as usw_union_encode_query; lt_m > 256; perm not a permutation per LT),
 * BAD_DTYPE, CAPACITY.
 */
usw_status usw_union_encode_reordered_query(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K,
                                            int32_t lt_m, int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type,
                                            const int32_t* perm, int64_t* payload, size_t* bytes_values,
                                            size_t* bytes_values_alloc);
usw_status usw_union_encode_reordered(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                                      int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type, const int32_t* perm,
                                      uint64_t* bitmaps, uint32_t* offsets, void* values, size_t values_capacity,
                                      uint16_t* scales, uint8_t* rowmap);

/*
 * On-device IE-BME encoder for a W already in GPU memory: the same bytes as
 * usw_union_encode for INT4 and 2-bit payloads (val_type USW_VAL_I4 or
 * USW_VAL_I2; rows in natural order).  Two calls, as for the TCA-BME device
 * encoder:
 *
 * usw_union_encode_device_index: union words, LT offsets (offsets[NLT] =
 * payload) and per-row scales.
 *   W:       device fp16 bits [M][K], 16-byte aligned (required).
 *   mask:    device uint8 [M][K], 8-byte aligned, or NULL (IEEE nonzeros).
 *   bitmaps: device output [NLT * NW]; offsets: device output [NLT+1],
 *            4-byte aligned; scales: device output fp16 [M] (the b-bit rule
 *            of the val_type).
 *
 * usw_union_encode_device_values: the Q aligned code streams of every LT,
 * from W, the mask (a pruned weight of an active group is stored as 0) and
 * what the first call wrote.
 *   payload: offsets[NLT] as read back by the caller.
 *   values:  device output of values_capacity >= ceil(payload / 2) bytes
 *            (INT4) or ceil(payload / 4) bytes (2-bit),
 *            16-byte aligned; bytes past the logical size are zeroed.  Writes
 *            stay below the logical size even when payload disagrees with
 *            offsets.
 * Both: stream as for usw_spmm.  Errors: NULL_ARG, BAD_SHAPE (as
 * usw_union_encode_query, and M*K >= 2^32), BAD_DTYPE, UNSUPPORTED (fp16
 * payload, LTs of more than 4096 elements, area rows not a multiple of 8
 * positions), CAPACITY (values only: payload negative or above M*K,
 * values_capacity too small), MISALIGNED, HIP.
 */
usw_status usw_union_encode_device_index(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                                         int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type,
                                         uint64_t* bitmaps, uint32_t* offsets, uint16_t* scales, void* stream);
usw_status usw_union_encode_device_values(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K,
                                          int32_t lt_m, int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type,
                                          const uint64_t* bitmaps, const uint32_t* offsets, const uint16_t* scales,
                                          int64_t payload, void* values, size_t values_capacity, void* stream);

/*
 * Bitmap-aware row reordering of the LTs ("UnionSparse", section on
 * bitmap-aware row reordering), an offline step before usw_union_encode.
 * Each LT (row-major order) is solved independently: its rows are split
 * into groups of r_a minimising the active union-mask entries (a group's
 * grouped columns j where any of its rows is kept in any of the c_a column
 * partitions), by the subset DP over the set of ungrouped rows that always
 * places the smallest one.  Ties go to the first minimum with the other rows
 * of a group in lexicographic order.  Groups are canonicalised (rows
 * ascending, groups lexicographic) and laid out partition-wise.
 *   W, mask:  host, as usw_union_encode_query (the mask decides what is kept).
 *   perm:     output int32 [NLT][lt_m]: perm[t*lt_m + i] is the LT-local row
 *             of LT t to place at row i (row p*(lt_m/r_a) + g holds the p-th
 *             row of group g).
 *   actives_before, actives_after: optional outputs int32 [NLT]: active
 *             union-mask entries of each LT as given and after its
 *             permutation (the DP minimum).
 * The DP is exponential in lt_m: LTs of at most 20 rows are accepted.  The
 * orders feed usw_union_encode_reordered, whose encoding (16-row LTs)
 * usw_union_spmm multiplies back onto the rows of W.
 * Errors: NULL_ARG (perm NULL, or W and mask both NULL), BAD_SHAPE (as
 * usw_union_encode_query), UNSUPPORTED (lt_m > 20).
 */
usw_status usw_union_reorder(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                             int32_t lt_k, int32_t r_a, int32_t c_a, int32_t* perm, int32_t* actives_before,
                             int32_t* actives_after);

/*
 * Workspace bytes and counter bytes of usw_union_spmm for this matrix, N and
 * split factor (splits = 0: automatic; otherwise clamped to
 * [ceil(K / (64 * 4 * (lt_m - 1))), max(1, K / 256)]).  The workspace starts with
 * the counter bytes, which must be zero when a call starts (each call leaves
 * them zero), then fp32 partial sums, which need not be initialised.  A
 * workspace whose counters are not zero gives wrong Y without an error;
 * calls that may run at the same time need separate workspaces.
 * Errors: as usw_union_spmm's checks.
 */
usw_status usw_union_spmm_workspace(const usw_union_fmt* fmt, int32_t N, int32_t splits, size_t* bytes);
usw_status usw_union_spmm_counter_bytes(const usw_union_fmt* fmt, int32_t N, int32_t splits, size_t* bytes);

/*
 * Y = W_sp . X on the GPU from an IE-BME encoding (device pointers), with the
 * same X, Y, workspace and stream conventions as usw_spmm, in passes of up
 * to 32 tokens (64 for 2 x 2 grids on 64 x 64 LTs without a rowmap).  The
 * kernels take INT4 or 2-bit values on LTs of 16, 32 or
 * 64 rows by 64 columns (M a multiple of 64), any area grid the format
 * allows with areas at least 8 columns wide (c_a <= 8), and a rowmap or none.
 * The section illustrates R_A = C_A = 2 and states the LSPD gather for a
 * general grid; 2 x 2 grids on 64 x 64 LTs (no rowmap) and on 16 x 64 LTs
 * run on kernels specialised for them, every other grid on one that takes
 * the grid at run time.  Each lane reads the rank of the union-mask byte it
 * needs once and gathers its row of every area stream with it (the LSPD
 * gather); with a rowmap it rebuilds the row of W it holds in the product
 * from the stored row the rowmap names, so every LT's products land on the
 * rows of W.  fp32 accumulation, deterministic.  Errors: NULL_ARG,
 * BAD_SHAPE, BAD_DTYPE, BAD_N, UNSUPPORTED (fp16 values, lt_k other than 64,
 * lt_m other than 16, 32 or 64, M not a multiple of 64, c_a > 8),
 * MISALIGNED, WORKSPACE, HIP.  The rowmap is not checked here
 * (usw_union_validate does).
 */
usw_status usw_union_spmm(const usw_union_fmt* fmt, const uint16_t* X, void* Y, int32_t y_type, int32_t N,
                          int32_t splits, void* ws, size_t ws_bytes, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Tiled-CBC and the dynamically pruned spMspV ("Unified Static-Dynamic
 * Pruning for Efficient LLM Inference", section 4.1 Tiled-CBC and section
 * 4.2 decode phase).
 *
 *   - GTile: 256 x 16 weights; GTiles of the matrix stored row-major.  A
 *     GTile is 16 column tiles of 256 x 1.
 *   - bitmaps[NGT * 16 * 4]: per column tile, 4 uint64 words; bit i of word
 *     j <-> row 64 j + i of the column, least significant bit first.
 *   - values: fp16 bits of the kept weights column by column (rows top to
 *     bottom), each column's run padded with +0.0 to a multiple of 8 values
 *     (16 bytes).
 *   - tile_offsets[NGT+1]: uint32 index of each GTile's first value
 *     (tile_offsets[NGT] = nnz_padded); colinfo[NGT * 16]: per column, its
 *     run's offset inside the GTile (upper 16 bits) and its kept count
 *     (lower 16 bits).
 *   Storage 4 (NGT+1) + 4 NGT 16 + 8 NBM + 2 nnz_padded bytes (the section's
 *   equation, NNZ counting the padded runs).
 * Dynamic pruning: column k takes part when |x_k| >= tau, compared in fp32;
 * the product is y = sum over those k of W_sp[:, k] x_k, fp32 accumulation.
 * ---------------------------------------------------------------------------
 */

/* Non-owning view of one Tiled-CBC encoding (device pointers for
 * usw_cbc_spmspv, host pointers for usw_cbc_validate). */
typedef struct usw_cbc_fmt {
  int32_t M, K;                 /* W is M x K, multiples of 256 and 16 */
  int32_t tile_m, tile_k;       /* 256, 16 */
  int32_t val_type;             /* USW_VAL_F16 */
  int32_t reserved;             /* must be 0 */
  int64_t nnz_padded;           /* stored values = tile_offsets[NGT] */
  const uint64_t* bitmaps;      /* [NGT * 64] */
  const uint32_t* tile_offsets; /* [NGT+1] */
  const uint32_t* colinfo;      /* [NGT * 16] */
  const uint16_t* values;       /* [nnz_padded] fp16 bits, 16-byte aligned */
} usw_cbc_fmt;

/*
 * Sizes of a Tiled-CBC encoding from the mask alone (host memory); W and
 * mask as usw_encode_query.  Outputs (each may be NULL): kept count, padded
 * count, byte sizes of bitmaps, tile_offsets, colinfo and values.
 * Errors: NULL_ARG, BAD_SHAPE (M not a multiple of 256 or K of 16),
 * CAPACITY (padded count >= 2^32).
 */
usw_status usw_cbc_encode_query(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int64_t* nnz,
                                int64_t* nnz_padded, size_t* bytes_bitmaps, size_t* bytes_tile_offsets,
                                size_t* bytes_colinfo, size_t* bytes_values);

/*
 * Encode W (host memory) into caller-allocated host buffers following the
 * Tiled-CBC construction above; values_capacity must be at least the values
 * size usw_cbc_encode_query reports.  Deterministic.
 * Errors: NULL_ARG, BAD_SHAPE, CAPACITY.
 */
usw_status usw_cbc_encode(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, uint64_t* bitmaps,
                          uint32_t* tile_offsets, uint32_t* colinfo, uint16_t* values, size_t values_capacity);

/*
 * Check a host copy of a Tiled-CBC encoding: shape fields, tile offsets
 * framing the values, and every ColInfo entry agreeing with its column's
 * bitmap words and with the padded runs before it.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, CORRUPT.
 */
usw_status usw_cbc_validate(const usw_cbc_fmt* host_fmt);

/*
 * On-device Tiled-CBC encoder for a W already in GPU memory: the same bytes
 * as usw_cbc_encode ([SPDP] section 4.1 layout above).  Two calls:
 *
 * usw_cbc_encode_device_index: bitmaps, ColInfo and TileOffsets
 * (tile_offsets[NGT] = nnz_padded when the stream reaches it).
 *   W:    device fp16 bits [M][K], 16-byte aligned (required).
 *   mask: device uint8 [M][K], 16-byte aligned, or NULL (IEEE nonzeros).
 *   bitmaps [NGT * 64], tile_offsets [NGT+1], colinfo [NGT * 16]: device
 *   outputs (8-, 4- and 4-byte aligned).
 *
 * usw_cbc_encode_device_values: the padded column runs, from W and what the
 * first call wrote (the mask is not needed: the bitmaps carry it).
 *   nnz_padded: tile_offsets[NGT] as read back by the caller.
 *   values: device output of values_capacity >= 2 * nnz_padded bytes,
 *           16-byte aligned; whole fp16 elements past the runs are zeroed.
 *           Writes stay below nnz_padded elements even when it disagrees with
 *           tile_offsets.
 * Both: stream as for usw_spmm.  Errors: NULL_ARG, BAD_SHAPE (as
 * usw_cbc_encode_query, and M*K >= 2^32), CAPACITY (values only), MISALIGNED,
 * HIP.
 */
usw_status usw_cbc_encode_device_index(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K,
                                       uint64_t* bitmaps, uint32_t* tile_offsets, uint32_t* colinfo, void* stream);
usw_status usw_cbc_encode_device_values(const uint16_t* W, int32_t M, int32_t K, const uint64_t* bitmaps,
                                        const uint32_t* tile_offsets, const uint32_t* colinfo, int64_t nnz_padded,
                                        uint16_t* values, size_t values_capacity, void* stream);

/*
 * Workspace bytes and leading counter bytes of usw_cbc_spmspv for this
 * matrix and split factor (splits = 0: automatic; otherwise clamped to
 * [1, K / 16]).  The counter bytes must be zero when a call starts; each
 * call leaves them zero.  The partial sums after them need not be
 * initialised.  A workspace whose counters are not zero gives wrong y
 * without an error; calls that may run at the same time need separate
 * workspaces.  Errors: as usw_cbc_spmspv's checks.
 */
usw_status usw_cbc_spmspv_workspace(const usw_cbc_fmt* fmt, int32_t splits, size_t* bytes, size_t* counter_bytes);

/*
 * y = W_sp x with dynamic pruning on the GPU (N = 1, the section's
 * spMspV): columns with |x_k| < tau are skipped, their bitmaps and values
 * are not read.  x: device fp16 bits [K], y: device [M] fp16 (y_type
 * USW_OUT_F16, rounded to nearest even from fp32) or fp32, both 16-byte
 * aligned; tau >= 0 (tau = 0 keeps every column).  fp32 accumulation;
 * deterministic (split partial sums added in split order).
 * Errors: NULL_ARG, BAD_SHAPE (also M > 2^28 or 2 nnz_padded >= 2^31 - 16
 * bytes), BAD_DTYPE, UNSUPPORTED (tile shape other than 256 x 16, values
 * other than fp16, tau negative or NaN), MISALIGNED, WORKSPACE, HIP.
 */
usw_status usw_cbc_spmspv(const usw_cbc_fmt* fmt, const uint16_t* x, void* y, int32_t y_type, float tau,
                          int32_t splits, void* ws, size_t ws_bytes, void* stream);

/*
 * Measurement utility, not part of the SpMM path: reads the first
 * bytes / 16 * 16 bytes of the device buffer buf once (16-byte loads,
 * non-temporal) on the stream, so that a caller can time the GPU's
 * streaming-read rate, the practical ceiling of the memory-bound SpMM.
 *   buf:  device pointer, 16-byte aligned.
 *   sink: device buffer of at least one uint32 word; the kernel may write it
 *         (its value carries no meaning).
 * Errors: NULL_ARG, MISALIGNED, BAD_SHAPE (more than 2^31 - 1 blocks of
 * 8 KB), HIP.
 */
usw_status usw_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* USW_H */
