// Device-side encoders for weights already in GPU memory, each writing the
// same bytes as its host counterpart: TCA-BME (usw_encode; this header's
// passes below), IE-BME union-mask INT4 or 2-bit (usw_union_encode) and
// Tiled-CBC (usw_cbc_encode), the last two in their own sections further
// down.  All three share the in-place scan, the b-bit row-scale kernel and
// the tail zeroing.
//
// Format: blog "SpInfer: How bitmaps make sparse LLMs actually fast", section
// "How TCA-BME addresses the indexing overhead" (8x8 BitmapTiles in one
// 64-bit word, 2x2 of them per 16x16 TCTile, TCTiles row-major in a
// GroupTile; Values in that tile order; one offset per GroupTile).  INT4
// values follow the round-to-nearest rule of usw_quant.h.
//
// Passes, in order on one stream:
//   1. index:  one wave per GroupTile, one BitmapTile per lane.  The lane
//      reads its 8 rows of 8 weights (one 16-byte load per row, or 8 mask
//      bytes), writes the 64-bit bitmap, and the wave's popcount goes to
//      offsets[g] as a count.
//   2. scan:   one workgroup turns the counts in offsets[0..NGT) into the
//      exclusive prefix offsets[0..NGT] in place.
//   3. scales (INT4, 2-bit): one wave per row: the largest kept magnitude
//      as sign-cleared fp16 bits, then int_scale_bits for the code width.
//   4. values: one wave per GroupTile: lane j ranks the kept weights of its
//      BitmapTile from the bitmap (the wave's exclusive popcount prefix plus
//      the position inside the tile) and stages the fp16 bits, or the INT4
//      codes, in LDS in storage order; the wave then writes the GroupTile's
//      run with consecutive lanes on consecutive elements.  INT4 byte b
//      (codes 2b and 2b + 1) is written by the GroupTile that holds code 2b;
//      when its run ends on an even code, the wave quantises the first kept
//      weight of the next non-empty GroupTile for the high nibble.
//   5. the values buffer past the logical size is zeroed.
// Every pass is bound by HBM: W is read once by pass 1 (the mask instead
// when one is given), once more by pass 3 for INT4, and pass 4 reads the
// 16-byte rows that hold kept weights.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "usw.h"
#include "usw_device.h"
#include "usw_internal.h"
#include "usw_quant.h"

namespace {

constexpr int kEThreads = 256;   // four waves, one GroupTile (or row) each
constexpr int kEWaves = kEThreads / 64;
constexpr int kMaxBt = 64;       // BitmapTiles per GroupTile handled by one wave

struct EncGeom {
  int K;           // row length
  int gt_m, gt_k;  // GroupTile shape
  int Gc;          // GroupTile columns
  int Tc;          // TCTiles per GroupTile row
  int bpg;         // BitmapTiles per GroupTile (<= 64)
  int ngt;         // GroupTiles
};

// Top-left element (row r0, column c0) of BitmapTile j of GroupTile gid:
// TCTile t = j / 4 (row-major in the GroupTile), BitmapTile j % 4 row-major
// in the TCTile.
__device__ inline void bt_origin(const EncGeom& g, int gid, int j, uint32_t& r0, uint32_t& c0) {
  const int gi = gid / g.Gc, gj = gid - gi * g.Gc;
  const int t = j >> 2, b = j & 3;
  const int ti = t / g.Tc, tj = t - ti * g.Tc;
  r0 = static_cast<uint32_t>(gi * g.gt_m + 16 * ti + 8 * (b >> 1));
  c0 = static_cast<uint32_t>(gj * g.gt_k + 16 * tj + 8 * (b & 1));
}

__device__ inline uint64_t elem(const EncGeom& g, uint32_t r, uint32_t c) {
  return static_cast<uint64_t>(r) * static_cast<uint64_t>(g.K) + c;
}

__device__ inline uint64_t elem_rc(int K, int r, int c) {
  return static_cast<uint64_t>(r) * static_cast<uint64_t>(K) + static_cast<uint64_t>(c);
}

// Bit c set where fp16 weight c of the 8 is nonzero in IEEE terms (+0 and
// -0 dropped, NaN and infinities kept).
__device__ inline uint32_t nonzero8(const uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r |= static_cast<uint32_t>((w[i] & 0x7FFFu) != 0) << (2 * i);
    r |= static_cast<uint32_t>((w[i] & 0x7FFF0000u) != 0) << (2 * i + 1);
  }
  return r;
}

// Bit c set where mask byte c of the 8 is nonzero.
__device__ inline uint32_t kept8(const uint2 m) {
  uint32_t r = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    r |= static_cast<uint32_t>(((m.x >> (8 * c)) & 0xFFu) != 0) << c;
    r |= static_cast<uint32_t>(((m.y >> (8 * c)) & 0xFFu) != 0) << (c + 4);
  }
  return r;
}

__device__ inline uint16_t half_of(const uint4 v, int c) {
  const uint32_t w = c < 2 ? v.x : c < 4 ? v.y : c < 6 ? v.z : v.w;
  return static_cast<uint16_t>(w >> (16 * (c & 1)));
}

template <bool MASK>
__global__ __launch_bounds__(kEThreads) void enc_index_kernel(const uint16_t* __restrict__ W,
                                                              const uint8_t* __restrict__ mask,
                                                              uint64_t* __restrict__ bitmaps,
                                                              uint32_t* __restrict__ counts, EncGeom g) {
  const int lane = threadIdx.x & 63;
  const int gid = blockIdx.x * kEWaves + (threadIdx.x >> 6);
  if (gid >= g.ngt) return;
  uint64_t bm = 0;
  if (lane < g.bpg) {
    uint32_t r0, c0;
    bt_origin(g, gid, lane, r0, c0);
    const uint64_t at = elem(g, r0, c0);
    uint32_t rows[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const uint64_t e = at + static_cast<uint64_t>(p) * g.K;
      rows[p] = MASK ? kept8(*reinterpret_cast<const uint2*>(mask + e))
                     : nonzero8(*reinterpret_cast<const uint4*>(W + e));
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) bm |= static_cast<uint64_t>(rows[p]) << (8 * p);
    bitmaps[static_cast<uint64_t>(gid) * g.bpg + lane] = bm;
  }
  uint32_t cnt = __popcll(bm);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if (lane == 0) counts[gid] = cnt;
}

// In-place exclusive prefix sum of offsets[0..n), total to offsets[n]; one
// workgroup of 1024 threads, four consecutive entries per thread per round.
__global__ __launch_bounds__(1024) void enc_scan_kernel(uint32_t* __restrict__ offsets, int n) {
  __shared__ uint32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t carry = 0;
  for (int base = 0; base < n; base += 4096) {
    const int i0 = base + 4 * tid;
    uint32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = i0 + k < n ? offsets[i0 + k] : 0u;
    const uint32_t s = v[0] + v[1] + v[2] + v[3];
    uint32_t inc = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    if (lane == 63) wsum[w] = inc;
    __syncthreads();
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const uint32_t x = wsum[q];
      before += q < w ? x : 0u;
      total += x;
    }
    uint32_t run = carry + before + inc - s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (i0 + k < n) offsets[i0 + k] = run;
      run += v[k];
    }
    carry += total;
    __syncthreads();   // wsum is rewritten by the next round
  }
  if (tid == 0) offsets[n] = carry;
}

template <bool MASK>
__global__ __launch_bounds__(kEThreads) void enc_scales_kernel(const uint16_t* __restrict__ W,
                                                               const uint8_t* __restrict__ mask,
                                                               uint16_t* __restrict__ scales, int M, int K, int qmax) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * kEWaves + (threadIdx.x >> 6);
  if (m >= M) return;
  const uint64_t row = static_cast<uint64_t>(m) * K;
  uint32_t amax = 0;
  for (int c = 8 * lane; c < K; c += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(W + row + c);
    const uint32_t keep = MASK ? kept8(*reinterpret_cast<const uint2*>(mask + row + c)) : nonzero8(v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t a = half_of(v, i) & 0x7FFFu;
      if ((keep >> i) & 1u) amax = a > amax ? a : amax;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t t = __shfl_xor(amax, o);
    amax = t > amax ? t : amax;
  }
  if (lane == 0) scales[m] = usw::int_scale_bits(static_cast<uint16_t>(amax), qmax);
}

// INT4 code of the first kept weight of GroupTile gid (0 when it has none).
// Wave-uniform: every lane returns the same value.
__device__ inline uint32_t first_code(const EncGeom& g, const uint16_t* W, const uint64_t* bitmaps,
                                      const uint16_t* scales, int gid, int lane) {
  const uint64_t bm = lane < g.bpg ? bitmaps[static_cast<uint64_t>(gid) * g.bpg + lane] : 0ull;
  const uint64_t any = __ballot(bm != 0);
  if (!any) return 0;
  const int f = __builtin_ctzll(any);
  const uint32_t lo = __shfl(static_cast<uint32_t>(bm), f), hi = __shfl(static_cast<uint32_t>(bm >> 32), f);
  const uint64_t word = (static_cast<uint64_t>(hi) << 32) | lo;
  const int p = __builtin_ctzll(word);
  uint32_t r0, c0;
  bt_origin(g, gid, f, r0, c0);
  const uint32_t row = r0 + (p >> 3);
  return static_cast<uint32_t>(usw::i4_code(W[elem(g, row, c0 + (p & 7))], usw::f16_to_f64(scales[row]))) & 0xFu;
}

template <bool I4>
__global__ __launch_bounds__(kEThreads) void enc_values_kernel(const uint16_t* __restrict__ W,
                                                               const uint64_t* __restrict__ bitmaps,
                                                               const uint32_t* __restrict__ offsets,
                                                               const uint16_t* __restrict__ scales,
                                                               void* __restrict__ values, EncGeom g, uint64_t nnz,
                                                               uint64_t logical) {
  // Four waves, each stages its GroupTile's run (fp16 bits, or INT4 codes)
  // in storage order.
  __shared__ uint16_t stage[kEWaves][kMaxBt * 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int gid = blockIdx.x * kEWaves + wv;
  if (gid >= g.ngt) return;
  uint16_t* st = stage[wv];
  const uint64_t o0 = offsets[gid];
  const uint64_t bm = lane < g.bpg ? bitmaps[static_cast<uint64_t>(gid) * g.bpg + lane] : 0ull;
  const uint32_t cnt = __popcll(bm);
  uint32_t inc = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  const uint32_t total = __shfl(inc, 63);
  if (bm) {
    uint32_t r0, c0;
    bt_origin(g, gid, lane, r0, c0);
    uint32_t pos = inc - cnt;
    for (int p = 0; p < 8; ++p) {
      const uint32_t byte = static_cast<uint32_t>(bm >> (8 * p)) & 0xFFu;
      if (!byte) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(W + elem(g, r0 + p, c0));
      double s = 0.0;
      if constexpr (I4) s = usw::f16_to_f64(scales[r0 + p]);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (!((byte >> c) & 1u)) continue;
        const uint16_t h = half_of(v, c);
        st[pos++] = I4 ? static_cast<uint16_t>(static_cast<uint32_t>(usw::i4_code(h, s)) & 0xFu) : h;
      }
    }
  }
  usw_dev::wave_sync();
  if constexpr (!I4) {
    // Element pairs on 4-byte boundaries go out as one 32-bit store; a
    // leading element (o0 odd) and a trailing one take 16-bit stores.
    uint16_t* out = static_cast<uint16_t*>(values);
    const uint32_t head = static_cast<uint32_t>(o0 & 1);
    if (total > head) {
      if (head && lane == 0 && o0 < nnz) out[o0] = st[0];
      const uint32_t pairs = (total - head) / 2;
      for (uint32_t j = lane; j < pairs; j += 64) {
        const uint32_t i = head + 2 * j;
        const uint64_t at = o0 + i;
        if (at + 1 < nnz)
          *reinterpret_cast<uint32_t*>(out + at) = st[i] | (static_cast<uint32_t>(st[i + 1]) << 16);
        else if (at < nnz)
          out[at] = st[i];
      }
      if (((total - head) & 1) && lane == 0 && o0 + total - 1 < nnz) out[o0 + total - 1] = st[total - 1];
    } else if (total == 1 && lane == 0 && o0 < nnz) {
      out[o0] = st[0];
    }
  } else {
    // INT4: bytes ceil(o0 / 2) .. ceil(e / 2) - 1 belong to this GroupTile.
    const uint64_t e = o0 + total;
    uint32_t next = 0;
    if (total && (e & 1) && e < nnz && gid + 1 < g.ngt) {
      // The GroupTile holding code e: the first one after gid whose run ends past e.
      int lo = gid + 1, hi = g.ngt - 1;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid + 1] > e)
          hi = mid;
        else
          lo = mid + 1;
      }
      next = first_code(g, W, bitmaps, scales, lo, lane);
    }
    uint8_t* out = static_cast<uint8_t*>(values);
    for (uint64_t b = (o0 + 1) / 2 + lane; b < (e + 1) / 2; b += 64) {
      const uint32_t lo4 = st[2 * b - o0];
      const uint32_t hi4 = 2 * b + 1 < e ? st[2 * b + 1 - o0] : next;
      if (b < logical) out[b] = static_cast<uint8_t>(lo4 | (hi4 << 4));
    }
  }
}

__global__ __launch_bounds__(kEThreads) void enc_zero_kernel(uint8_t* __restrict__ p, uint64_t n) {
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kEThreads + threadIdx.x; i < n;
       i += static_cast<uint64_t>(gridDim.x) * kEThreads)
    p[i] = 0;
}

// ---------------------------------------------------------------------------
// IE-BME union-mask encoding on the device ("UnionSparse", IE-BME: one union
// bit per area-aligned group of an LT, Q aligned streams of INT4 or 2-bit
// codes per LT, stream q of LT t at offsets[t] + q P_t, P_t the LT's active
// positions).  The same bytes as usw_union_encode for those payloads (what
// the union kernels run); reordered rows are a host-side step.
// ---------------------------------------------------------------------------

struct UnionGeom {
  int K;
  int lt_m, lt_k;
  int am, ak;       // area shape = union-mask shape
  int c_a, Q;
  int lc;           // LT columns
  int nw;           // union words per LT (<= 64)
  int nlt;
};

// Linear index in W of position p (row-major in the area) of area q of LT t.
__device__ inline uint64_t union_elem(const UnionGeom& g, int t, int q, int p) {
  const int ti = t / g.lc, tj = t - ti * g.lc;
  const int ar = q / g.c_a, ac = q - ar * g.c_a;
  const int i = p / g.ak, j = p - i * g.ak;
  return static_cast<uint64_t>(ti * g.lt_m + ar * g.am + i) * static_cast<uint64_t>(g.K) +
         static_cast<uint64_t>(tj * g.lt_k + ac * g.ak + j);
}

// Kept bits of the 8 positions p0 .. p0 + 7 (one row of an area: ak is a
// multiple of 8) of area q; v receives their fp16 bits.
template <bool MASK>
__device__ inline uint32_t union_chunk(const UnionGeom& g, const uint16_t* W, const uint8_t* mask, int t, int q,
                                       int p0, uint4& v) {
  const uint64_t e = union_elem(g, t, q, p0);
  v = *reinterpret_cast<const uint4*>(W + e);
  return MASK ? kept8(*reinterpret_cast<const uint2*>(mask + e)) : nonzero8(v);
}

// One wave per LT, lane w Q + q reads area q of union word w (positions
// 64 w .. 64 w + 63, eight rows of 8) -- nw Q <= 64 since an LT holds at
// most 4096 elements; the Q partial words are ORed through LDS by lane w Q.
// The LT's count is Q times the popcount of its words.
template <bool MASK>
__global__ __launch_bounds__(kEThreads) void union_index_kernel(const uint16_t* __restrict__ W,
                                                                const uint8_t* __restrict__ mask,
                                                                uint64_t* __restrict__ bitmaps,
                                                                uint32_t* __restrict__ counts, UnionGeom g) {
  __shared__ uint64_t part[kEWaves][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kEWaves + wv;
  if (t >= g.nlt) return;
  const int w = lane / g.Q, q = lane - w * g.Q;
  uint64_t bits = 0;
  if (w < g.nw) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint4 v;
      bits |= static_cast<uint64_t>(union_chunk<MASK>(g, W, mask, t, q, 64 * w + 8 * c, v)) << (8 * c);
    }
  }
  part[wv][lane] = bits;
  usw_dev::wave_sync();
  uint64_t word = 0;
  if (w < g.nw && q == 0) {
    for (int k = 0; k < g.Q; ++k) word |= part[wv][lane + k];
    bitmaps[static_cast<uint64_t>(t) * g.nw + w] = word;
  }
  uint32_t cnt = __popcll(word);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if (lane == 0) counts[t] = static_cast<uint32_t>(g.Q) * cnt;
}

// b-bit code of payload element x (x >= offsets[t + 1], x < payload): the
// LT t' holding it (offsets[t'] <= x < offsets[t' + 1], found by binary
// search among the LTs after t), its stream q and rank r there, the r-th
// active position of t' (wave prefix of its word popcounts, then the r'-th
// set bit of the word that holds it), and that position's weight in area q
// (0 where pruned).  Wave-uniform: every lane returns the same value.
template <bool MASK, int BITS>
__device__ inline uint32_t union_code_at(const UnionGeom& g, const uint16_t* W, const uint8_t* mask,
                                         const uint64_t* bitmaps, const uint32_t* offsets, const uint16_t* scales,
                                         int t, uint64_t x, int lane) {
  constexpr int kQmax = (1 << (BITS - 1)) - 1;
  int lo = t + 1, hi = g.nlt - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid + 1] > x)
      hi = mid;
    else
      lo = mid + 1;
  }
  const uint64_t ox = offsets[lo];
  const uint32_t P = static_cast<uint32_t>((offsets[lo + 1] - ox) / static_cast<uint64_t>(g.Q));
  if (P == 0) return 0;   // offsets that disagree with the words: stay inside the LT
  const uint32_t i = static_cast<uint32_t>(x - ox);
  const int q = static_cast<int>(min(i / P, static_cast<uint32_t>(g.Q - 1)));
  const uint32_t r = i - static_cast<uint32_t>(q) * P;
  const uint64_t word = lane < g.nw ? bitmaps[static_cast<uint64_t>(lo) * g.nw + lane] : 0ull;
  const uint32_t pc = __popcll(word);
  uint32_t incl = pc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  const uint64_t past = __ballot(incl > r);
  if (!past) return 0;
  const int owner = __builtin_ctzll(past);
  const uint32_t before = __shfl(incl - pc, owner);
  uint64_t w = (static_cast<uint64_t>(static_cast<uint32_t>(__shfl(static_cast<int>(word >> 32), owner))) << 32) |
               static_cast<uint32_t>(__shfl(static_cast<int>(word), owner));
  for (uint32_t k = before; k < r; ++k) w &= w - 1;   // drop the active positions ranked before r
  if (w == 0) return 0;
  const int p = 64 * owner + __builtin_ctzll(w);
  const uint64_t e = union_elem(g, lo, q, p);
  const bool kept = MASK ? mask[e] != 0 : (W[e] & 0x7FFFu) != 0;
  if (!kept) return 0;
  const uint32_t row = static_cast<uint32_t>(e / static_cast<uint64_t>(g.K));
  return static_cast<uint32_t>(usw::int_code(W[e], usw::f16_to_f64(scales[row]), kQmax)) & ((1u << BITS) - 1u);
}

// One wave per LT, lane w Q + q for area q of union word w: it ranks the
// active positions of word w (wave prefix of the word popcounts plus the
// position in the word) and stages the area's codes at q P + rank in LDS (0
// for a pruned weight); the run of Q P codes is then packed 8 / BITS per
// byte, byte b written by the LT holding its first code (codes of the byte
// past the run come from the following LTs).
template <bool MASK, int BITS>
__global__ __launch_bounds__(kEThreads) void union_values_kernel(const uint16_t* __restrict__ W,
                                                                 const uint8_t* __restrict__ mask,
                                                                 const uint64_t* __restrict__ bitmaps,
                                                                 const uint32_t* __restrict__ offsets,
                                                                 const uint16_t* __restrict__ scales,
                                                                 uint8_t* __restrict__ values, UnionGeom g,
                                                                 uint64_t payload, uint64_t logical) {
  constexpr int kQmax = (1 << (BITS - 1)) - 1;
  constexpr uint32_t kPer = 8 / BITS;
  constexpr uint32_t kCodeMask = (1u << BITS) - 1u;
  __shared__ uint8_t stage[kEWaves][kMaxBt * 64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kEWaves + wv;
  if (t >= g.nlt) return;
  uint8_t* st = stage[wv];
  const uint64_t o0 = offsets[t];
  const int w = lane / g.Q, q = lane - w * g.Q;
  const uint64_t word = w < g.nw ? bitmaps[static_cast<uint64_t>(t) * g.nw + w] : 0ull;
  const uint32_t cnt = __popcll(word);
  uint32_t inc = q == 0 ? cnt : 0u;   // each word counted once, by its area-0 lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t x = __shfl_up(inc, o);
    if (lane >= o) inc += x;
  }
  const uint32_t P = __shfl(inc, 63);
  if (word) {
    for (int c = 0; c < 8; ++c) {
      const uint32_t byte = static_cast<uint32_t>(word >> (8 * c)) & 0xFFu;
      if (!byte) continue;
      uint32_t r = inc - cnt + __popcll(word & ((1ull << (8 * c)) - 1));
      uint4 v;
      const uint32_t keep = union_chunk<MASK>(g, W, mask, t, q, 64 * w + 8 * c, v);
      const double s = usw::f16_to_f64(scales[union_elem(g, t, q, 64 * w + 8 * c) / static_cast<uint64_t>(g.K)]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (!((byte >> k) & 1u)) continue;
        const uint32_t code =
            ((keep >> k) & 1u) ? static_cast<uint32_t>(usw::int_code(half_of(v, k), s, kQmax)) & kCodeMask : 0u;
        st[q * P + r] = static_cast<uint8_t>(code);
        ++r;
      }
    }
  }
  usw_dev::wave_sync();
  const uint64_t e = o0 + static_cast<uint64_t>(g.Q) * P;
  // Codes after the run that share its last byte (the following LTs' first
  // ones; 0 past the payload).
  uint32_t tail[kPer - 1];
#pragma unroll
  for (uint32_t j = 0; j + 1 < kPer; ++j) {
    const uint64_t x = e + j;
    tail[j] = (P && x % kPer != 0 && x < payload && t + 1 < g.nlt && (x / kPer) == ((e - 1) / kPer))
                  ? union_code_at<MASK, BITS>(g, W, mask, bitmaps, offsets, scales, t, x, lane)
                  : 0u;
  }
  for (uint64_t b = (o0 + kPer - 1) / kPer + lane; b * kPer < e; b += 64) {
    uint32_t packed = 0;
#pragma unroll
    for (uint32_t j = 0; j < kPer; ++j) {
      const uint64_t x = b * kPer + j;
      uint32_t c = 0;
      if (x < e) {
        c = st[x - o0];
      } else {
#pragma unroll
        for (uint32_t k = 0; k + 1 < kPer; ++k)
          if (x == e + k) c = tail[k];
      }
      packed |= c << (BITS * j);
    }
    if (b < logical) values[b] = static_cast<uint8_t>(packed);
  }
}

// ---------------------------------------------------------------------------
// Tiled-CBC encoding on the device ("Unified Static-Dynamic Pruning for
// Efficient LLM Inference", section 4.1: GTiles of 256 x 16, four 64-bit
// words per column, each column's kept weights top to bottom padded with +0
// to a multiple of 8, ColInfo = run offset << 16 | kept count, TileOffset per
// GTile).  The same bytes as usw_cbc_encode.
// ---------------------------------------------------------------------------

constexpr int kCbcRows = 256, kCbcCols = 16;

// Kept bits of the 16 columns of one GTile row (mask bytes, or fp16 W).
template <bool MASK>
__device__ inline uint32_t cbc_row_bits(const uint16_t* W, const uint8_t* mask, uint64_t e, uint4& w0, uint4& w1) {
  w0 = *reinterpret_cast<const uint4*>(W + e);
  w1 = *reinterpret_cast<const uint4*>(W + e + 8);
  if (MASK) {
    const uint4 m = *reinterpret_cast<const uint4*>(mask + e);
    return kept8(make_uint2(m.x, m.y)) | (kept8(make_uint2(m.z, m.w)) << 8);
  }
  return nonzero8(w0) | (nonzero8(w1) << 8);
}

// One wave per GTile; lane l holds rows l, 64 + l, 128 + l, 192 + l.  Word q
// of column c is the wave's ballot of column c's kept bit over rows 64 q + l;
// lane 4 c + q stores it.  Column counts, their padded runs and ColInfo are
// wave-uniform; the GTile's padded total goes to counts[t].
template <bool MASK>
__global__ __launch_bounds__(kEThreads) void cbc_index_kernel(const uint16_t* __restrict__ W,
                                                              const uint8_t* __restrict__ mask,
                                                              uint64_t* __restrict__ bitmaps,
                                                              uint32_t* __restrict__ counts,
                                                              uint32_t* __restrict__ colinfo, int K, int gc, int ngt) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kEWaves + (threadIdx.x >> 6);
  if (t >= ngt) return;
  const int ti = t / gc, tj = t - ti * gc;
  uint32_t bits[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 w0, w1;
    bits[q] = cbc_row_bits<MASK>(W, mask, elem_rc(K, ti * kCbcRows + 64 * q + lane, tj * kCbcCols), w0, w1);
  }
  uint64_t mine = 0;
  uint32_t run = 0, info = 0;
  for (int c = 0; c < kCbcCols; ++c) {
    uint32_t n = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t word = __ballot((bits[q] >> c) & 1u);
      n += __popcll(word);
      if (lane == 4 * c + q) mine = word;
    }
    if (lane == c) info = (run << 16) | n;
    run += (n + 7) & ~7u;
  }
  bitmaps[static_cast<uint64_t>(t) * 64 + lane] = mine;
  if (lane < kCbcCols) colinfo[static_cast<uint64_t>(t) * kCbcCols + lane] = info;
  if (lane == 0) counts[t] = run;
}

// One wave per GTile, lane l on rows l, 64 + l, 128 + l, 192 + l again: for
// each column the kept weight of row 64 q + l goes to TileOffset + run +
// (kept rows above it: earlier words' popcounts plus v_mbcnt of its word),
// and lanes 0 .. pad - 1 write the column's +0 padding.
__global__ __launch_bounds__(kEThreads) void cbc_values_kernel(const uint16_t* __restrict__ W,
                                                               const uint64_t* __restrict__ bitmaps,
                                                               const uint32_t* __restrict__ toff,
                                                               const uint32_t* __restrict__ colinfo,
                                                               uint16_t* __restrict__ values, int K, int gc, int ngt,
                                                               uint64_t nvals) {
  // The GTile's padded runs are staged in LDS and written out in 16-byte
  // pieces: every run is a multiple of 8 values, so each TileOffset is too.
  __shared__ __align__(16) uint16_t stage[kEWaves][kCbcRows * kCbcCols];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * kEWaves + wv;
  if (t >= ngt) return;
  uint16_t* st = stage[wv];
  const int ti = t / gc, tj = t - ti * gc;
  const uint64_t base = toff[t];
  const uint64_t myword = bitmaps[static_cast<uint64_t>(t) * 64 + lane];
  const uint32_t myinfo = lane < kCbcCols ? colinfo[static_cast<uint64_t>(t) * kCbcCols + lane] : 0u;
  uint4 w[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t e = elem_rc(K, ti * kCbcRows + 64 * q + lane, tj * kCbcCols);
    w[q][0] = *reinterpret_cast<const uint4*>(W + e);
    w[q][1] = *reinterpret_cast<const uint4*>(W + e + 8);
  }
  // Column c's ColInfo and words sit in lanes c and 4 c + q: the lane index
  // is wave-uniform, so v_readlane brings them into scalar registers.
  uint32_t total = 0;
  for (int c = 0; c < kCbcCols; ++c) {
    const uint32_t info = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(myinfo), c));
    const uint32_t col = info >> 16;
    const uint32_t n = info & 0xFFFFu;
    uint32_t above = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(myword), 4 * c + q));
      const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(myword >> 32), 4 * c + q));
      const uint64_t word = (static_cast<uint64_t>(hi) << 32) | lo;
      if ((word >> lane) & 1ull) {
        const uint32_t rank = above + __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0u));
        const uint4 v = c < 8 ? w[q][0] : w[q][1];   // a select, not a dynamic register index
        if (col + rank < kCbcRows * kCbcCols) st[col + rank] = half_of(v, c & 7);
      }
      above += __popcll(word);
    }
    const uint32_t np = (n + 7) & ~7u;
    if (static_cast<uint32_t>(lane) < np - n && col + n + lane < kCbcRows * kCbcCols) st[col + n + lane] = 0;
    total = col + np;
  }
  usw_dev::wave_sync();
  for (uint32_t i = 8 * lane; i < total && i < kCbcRows * kCbcCols; i += 512)
    if (base + i + 8 <= nvals)
      *reinterpret_cast<uint4*>(values + base + i) = *reinterpret_cast<const uint4*>(st + i);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

usw_status enc_geometry(int32_t M, int32_t K, int32_t gt_m, int32_t gt_k, int32_t val_type, usw::Geometry* g,
                        EncGeom* eg) {
  usw_status st = usw::make_geometry(M, K, gt_m, gt_k, g);
  if (st) return st;
  if (val_type != USW_VAL_F16 && val_type != USW_VAL_I4) return USW_ERR_BAD_DTYPE;
  if (g->M * g->K >= (int64_t(1) << 32)) return USW_ERR_BAD_SHAPE;   // NNZ then fits the 32-bit offsets
  if (g->bt_per_gt > kMaxBt) return USW_ERR_UNSUPPORTED;
  eg->K = static_cast<int>(g->K);
  eg->gt_m = static_cast<int>(g->gt_m);
  eg->gt_k = static_cast<int>(g->gt_k);
  eg->Gc = static_cast<int>(g->Gc);
  eg->Tc = static_cast<int>(g->Tc);
  eg->bpg = static_cast<int>(g->bt_per_gt);
  eg->ngt = static_cast<int>(g->ngt);
  return USW_OK;
}

usw_status union_enc_geometry(int32_t M, int32_t K, int32_t lt_m, int32_t lt_k, int32_t r_a, int32_t c_a,
                              int32_t val_type, usw::UnionGeometry* g, UnionGeom* ug) {
  usw_status st = usw::make_union_geometry(M, K, lt_m, lt_k, r_a, c_a, g);
  if (st) return st;
  if (val_type != USW_VAL_F16 && val_type != USW_VAL_I4 && val_type != USW_VAL_I2) return USW_ERR_BAD_DTYPE;
  if (g->M * g->K >= (int64_t(1) << 32)) return USW_ERR_BAD_SHAPE;   // payload then fits the 32-bit offsets
  // INT4 or 2-bit payload; LTs of at most 4096 elements (one wave stages
  // the whole run in LDS), areas whose rows are multiples of 8 positions.
  if (val_type == USW_VAL_F16 || g->lt_m * g->lt_k > kMaxBt * 64 || g->ak % 8) return USW_ERR_UNSUPPORTED;
  ug->K = static_cast<int>(g->K);
  ug->lt_m = static_cast<int>(g->lt_m);
  ug->lt_k = static_cast<int>(g->lt_k);
  ug->am = static_cast<int>(g->am);
  ug->ak = static_cast<int>(g->ak);
  ug->c_a = static_cast<int>(g->c_a);
  ug->Q = static_cast<int>(g->Q);
  ug->lc = static_cast<int>(g->lc);
  ug->nw = static_cast<int>(g->nw);
  ug->nlt = static_cast<int>(g->nlt);
  return USW_OK;
}

unsigned blocks_for(int64_t items) { return static_cast<unsigned>((items + kEWaves - 1) / kEWaves); }

}  // namespace

extern "C" {

usw_status usw_encode_device_index(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t gt_m,
                                   int32_t gt_k, int32_t val_type, uint64_t* bitmaps, uint32_t* offsets,
                                   uint16_t* scales, void* stream) {
  if (!W || !bitmaps || !offsets) return USW_ERR_NULL_ARG;
  usw::Geometry g;
  EncGeom eg;
  usw_status st = enc_geometry(M, K, gt_m, gt_k, val_type, &g, &eg);
  if (st) return st;
  if (val_type == USW_VAL_I4 && !scales) return USW_ERR_NULL_ARG;
  if (!aligned(W, 16) || (mask && !aligned(mask, 8)) || !aligned(bitmaps, 8) || !aligned(offsets, 4) ||
      (val_type == USW_VAL_I4 && !aligned(scales, 2)))
    return USW_ERR_MISALIGNED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (mask)
    enc_index_kernel<true><<<blocks_for(g.ngt), kEThreads, 0, hs>>>(W, mask, bitmaps, offsets, eg);
  else
    enc_index_kernel<false><<<blocks_for(g.ngt), kEThreads, 0, hs>>>(W, mask, bitmaps, offsets, eg);
  enc_scan_kernel<<<1, 1024, 0, hs>>>(offsets, eg.ngt);
  if (val_type == USW_VAL_I4) {
    if (mask)
      enc_scales_kernel<true><<<blocks_for(g.M), kEThreads, 0, hs>>>(W, mask, scales, M, K, 7);
    else
      enc_scales_kernel<false><<<blocks_for(g.M), kEThreads, 0, hs>>>(W, mask, scales, M, K, 7);
  }
  return hipGetLastError() == hipSuccess ? USW_OK : USW_ERR_HIP;
}

usw_status usw_encode_device_values(const uint16_t* W, int32_t M, int32_t K, int32_t gt_m, int32_t gt_k,
                                    int32_t val_type, const uint64_t* bitmaps, const uint32_t* offsets,
                                    const uint16_t* scales, int64_t nnz, void* values, size_t values_capacity,
                                    void* stream) {
  if (!W || !bitmaps || !offsets || !values) return USW_ERR_NULL_ARG;
  usw::Geometry g;
  EncGeom eg;
  usw_status st = enc_geometry(M, K, gt_m, gt_k, val_type, &g, &eg);
  if (st) return st;
  if (val_type == USW_VAL_I4 && !scales) return USW_ERR_NULL_ARG;
  if (nnz < 0 || nnz > g.M * g.K) return USW_ERR_CAPACITY;
  const bool i4 = val_type == USW_VAL_I4;
  const uint64_t logical = i4 ? static_cast<uint64_t>(nnz + 1) / 2 : 2 * static_cast<uint64_t>(nnz);
  if (values_capacity < logical) return USW_ERR_CAPACITY;
  if (!aligned(W, 16) || !aligned(bitmaps, 8) || !aligned(offsets, 4) || !aligned(values, 16) ||
      (i4 && !aligned(scales, 2)))
    return USW_ERR_MISALIGNED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (i4)
    enc_values_kernel<true><<<blocks_for(g.ngt), kEThreads, 0, hs>>>(W, bitmaps, offsets, scales, values, eg,
                                                                      static_cast<uint64_t>(nnz), logical);
  else
    enc_values_kernel<false><<<blocks_for(g.ngt), kEThreads, 0, hs>>>(W, bitmaps, offsets, scales, values, eg,
                                                                       static_cast<uint64_t>(nnz), logical);
  const uint64_t tail = values_capacity - logical;
  if (tail) {
    const uint64_t blocks = (tail + kEThreads - 1) / kEThreads;
    enc_zero_kernel<<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), kEThreads, 0, hs>>>(
        static_cast<uint8_t*>(values) + logical, tail);
  }
  return hipGetLastError() == hipSuccess ? USW_OK : USW_ERR_HIP;
}

usw_status usw_union_encode_device_index(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K, int32_t lt_m,
                                         int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type,
                                         uint64_t* bitmaps, uint32_t* offsets, uint16_t* scales, void* stream) {
  if (!W || !bitmaps || !offsets || !scales) return USW_ERR_NULL_ARG;
  usw::UnionGeometry g;
  UnionGeom ug;
  usw_status st = union_enc_geometry(M, K, lt_m, lt_k, r_a, c_a, val_type, &g, &ug);
  if (st) return st;
  if (!aligned(W, 16) || (mask && !aligned(mask, 8)) || !aligned(bitmaps, 8) || !aligned(offsets, 4) ||
      !aligned(scales, 2))
    return USW_ERR_MISALIGNED;
  const int qmax = val_type == USW_VAL_I2 ? 1 : 7;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (mask) {
    union_index_kernel<true><<<blocks_for(g.nlt), kEThreads, 0, hs>>>(W, mask, bitmaps, offsets, ug);
    enc_scan_kernel<<<1, 1024, 0, hs>>>(offsets, ug.nlt);
    enc_scales_kernel<true><<<blocks_for(g.M), kEThreads, 0, hs>>>(W, mask, scales, M, K, qmax);
  } else {
    union_index_kernel<false><<<blocks_for(g.nlt), kEThreads, 0, hs>>>(W, mask, bitmaps, offsets, ug);
    enc_scan_kernel<<<1, 1024, 0, hs>>>(offsets, ug.nlt);
    enc_scales_kernel<false><<<blocks_for(g.M), kEThreads, 0, hs>>>(W, mask, scales, M, K, qmax);
  }
  return hipGetLastError() == hipSuccess ? USW_OK : USW_ERR_HIP;
}

usw_status usw_union_encode_device_values(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K,
                                          int32_t lt_m, int32_t lt_k, int32_t r_a, int32_t c_a, int32_t val_type,
                                          const uint64_t* bitmaps, const uint32_t* offsets, const uint16_t* scales,
                                          int64_t payload, void* values, size_t values_capacity, void* stream) {
  if (!W || !bitmaps || !offsets || !scales || !values) return USW_ERR_NULL_ARG;
  usw::UnionGeometry g;
  UnionGeom ug;
  usw_status st = union_enc_geometry(M, K, lt_m, lt_k, r_a, c_a, val_type, &g, &ug);
  if (st) return st;
  if (payload < 0 || payload > g.M * g.K) return USW_ERR_CAPACITY;
  const bool i2 = val_type == USW_VAL_I2;
  const uint64_t logical = i2 ? static_cast<uint64_t>(payload + 3) / 4 : static_cast<uint64_t>(payload + 1) / 2;
  if (values_capacity < logical) return USW_ERR_CAPACITY;
  if (!aligned(W, 16) || (mask && !aligned(mask, 8)) || !aligned(bitmaps, 8) || !aligned(offsets, 4) ||
      !aligned(scales, 2) || !aligned(values, 16))
    return USW_ERR_MISALIGNED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint8_t* vb = static_cast<uint8_t*>(values);
  const uint64_t pl = static_cast<uint64_t>(payload);
  const dim3 grid = blocks_for(g.nlt);
  if (mask) {
    if (i2)
      union_values_kernel<true, 2><<<grid, kEThreads, 0, hs>>>(W, mask, bitmaps, offsets, scales, vb, ug, pl, logical);
    else
      union_values_kernel<true, 4><<<grid, kEThreads, 0, hs>>>(W, mask, bitmaps, offsets, scales, vb, ug, pl, logical);
  } else if (i2) {
    union_values_kernel<false, 2><<<grid, kEThreads, 0, hs>>>(W, mask, bitmaps, offsets, scales, vb, ug, pl, logical);
  } else {
    union_values_kernel<false, 4><<<grid, kEThreads, 0, hs>>>(W, mask, bitmaps, offsets, scales, vb, ug, pl, logical);
  }
  const uint64_t tail = values_capacity - logical;
  if (tail) {
    const uint64_t blocks = (tail + kEThreads - 1) / kEThreads;
    enc_zero_kernel<<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), kEThreads, 0, hs>>>(vb + logical, tail);
  }
  return hipGetLastError() == hipSuccess ? USW_OK : USW_ERR_HIP;
}

usw_status usw_cbc_encode_device_index(const uint16_t* W, const uint8_t* mask, int32_t M, int32_t K,
                                       uint64_t* bitmaps, uint32_t* tile_offsets, uint32_t* colinfo, void* stream) {
  if (!W || !bitmaps || !tile_offsets || !colinfo) return USW_ERR_NULL_ARG;
  usw::CbcGeometry g;
  usw_status st = usw::make_cbc_geometry(M, K, &g);
  if (st) return st;
  if (g.M * g.K >= (int64_t(1) << 32)) return USW_ERR_BAD_SHAPE;
  if (!aligned(W, 16) || (mask && !aligned(mask, 16)) || !aligned(bitmaps, 8) || !aligned(tile_offsets, 4) ||
      !aligned(colinfo, 4))
    return USW_ERR_MISALIGNED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int gc = static_cast<int>(g.gc), ngt = static_cast<int>(g.ngt);
  if (mask)
    cbc_index_kernel<true><<<blocks_for(g.ngt), kEThreads, 0, hs>>>(W, mask, bitmaps, tile_offsets, colinfo, K, gc,
                                                                     ngt);
  else
    cbc_index_kernel<false><<<blocks_for(g.ngt), kEThreads, 0, hs>>>(W, mask, bitmaps, tile_offsets, colinfo, K, gc,
                                                                      ngt);
  enc_scan_kernel<<<1, 1024, 0, hs>>>(tile_offsets, ngt);
  return hipGetLastError() == hipSuccess ? USW_OK : USW_ERR_HIP;
}

usw_status usw_cbc_encode_device_values(const uint16_t* W, int32_t M, int32_t K, const uint64_t* bitmaps,
                                        const uint32_t* tile_offsets, const uint32_t* colinfo, int64_t nnz_padded,
                                        uint16_t* values, size_t values_capacity, void* stream) {
  if (!W || !bitmaps || !tile_offsets || !colinfo || !values) return USW_ERR_NULL_ARG;
  usw::CbcGeometry g;
  usw_status st = usw::make_cbc_geometry(M, K, &g);
  if (st) return st;
  if (g.M * g.K >= (int64_t(1) << 32)) return USW_ERR_BAD_SHAPE;
  if (nnz_padded < 0 || nnz_padded > g.M * g.K) return USW_ERR_CAPACITY;
  if (values_capacity < 2 * static_cast<uint64_t>(nnz_padded)) return USW_ERR_CAPACITY;
  if (!aligned(W, 16) || !aligned(bitmaps, 8) || !aligned(tile_offsets, 4) || !aligned(colinfo, 4) ||
      !aligned(values, 16))
    return USW_ERR_MISALIGNED;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  cbc_values_kernel<<<blocks_for(g.ngt), kEThreads, 0, hs>>>(W, bitmaps, tile_offsets, colinfo, values,
                                                             static_cast<int>(K), static_cast<int>(g.gc),
                                                             static_cast<int>(g.ngt),
                                                             static_cast<uint64_t>(nnz_padded));
  // Whole fp16 elements past the padded runs are zeroed (a trailing odd byte
  // of the capacity is left alone, as the host encoder does).
  const uint64_t tail = (values_capacity / 2 - static_cast<uint64_t>(nnz_padded)) * 2;
  if (tail) {
    const uint64_t blocks = (tail + kEThreads - 1) / kEThreads;
    enc_zero_kernel<<<static_cast<unsigned>(blocks < 4096 ? blocks : 4096), kEThreads, 0, hs>>>(
        reinterpret_cast<uint8_t*>(values + nnz_padded), tail);
  }
  return hipGetLastError() == hipSuccess ? USW_OK : USW_ERR_HIP;
}

}  // extern "C"
