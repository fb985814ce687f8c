// Device half of libusw: the bitmap SpMM decode kernels for gfx950 and the
// usw_spmm dispatcher.
//
// What is computed: Y[n][m] = sum_k W_sp[m][k] X[n][k], W_sp held in the
// TCA-BME bitmap format (blog "SpInfer: How bitmaps make sparse LLMs actually
// fast", section "How TCA-BME addresses the indexing overhead").  Values are
// located by masked popcount (same blog, "Shared Memory Bitmap Decoding").
//
// Design (gfx950, wave64):
//   * One workgroup owns one 64-row strip of GroupTiles (64x64) and a range
//     of GroupTile columns; each of its waves streams its own contiguous run
//     of GroupTiles (bitmaps and values of consecutive GroupTiles of a strip
//     are contiguous in memory), so the main loop has no workgroup barrier.
//   * Loads run two GroupTiles ahead of the compute: the 16-byte global loads
//     of GroupTiles c+1 and c+2 (bitmaps, the value range [offsets[g],
//     offsets[g+1]) from a 16-byte aligned start, and the X^T fragments) sit
//     in registers while GroupTile c, already copied into the wave's private
//     LDS buffer, is rebuilt and multiplied.
//   * Rebuild: v_mfma_f32_16x16x32_f16 gives lane l the row l%16 and the 8
//     consecutive columns 8*(l/16)..+7 of a 16x32 block, which is exactly one
//     row of one BitmapTile; its kept values are contiguous in the stream.
//     The lane finds where they start (GroupTile offset + popcounts of the
//     earlier BitmapTiles, from a DPP wave prefix scan, + popcount of the
//     earlier rows of its own BitmapTile) and expands them into 8 slots with
//     two aligned LDS windows and v_perm_b32 byte selectors looked up by the
//     row's 8-bit mask (zero for clear bits).
//   * The rebuilt 16x32 fragment meets the X^T fragment (X is [N][K], so each
//     lane's 8 k values are one 16-byte load) on the matrix cores with fp32
//     accumulation, which leaves the vector ALUs to the rebuild.
//   * Partial sums of the waves of a workgroup are added in LDS in a fixed
//     order; across workgroups (split K) they go through an fp32 workspace and
//     a second kernel adds them in a fixed order: results are deterministic.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>

#include "usw.h"
#include "usw_internal.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGT = 64;                   // GroupTile side the kernels are built for
constexpr int kBtPerGt = 64;              // BitmapTiles per 64x64 GroupTile
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kThreads = 64 * kWaves;

// Per-value-type constants.  Every one of a GroupTile's kChunks*64 16-byte
// chunk slots is loaded and stored unconditionally (slots past the
// GroupTile's last chunk repeat that chunk), so the loads carry no branches
// and the compiler can wait for exactly the GroupTile being consumed.
template <bool I4>
struct ValTraits;
template <>
struct ValTraits<false> {
  static constexpr int kChunks = 6;       // 16-byte chunks per lane kept in flight (6 KB per GroupTile)
  // A dense GroupTile is 8192 B of values; the buffer adds the <16 B head
  // before the first value and the <16 B a window reads past the last one.
  static constexpr int kVbuf = 8192 + 64;
};
template <>
struct ValTraits<true> {
  static constexpr int kChunks = 3;       // covers every GroupTile (<= 2064 B)
  static constexpr int kVbuf = 3 * 1024 + 64;
};
static_assert(ValTraits<false>::kVbuf >= 1024 * ValTraits<false>::kChunks, "unconditional stores fit");

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Inclusive prefix sum over the 64 lanes with DPP (no LDS round trips):
// Hillis-Steele inside each 16-lane row, then the row totals are carried by
// the row_bcast:15 and row_bcast:31 broadcasts.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

// v_perm_b32 byte selectors that expand the packed fp16 values of one 4-bit
// nibble of a BitmapTile row into 4 slots.  Packed value k of the window
// occupies bytes 2k, 2k+1 (window dword 0 = selector bytes 0-3, dword 1 =
// bytes 4-7); a clear bit selects 0x0C, which v_perm turns into 0x00.
__device__ __forceinline__ uint32_t nibble_selector(uint32_t q, int j) {
  uint32_t sel = 0;
  for (int h = 0; h < 2; ++h) {
    const int p = 2 * j + h;
    uint32_t s16 = 0x0C0Cu;
    if ((q >> p) & 1u) {
      const uint32_t k = __builtin_popcount(q & ((1u << p) - 1u));
      s16 = (2u * k) | ((2u * k + 1u) << 8);
    }
    sel |= s16 << (16 * h);
  }
  return sel;
}

// v_perm selectors that expand the 8 packed nibbles of one BitmapTile row
// into 8 byte slots.  Packed nibble k sits in byte k/2 of lo4 (k even) or of
// hi4 (k odd), lo4 = w & 0x0F0F0F0F and hi4 = (w >> 4) & 0x0F0F0F0F, and
// v_perm(hi4, lo4, sel) numbers lo4's bytes 0-3 and hi4's bytes 4-7.
__device__ __forceinline__ uint32_t nibble_byte_selector(uint32_t b, int half) {
  uint32_t sel = 0;
  for (int s = 0; s < 4; ++s) {
    const int p = 4 * half + s;
    uint32_t v = 0x0Cu;
    if ((b >> p) & 1u) {
      const uint32_t k = __builtin_popcount(b & ((1u << p) - 1u));
      v = (k & 1u) ? 4u + (k >> 1) : (k >> 1);
    }
    sel |= v << (8 * s);
  }
  return sel;
}

// Two dwords holding packed fp16 values e, e+1, e+2, e+3 of an LDS buffer
// (element e starts at byte 2e; the buffer is dword aligned).
__device__ __forceinline__ u32x2_t lds_window_f16(const uint8_t* buf, uint32_t e) {
  const uint32_t ba = 2u * e;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(buf + (ba & ~3u));
  const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
  u32x2_t w;
  w.x = __builtin_amdgcn_alignbyte(d1, d0, ba & 3u);
  w.y = __builtin_amdgcn_alignbyte(d2, d1, ba & 3u);
  return w;
}

// The 8 dense fp16 slots (one BitmapTile row) of a lane's A fragment.
template <bool I4>
__device__ __forceinline__ half8_t rebuild_row(const uint8_t* vb, const uint32_t* lut, uint32_t rb, uint32_t byte) {
  if constexpr (!I4) {
    const u32x4_t sel = reinterpret_cast<const u32x4_t*>(lut)[byte];
    const uint32_t pcl = __builtin_popcount(byte & 0xFu);
    const u32x2_t lo = lds_window_f16(vb, rb);
    const u32x2_t hi = lds_window_f16(vb, rb + pcl);
    u32x4_t a;
    a.x = __builtin_amdgcn_perm(lo.y, lo.x, sel.x);
    a.y = __builtin_amdgcn_perm(lo.y, lo.x, sel.y);
    a.z = __builtin_amdgcn_perm(hi.y, hi.x, sel.z);
    a.w = __builtin_amdgcn_perm(hi.y, hi.x, sel.w);
    return __builtin_bit_cast(half8_t, a);
  } else {
    const u32x2_t sel = reinterpret_cast<const u32x2_t*>(lut)[byte];
    // 8 packed nibbles starting at nibble rb.
    const uint32_t ba = rb >> 1;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(vb + (ba & ~3u));
    const uint32_t sh = ((ba & 3u) << 3) | ((rb & 1u) << 2);
    const uint32_t win = __builtin_amdgcn_alignbit(p[1], p[0], sh);
    const uint32_t lo4 = win & 0x0F0F0F0Fu;
    const uint32_t hi4 = (win >> 4) & 0x0F0F0F0Fu;
    // Slots as bytes; xor 8 maps the two's-complement nibble q to q + 8 in
    // [0, 15] (an empty slot's 0 becomes 8, i.e. q = 0).
    const uint32_t e0 = __builtin_amdgcn_perm(hi4, lo4, sel.x) ^ 0x08080808u;
    const uint32_t e1 = __builtin_amdgcn_perm(hi4, lo4, sel.y) ^ 0x08080808u;
    // fp16 bit pattern 0x6400 | u is 1024 + u exactly; subtracting 1032
    // leaves q exactly.
    u32x4_t a;
    a.x = __builtin_amdgcn_perm(0x64646464u, e0, 0x04010400u);
    a.y = __builtin_amdgcn_perm(0x64646464u, e0, 0x04030402u);
    a.z = __builtin_amdgcn_perm(0x64646464u, e1, 0x04010400u);
    a.w = __builtin_amdgcn_perm(0x64646464u, e1, 0x04030402u);
    half8_t h = __builtin_bit_cast(half8_t, a);
    h += static_cast<_Float16>(-1032.0f);
    return h;
  }
}

// Registers holding one GroupTile's loads until they are copied into LDS.
template <int NB, bool I4>
struct Slot {
  u32x4_t v[ValTraits<I4>::kChunks];
  u32x4_t bm;
  u32x4_t x[2][NB];
  uint32_t nch;     // 16-byte chunks of values spanned (wave-uniform)
  uint32_t delta;   // value elements before the GroupTile's first one in its first chunk
  uint64_t a0;      // byte offset of the first chunk
};

struct Args {
  const uint64_t* __restrict__ bitmaps;
  const uint32_t* __restrict__ offsets;
  const uint8_t* __restrict__ values;
  const uint16_t* __restrict__ scales;
  const uint16_t* __restrict__ X;
  void* __restrict__ Y;
  float* __restrict__ ws;
  uint64_t values_alloc;   // padded size of the values buffer in bytes (>= 16)
  int M, K, N, Gc, splits;
};

template <int NB, bool I4>
__device__ __forceinline__ void slot_load(Slot<NB, I4>& s, const Args& a, int gi, int c, int lane) {
  const int64_t g = static_cast<int64_t>(gi) * a.Gc + c;
  const uint32_t o0 = a.offsets[g];
  const uint32_t o1 = a.offsets[g + 1];
  if constexpr (!I4) {
    s.a0 = (2ull * o0) & ~15ull;
    s.nch = static_cast<uint32_t>((2ull * o1 - s.a0 + 15ull) >> 4);
    s.delta = static_cast<uint32_t>((2ull * o0 - s.a0) >> 1);
  } else {
    s.a0 = (static_cast<uint64_t>(o0) >> 1) & ~15ull;
    const uint64_t bend = (static_cast<uint64_t>(o1) + 1) >> 1;   // first byte past the last nibble
    s.nch = static_cast<uint32_t>((bend - s.a0 + 15ull) >> 4);
    s.delta = static_cast<uint32_t>(o0 - 2 * s.a0);
  }
  // Chunk slots past the last chunk reload it (chunk 0 of an empty
  // GroupTile lies inside the padded allocation).  The clamps keep every
  // load inside the buffer and every store inside the LDS slot even for
  // offsets that disagree with the bitmaps.
  const uint64_t top = a.values_alloc - 16;
  s.a0 = min(s.a0, top);
  s.nch = min(s.nch, static_cast<uint32_t>((ValTraits<I4>::kVbuf - 16) / 16));
  const uint32_t last = min(s.nch > 0 ? s.nch - 1 : 0u, static_cast<uint32_t>((top - s.a0) >> 4));
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.values + s.a0);
#pragma unroll
  for (int i = 0; i < ValTraits<I4>::kChunks; ++i) s.v[i] = src[min(static_cast<uint32_t>(lane + 64 * i), last)];
  s.bm = reinterpret_cast<const u32x4_t*>(a.bitmaps + g * kBtPerGt)[lane & 31];
  // X^T fragments.  Columns n >= N of B only feed columns n >= N of the
  // product, which are never stored, so those lanes just repeat row N-1.
  const int row = lane & 15, kb = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = min(nb * 16 + row, a.N - 1);
      s.x[ks][nb] = *reinterpret_cast<const u32x4_t*>(a.X + static_cast<size_t>(n) * a.K + c * kGT + ks * 32 + kb * 8);
    }
}

template <int NB, bool I4>
__device__ __forceinline__ void slot_commit(const Slot<NB, I4>& s, uint8_t* vb, uint64_t* bb, int lane) {
#pragma unroll
  for (int i = 0; i < ValTraits<I4>::kChunks; ++i) reinterpret_cast<u32x4_t*>(vb)[lane + 64 * i] = s.v[i];
  // Both half-waves hold the same 512 B of bitmaps and store them alike.
  reinterpret_cast<u32x4_t*>(bb)[lane & 31] = s.bm;
}

// Copies the chunks a slot does not hold (GroupTiles denser than the slot
// covers; only the unpipelined path meets them).
template <int NB, bool I4>
__device__ __forceinline__ void slot_commit_rest(const Slot<NB, I4>& s, const Args& a, uint8_t* vb, int lane) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.values + s.a0);
  const uint32_t last = static_cast<uint32_t>((a.values_alloc - 16 - s.a0) >> 4);
  for (uint32_t ch = lane + 64 * ValTraits<I4>::kChunks; ch < s.nch; ch += 64)
    reinterpret_cast<u32x4_t*>(vb)[ch] = src[min(ch, last)];
}

// Rebuild and multiply one GroupTile already in LDS.
template <int NB, bool I4>
__device__ __forceinline__ void tile_compute(const Slot<NB, I4>& s, const uint8_t* vb, const uint64_t* bb,
                                             const uint32_t* lut, f32x4_t (&acc)[4][NB], int lane, int bt_lane,
                                             int r8, uint64_t rowmask) {
  const uint64_t bme = bb[lane];
  const uint32_t pc = __popcll(bme);
  const uint32_t ebase = wave_inclusive_scan(pc) - pc + s.delta;
#pragma unroll
  for (int rs = 0; rs < 4; ++rs) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int bt = 16 * rs + 8 * ks + bt_lane;
      const uint64_t bm = bb[bt];
      const uint32_t base = __builtin_amdgcn_ds_bpermute(bt << 2, ebase);
      const uint32_t rb = base + __popcll(bm & rowmask);
      const uint32_t byte = static_cast<uint32_t>(bm >> (8 * r8)) & 0xFFu;
      const half8_t ah = rebuild_row<I4>(vb, lut, rb, byte);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[rs][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(half8_t, s.x[ks][nb]),
                                                             acc[rs][nb], 0, 0, 0);
    }
  }
}

template <int NB, bool I4, bool OUT_F16>
__global__ __launch_bounds__(kThreads) void decode_kernel(Args a) {
  using VT = ValTraits<I4>;
  __shared__ __attribute__((aligned(16))) uint32_t lut[I4 ? 2 * 256 : 4 * 256];
  // Staging (per wave: values, then bitmaps); reused for the final reduction.
  constexpr int kStage = kWaves * (VT::kVbuf + 8 * kBtPerGt);
  constexpr int kRed = kWaves * 4 * NB * 64 * 4 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStage > kRed ? kStage : kRed];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is uniform across the wave; saying so keeps the wave's
  // GroupTile range, the offsets loads and the loop control scalar.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gi = blockIdx.x / a.splits;
  const int sidx = blockIdx.x - gi * a.splits;

  for (int b = tid; b < 256; b += kThreads) {
    if constexpr (!I4) {
      u32x4_t e;
      e.x = nibble_selector(b & 15, 0);
      e.y = nibble_selector(b & 15, 1);
      e.z = nibble_selector(b >> 4, 0);
      e.w = nibble_selector(b >> 4, 1);
      reinterpret_cast<u32x4_t*>(lut)[b] = e;
    } else {
      u32x2_t e;
      e.x = nibble_byte_selector(b, 0);
      e.y = nibble_byte_selector(b, 1);
      reinterpret_cast<u32x2_t*>(lut)[b] = e;
    }
  }
  __syncthreads();

  // Columns of GroupTiles this wave streams.
  const int parts = a.splits * kWaves;
  const int q = sidx * kWaves + w;
  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * q / parts);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (q + 1) / parts);

  // Lane constants of the 16x32 A fragment.
  const int row = lane & 15;               // row inside the 16-row slice
  const int kb = lane >> 4;                // which 8-column group of the 32
  const int r8 = row & 7;                  // row inside the BitmapTile
  const int bt_lane = 4 * (kb >> 1) + 2 * (row >> 3) + (kb & 1);  // BitmapTile among the 8 of a fragment
  const uint64_t rowmask = (1ull << (8 * r8)) - 1ull;

  f32x4_t acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint8_t* vb = smem + w * VT::kVbuf;
  uint64_t* bb = reinterpret_cast<uint64_t*>(smem + kWaves * VT::kVbuf) + w * kBtPerGt;

  // A wave may own no GroupTile column (K < 256): it only joins the
  // reduction.  A GroupTile whose values span more chunks than a slot holds
  // (fp16 density above ~75%) sends the whole wave down the unpipelined path.
  uint32_t widest = 0;
  for (int c = c_begin; c < c_end; ++c) {
    const int64_t g = static_cast<int64_t>(gi) * a.Gc + c;
    widest = max(widest, a.offsets[g + 1] - a.offsets[g]);
  }
  const uint32_t fast_limit = I4 ? 4096u : (16u * 64u * VT::kChunks - 32u) / 2u;

  if (c_begin >= c_end) {
    // nothing to stream
  } else if (widest > fast_limit) {
    for (int c = c_begin; c < c_end; ++c) {
      Slot<NB, I4> s0;
      slot_load(s0, a, gi, c, lane);
      slot_commit(s0, vb, bb, lane);
      slot_commit_rest(s0, a, vb, lane);
      wave_sync();
      tile_compute(s0, vb, bb, lut, acc, lane, bt_lane, r8, rowmask);
      wave_sync();
    }
  } else {
    // Three register slots: GroupTile c is in LDS while c+1 and c+2 load.
    // Loads past the wave's last GroupTile repeat it (every wave owns at
    // least one), so each step issues the same loads and waits for exactly
    // one slot.
    const int c_last = c_end - 1;
    Slot<NB, I4> s0, s1, s2;
    slot_load(s0, a, gi, c_begin, lane);
    slot_load(s1, a, gi, min(c_begin + 1, c_last), lane);
    auto step = [&](Slot<NB, I4>& cur, int c, Slot<NB, I4>& nxt) {
      slot_commit(cur, vb, bb, lane);
      wave_sync();
      slot_load(nxt, a, gi, min(c + 2, c_last), lane);
      tile_compute(cur, vb, bb, lut, acc, lane, bt_lane, r8, rowmask);
      wave_sync();
    };
    int c = c_begin;
    for (; c + 3 <= c_end; c += 3) {
      step(s0, c, s2);
      step(s1, c + 1, s0);
      step(s2, c + 2, s1);
    }
    if (c < c_end) step(s0, c, s2);
    if (c + 1 < c_end) step(s1, c + 1, s0);
  }

  // Workgroup reduction over waves (fixed order), then store.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [kWaves][4][NB][64 lanes][4]
#pragma unroll
  for (int rs = 0; rs < 4; ++rs)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4_t*>(red + (((w * 4 + rs) * NB + nb) * 64 + lane) * 4) = acc[rs][nb];
  __syncthreads();

  const int m0 = gi * kGT;
  for (int e = tid; e < 64 * 16 * NB; e += kThreads) {
    const int n = e >> 6;
    const int ml = e & 63;
    if (n >= a.N) continue;
    const int rs = ml >> 4, r16 = ml & 15;
    const int ln = ((r16 >> 2) << 4) | (n & 15);
    const int i = r16 & 3;
    const int nb = n >> 4;
    float sum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) sum += red[(((ww * 4 + rs) * NB + nb) * 64 + ln) * 4 + i];
    const size_t yi = static_cast<size_t>(n) * a.M + m0 + ml;
    if (a.splits > 1) {
      a.ws[static_cast<size_t>(sidx) * a.N * a.M + yi] = sum;   // INT4: unscaled; the reduction scales
    } else {
      if constexpr (I4) sum *= static_cast<float>(__builtin_bit_cast(_Float16, a.scales[m0 + ml]));
      if constexpr (OUT_F16)
        reinterpret_cast<_Float16*>(a.Y)[yi] = static_cast<_Float16>(sum);
      else
        reinterpret_cast<float*>(a.Y)[yi] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K reduction: Y[n][m] = scale[m] * sum_{s} ws[s][n][m], fixed order.
// ---------------------------------------------------------------------------
template <bool OUT_F16>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, void* __restrict__ Y,
                                                            const uint16_t* __restrict__ scales, int M, int N,
                                                            int splits) {
  const size_t total = static_cast<size_t>(M) * N;
  for (size_t i = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<size_t>(gridDim.x) * blockDim.x) {
    float s = 0.f;
    for (int p = 0; p < splits; ++p) s += ws[static_cast<size_t>(p) * total + i];
    if (scales) s *= static_cast<float>(__builtin_bit_cast(_Float16, scales[i % M]));
    if (OUT_F16)
      reinterpret_cast<_Float16*>(Y)[i] = static_cast<_Float16>(s);
    else
      reinterpret_cast<float*>(Y)[i] = s;
  }
}

// ---------------------------------------------------------------------------
// Host dispatch
// ---------------------------------------------------------------------------

struct Plan {
  int splits;     // workgroups per 64-row strip
  int nchunk;     // columns of N per kernel pass (16 or 32)
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

Plan make_plan(const usw::Geometry& g, int N, int splits_req) {
  Plan p;
  p.nchunk = N <= 16 ? 16 : 32;
  int s = splits_req;
  if (s <= 0) {
    // Enough workgroups to cover the 256 compute units, but each wave keeps
    // at least 4 GroupTiles to stream.
    s = static_cast<int>((256 + g.Gr - 1) / g.Gr);
    const int cap = static_cast<int>(std::max<int64_t>(1, g.Gc / (kWaves * 4)));
    s = std::min(s, cap);
  }
  const int smax = static_cast<int>(std::max<int64_t>(1, g.Gc / kWaves));
  p.splits = std::max(1, std::min(s, smax));
  return p;
}

usw_status check_common(const usw_fmt* f, int32_t y_type, int32_t N, usw::Geometry* g) {
  if (!f) return USW_ERR_NULL_ARG;
  usw_status st = usw::make_geometry(f->M, f->K, f->gt_m, f->gt_k, g);
  if (st) return st;
  if (f->val_type != USW_VAL_F16 && f->val_type != USW_VAL_I4) return USW_ERR_BAD_DTYPE;
  if (y_type != USW_OUT_F16 && y_type != USW_OUT_F32) return USW_ERR_BAD_DTYPE;
  if (N < 1) return USW_ERR_BAD_N;
  if (f->reserved != 0) return USW_ERR_BAD_SHAPE;
  if (f->gt_m != kGT || f->gt_k != kGT) return USW_ERR_UNSUPPORTED;
  if (f->val_type == USW_VAL_I4 && N > 32) return USW_ERR_UNSUPPORTED;
  if (f->nnz < 0 || f->nnz >= (int64_t(1) << 32)) return USW_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(N) * g->M > (int64_t(1) << 40)) return USW_ERR_BAD_SHAPE;
  return USW_OK;
}

size_t workspace_bytes(const usw::Geometry& g, const Plan& p) {
  if (p.splits <= 1) return 0;
  return static_cast<size_t>(p.splits) * p.nchunk * g.M * sizeof(float);
}

template <int NB, bool I4>
void launch_decode(const Args& a, bool f16out, dim3 grid, hipStream_t s) {
  if (f16out)
    decode_kernel<NB, I4, true><<<grid, kThreads, 0, s>>>(a);
  else
    decode_kernel<NB, I4, false><<<grid, kThreads, 0, s>>>(a);
}

usw_status spmm_impl(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N, void* ws,
                     size_t ws_bytes, void* stream, int splits_req) {
  usw::Geometry g;
  usw_status st = check_common(f, y_type, N, &g);
  if (st) return st;
  if (!X || !Y || !f->bitmaps || !f->offsets || !f->values) return USW_ERR_NULL_ARG;
  if (f->val_type == USW_VAL_I4 && !f->scales) return USW_ERR_NULL_ARG;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(f->bitmaps) || !aligned16(f->values) ||
      (reinterpret_cast<uintptr_t>(f->offsets) & 3u))
    return USW_ERR_MISALIGNED;
  const Plan p = make_plan(g, N, splits_req);
  const size_t need = workspace_bytes(g, p);
  if (need > 0) {
    if (!ws || ws_bytes < need) return USW_ERR_WORKSPACE;
    if (!aligned16(ws)) return USW_ERR_MISALIGNED;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(g.Gr * p.splits));
  const int M = static_cast<int>(g.M), K = static_cast<int>(g.K), Gc = static_cast<int>(g.Gc);
  const size_t ybytes = y_type == USW_OUT_F16 ? 2 : 4;
  const bool f16out = y_type == USW_OUT_F16;
  const bool i4 = f->val_type == USW_VAL_I4;

  for (int n0 = 0; n0 < N; n0 += p.nchunk) {
    const int nc = std::min(p.nchunk, N - n0);
    Args a;
    a.bitmaps = f->bitmaps;
    a.offsets = f->offsets;
    a.values = static_cast<const uint8_t*>(f->values);
    a.scales = i4 ? f->scales : nullptr;
    a.X = X + static_cast<size_t>(n0) * K;
    a.Y = static_cast<uint8_t*>(Y) + static_cast<size_t>(n0) * M * ybytes;
    a.ws = static_cast<float*>(ws);
    a.values_alloc = usw::values_alloc_bytes(f->val_type, f->nnz);
    a.M = M;
    a.K = K;
    a.N = nc;
    a.Gc = Gc;
    a.splits = p.splits;
    const bool two = nc > 16;
    if (i4) {
      if (two) launch_decode<2, true>(a, f16out, grid, s);
      else launch_decode<1, true>(a, f16out, grid, s);
    } else {
      if (two) launch_decode<2, false>(a, f16out, grid, s);
      else launch_decode<1, false>(a, f16out, grid, s);
    }
    if (hipGetLastError() != hipSuccess) return USW_ERR_HIP;
    if (p.splits > 1) {
      const size_t total = static_cast<size_t>(M) * nc;
      const unsigned rg = static_cast<unsigned>(std::min<size_t>((total + 255) / 256, 4096));
      if (f16out)
        splitk_reduce_kernel<true><<<rg, 256, 0, s>>>(a.ws, a.Y, a.scales, M, nc, p.splits);
      else
        splitk_reduce_kernel<false><<<rg, 256, 0, s>>>(a.ws, a.Y, a.scales, M, nc, p.splits);
      if (hipGetLastError() != hipSuccess) return USW_ERR_HIP;
    }
  }
  return USW_OK;
}

}  // namespace

extern "C" {

usw_status usw_spmm_workspace(const usw_fmt* f, int32_t N, size_t* bytes) {
  return usw_spmm_workspace_ex(f, N, 0, bytes);
}

usw_status usw_spmm(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N, void* ws,
                    size_t ws_bytes, void* stream) {
  return spmm_impl(f, X, Y, y_type, N, ws, ws_bytes, stream, 0);
}

usw_status usw_spmm_workspace_ex(const usw_fmt* f, int32_t N, int32_t splits, size_t* bytes) {
  if (!bytes) return USW_ERR_NULL_ARG;
  usw::Geometry g;
  usw_status st = check_common(f, USW_OUT_F16, N, &g);
  if (st) return st;
  *bytes = workspace_bytes(g, make_plan(g, N, splits < 0 ? 0 : splits));
  return USW_OK;
}

usw_status usw_spmm_ex(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N, int32_t splits,
                       void* ws, size_t ws_bytes, void* stream) {
  return spmm_impl(f, X, Y, y_type, N, ws, ws_bytes, stream, splits < 0 ? 0 : splits);
}

}  // extern "C"
