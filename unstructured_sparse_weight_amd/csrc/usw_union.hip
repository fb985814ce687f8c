// Device half of the IE-BME union-mask path: the INT4 decode kernel for
// gfx950 and the usw_union_spmm dispatcher.
//
// What is computed: Y[n][m] = sum_k W_sp[m][k] X[n][k], W_sp held in the
// IE-BME union-mask format ("UnionSparse: An Index-Efficient Sparsity
// Framework for Low-Bit Sparse LLM Inference on Edge", section on IE-BME):
// a 64 x 64 local tile (LT) is cut into a 2 x 2 grid of 32 x 32 areas, one
// union bit covers the four area-aligned weights of a position, and the four
// areas' values sit in four aligned streams indexed by one compact rank.
//
// Design (wave64, MFMA v_mfma_f32_16x16x32_f16):
//   * One workgroup owns one 64-row strip of LTs and a range of LT columns;
//     each of its four waves streams its own run of LTs, one LT ahead in
//     registers (union words, the LT's payload chunks, X^T fragments), the
//     current LT in the wave's LDS buffer.  No workgroup barrier in the loop.
//   * Fragment (f, ks) of an LT (strip rows 16f..16f+15, LT columns
//     32ks..32ks+31) lies in area (f / 2, ks), logical rows 16 (f % 2) ..
//     +15.  Lane l (i = l % 16, g = l / 16) holds its row i, columns
//     8g..8g+7, i.e. byte g of logical row r = 16 (f % 2) + i of the union
//     mask.  The four fragments f % 2 = h, f / 2 and ks free, share that byte
//     and its rank: the lane reads the row's word and the rank of its first
//     bit once (a 32-entry LDS table per LT, written by lanes 0-31 with a
//     DPP prefix scan), adds one masked popcount and looks up the v_perm
//     selectors of the whole byte once, then gathers the row of each area
//     from stream q at rank + q P_t: one bitmap traversal and one rank for Q
//     payload rows, the point of the section's LSPD gather.
//   * A row's at most 8 values are the 8 nibbles from its rank on, so one
//     v_alignbit window per area row holds them all; the 256-entry selector
//     table (8 bytes per mask byte) places nibble k of the window into the
//     slot of the k-th set bit (zero for clear bits), and the 0x6400 bias
//     turns each slot into exact fp16.
//   * The per-row scale is applied in the split-K epilogue shared with the
//     TCA-BME decode kernels.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "usw.h"
#include "usw_internal.h"
#include "usw_device.h"
#include "usw_decode_common.h"

namespace {

using namespace usw_dev;

constexpr int kLtWords = 16;                    // union words per 64x64 LT (32 x 32 bits)
constexpr int kUChunks = 3;                     // 1 KB value chunks per LT: payload <= 2 KB plus head
constexpr int kUVbuf = kUChunks * 1024 + 64;    // wave's LDS value buffer (+ what a window reads past it)
constexpr int kURowTab = 32 * 8;                // per logical row: its bits and the rank of its first bit
constexpr int kUWaves = 4;
constexpr int kUThreads = 64 * kUWaves;
static_assert(16 * 64 * kUChunks >= 4 * 1024 / 2 + 16, "every LT's payload fits a slot");
static_assert(kUThreads == 256, "one thread per entry of the selector table");

// Registers holding one LT's loads until they are copied into LDS.
template <int NB>
struct USlot {
  u32x4_t v[kUChunks];
  uint32_t rowbits;    // lane t: union row t % 32
  u32x4_t x[2][NB];
  uint32_t delta;      // payload elements before the LT's first one in its first piece
  uint32_t P;          // active union positions of the LT (wave-uniform)
};

// Issue the loads of LT column c of strip gi, whose payload occupies
// elements [o0, o1) of the stream.
template <int NB, int BITS>
__device__ __forceinline__ void uslot_load(USlot<NB>& s, const Args& a, int gi, int c, int lane, uint32_t o0,
                                           uint32_t o1) {
  const int64_t t = static_cast<int64_t>(gi) * a.Gc + c;
  // Union words first: the LT's row table is written while its payload and
  // X^T fragments may still be in flight.  Row r of the 32 x 32 mask is
  // dword r of the LT's words (little-endian 64-bit words, rows of 32 bits).
  s.rowbits = reinterpret_cast<const uint32_t*>(a.bitmaps + t * kLtWords)[lane & 31];
  // An LT holds at most 1024 active positions; the clamp keeps every window
  // inside the wave's LDS buffer even for offsets that disagree with the
  // union words.
  s.P = min((o1 - o0) >> 2, 1024u);
  const uint64_t top = a.values_alloc - 16;
  const uint64_t a0 = min(Packed<BITS>::chunk_start(o0), top);
  s.delta = Packed<BITS>::chunk_delta(o0, a0);
  const uint32_t nch = min(Packed<BITS>::chunk_count(o1, a0), static_cast<uint32_t>((kUVbuf - 16) / 16));
  // Buffer resources that end after the LT's last piece: pieces past it read
  // as zero, one vector offset (the lane's) for all chunks.  The size is
  // wave-uniform; saying so keeps the compiler from wrapping each load in a
  // loop over distinct descriptors.
  const uint32_t last = min(nch > 0 ? nch - 1 : 0u, static_cast<uint32_t>((top - a0) >> 4));
  const int span = __builtin_amdgcn_readfirstlane(static_cast<int>(16 * (last + 1)));
#pragma unroll
  for (int i = 0; i < kUChunks; ++i) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values + a0 + 1024 * i), 0,
                                                        max(span - 1024 * i, 0), kBufferRsrcWord3);
    s.v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * lane, 0, 0));
  }
  // X^T fragments; tokens past N repeat N-1 (they only feed outputs that are
  // never stored).
  const int row = lane & 15, kb = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = min(nb * 16 + row, a.N - 1);
      s.x[ks][nb] = *reinterpret_cast<const u32x4_t*>(a.X + static_cast<size_t>(n) * a.K + c * kGT + ks * 32 + kb * 8);
    }
}

// The row table of an LT: entry r = {row r's bits, element position of the
// row's first active value in the LDS buffer (area 0's stream)}.
__device__ __forceinline__ void urow_tab_write(uint8_t* tab, uint32_t rowbits, uint32_t base, int lane) {
  const uint32_t pc = lane < 32 ? __builtin_popcount(rowbits) : 0u;
  const uint32_t excl = wave_inclusive_scan(pc) - pc;
  if (lane < 32) {
    u32x2_t e;
    e.x = rowbits;
    e.y = base + excl;
    reinterpret_cast<u32x2_t*>(tab)[lane] = e;
  }
}

// Rebuild the 8 fragments of an LT whose row table is at tab and whose
// payload is in LDS, and multiply them with the X^T fragments.
template <int NB, int BITS>
__device__ __forceinline__ void union_tile_mma(const u32x4_t (&x)[2][NB], const uint8_t* smem, const uint8_t* tab,
                                               const u32x2_t* lut, uint32_t P, f32x4_t (&acc)[4][NB],
                                               f32x4_t (&corr)[NB], int lane) {
  code_offset_collect<NB>(corr, x);
  const int i = lane & 15;
  const uint32_t sh = 8u * static_cast<uint32_t>(lane >> 4);
  const uint32_t pmask = (1u << sh) - 1u;
  u32x2_t e[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) e[h] = reinterpret_cast<const u32x2_t*>(tab)[16 * h + i];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t byte = __builtin_amdgcn_ubfe(e[h].x, sh, 8);
    const uint32_t rb = e[h].y + __builtin_popcount(e[h].x & pmask);
    const u32x2_t sel = lut[byte];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const half8_t av = expand_row_i4(Packed<BITS>::window(smem, rb + static_cast<uint32_t>(q) * P), sel);
      const int f = 2 * (q >> 1) + h;   // area row q / 2, logical row half h
      const int ks = q & 1;             // area column
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[f][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8_t, x[ks][nb]), acc[f][nb],
                                                            0, 0, 0);
    }
  }
}

template <int NB, int BITS, bool OUT_F16, int OCC>
__global__ __launch_bounds__(kUThreads, OCC) void union_decode_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) u32x2_t lut[256];
  constexpr int kStage = kUWaves * (kUVbuf + kURowTab);
  constexpr int kRed = kUWaves * 4 * NB * 64 * 4 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStage > kRed ? kStage : kRed];
  __shared__ uint32_t last_flag;
  USW_LDS_POISON(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = static_cast<int>(gridDim.x);
  const int b = static_cast<int>(blockIdx.x);
  const int L = a.remap ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int gi = L / a.splits;
  const int sidx = L - gi * a.splits;

  lut[tid] = row_byte_selectors(static_cast<uint32_t>(tid));
  __syncthreads();

  const int parts = a.splits * kUWaves;
  const int qw = sidx * kUWaves + w;
  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * qw / parts);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (qw + 1) / parts);

  f32x4_t acc[4][NB];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[f][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t corr[NB];   // the code expansion offset's correction, same for every row
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) corr[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint8_t* vb = smem + w * kUVbuf;
  uint8_t* tab = smem + kUWaves * kUVbuf + w * kURowTab;
  // Windows address smem directly: the wave buffer's offset in payload
  // elements (nibbles) is folded into the row bases.
  const uint32_t vb_elems = static_cast<uint32_t>(w * kUVbuf) * Packed<BITS>::kPerByte;

  // The wave's LT offsets, lane i holding offsets[t_begin + i] (the host
  // keeps the count <= 63).
  const int cnt = c_end - c_begin;
  const int64_t t_begin = static_cast<int64_t>(gi) * a.Gc + c_begin;
  const uint32_t ov = a.offsets[t_begin + min(lane, max(cnt, 0))];
  auto off_at = [&](int c) -> uint32_t { return __builtin_amdgcn_readlane(ov, min(c - c_begin, 63)); };

  if (cnt > 0) {
    // Two register slots: LT c is in LDS while c+1 loads.  Loads past the
    // wave's last LT repeat it, so every step issues the same loads.
    const int c_last = c_end - 1;
    auto load = [&](USlot<NB>& sl, int c) {
      const int cc = min(c, c_last);
      uslot_load<NB, BITS>(sl, a, gi, cc, lane, off_at(cc), off_at(cc + 1));
    };
    auto commit = [&](const USlot<NB>& sl) {
#pragma unroll
      for (int i = 0; i < kUChunks; ++i) reinterpret_cast<u32x4_t*>(vb)[lane + 64 * i] = sl.v[i];
    };
    auto write_tab = [&](const USlot<NB>& sl) { urow_tab_write(tab, sl.rowbits, sl.delta + vb_elems, lane); };
    USlot<NB> s[2];
    load(s[0], c_begin);
    write_tab(s[0]);
    auto step = [&](USlot<NB>& cur, int c, USlot<NB>& nxt) {
      __builtin_amdgcn_s_setprio(2);   // loads first (see the TCA-BME decode step)
      load(nxt, c + 1);
      __builtin_amdgcn_s_setprio(0);
      commit(cur);
      wave_sync();
      union_tile_mma<NB, BITS>(cur.x, smem, tab, lut, cur.P, acc, corr, lane);
      wave_sync();
      write_tab(nxt);
    };
    int c = c_begin;
    for (; c + 2 <= c_end; c += 2) {
      step(s[0], c, s[1]);
      step(s[1], c + 1, s[0]);
    }
    if (c < c_end) step(s[0], c, s[1]);
  }

  // Workgroup reduction over waves (fixed order).
  code_offset_finish<NB>(corr);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [waves][4][NB][64 lanes][4]
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4_t*>(red + (((w * 4 + f) * NB + nb) * 64 + lane) * 4) =
          (acc[f][nb] + corr[nb]) * Packed<BITS>::kSumScale;
  __syncthreads();

  finish_strip<NB, true, OUT_F16>(a, gi, sidx, kUThreads, last_flag, [&](int n, int ml) {
    // Strip rows ml .. ml+3 are D rows 4g .. 4g+3 (g = (ml / 4) % 4) of
    // fragment ml / 16: registers 0-3 of lane 16 g + n % 16.
    const int f = ml >> 4;
    const int ln = 16 * ((ml >> 2) & 3) + (n & 15);
    const int nb = n >> 4;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < kUWaves; ++ww)
      sum += *reinterpret_cast<const f32x4_t*>(red + (((ww * 4 + f) * NB + nb) * 64 + ln) * 4);
    return sum;
  });
}

// ---------------------------------------------------------------------------
// 16 x 64 LTs (2 x 2 areas of 8 x 32), optionally with reordered rows
// ---------------------------------------------------------------------------
//
// The LT height the row-reordering solver handles.  Bitmap-aware row
// reordering ("UnionSparse", section on bitmap-aware row reordering)
// rearranges each LT's rows before compression, so the stored rows of one LT
// are a permutation of the rows of W it covers, a different one per LT.
// Partial products of different LTs can only be summed once they sit on the
// rows of W; here that happens before the products: the lane that holds row
// i of W in an MFMA fragment rebuilds it from the stored row the LT's rowmap
// names, so every accumulator row is a row of W across all LTs.
//
//   * One workgroup owns one 64-row strip (four LT rows) and a range of LT
//     columns; each of its waves streams its own run of columns, one column
//     ahead in registers.  A column step takes the four stacked LTs
//     f = 0..3 (LT row 4 gi + f): their union words, row maps and payloads
//     are four separate ranges, and the column's X^T fragments are loaded
//     once for all four.
//   * Fragment (f, ks) is LT f's 16 rows by area column ks.  Lane l
//     (i = l % 16, g = l / 16) holds row i of W within LT f and columns
//     8 g .. 8 g + 7 of the area column.  Its stored row is s = rowmap_f[i]
//     (s = i without a rowmap): logical union row s % 8, area row s / 8.  The
//     union byte g of that row, its rank (from a table of the four LTs' 8
//     rows, written with a DPP prefix scan) and its v_perm selectors serve
//     both area columns: the payload sits at rank + q P_f in streams
//     q = 2 (s / 8) + ks (the LSPD gather).
//   * One LT holds at most 4 x 256 nibbles, so one 16-byte piece per lane
//     covers its payload and head.

constexpr int kU16Vbuf = 1024 + 64;          // LDS payload buffer per LT (+ what a window reads past it)
constexpr int kU16Tab = 32 * 8;              // 4 LTs x 8 logical rows: bits and the rank of the first bit
constexpr int kU16Waves = 4;
constexpr int kU16Threads = 64 * kU16Waves;

template <int NB>
struct U16Slot {
  u32x4_t v[4];        // lane's 16-byte piece of LT f's payload
  uint32_t rowbits;    // lane l < 32: union row l % 8 of LT l / 8
  uint32_t srow[4];    // stored row of the lane's row of W in LT f (with a rowmap)
  u32x4_t x[2][NB];
  uint32_t delta[4];   // payload elements before LT f's first one in its first piece (wave-uniform)
  uint32_t P[4];       // active union positions of LT f (wave-uniform)
};

// Issue the loads of LT column c of strip gi; o0[f], o1[f] frame LT f's
// payload elements.
template <int NB, int BITS>
__device__ __forceinline__ void u16slot_load(U16Slot<NB>& s, const Args& a, int gi, int c, int lane,
                                             const uint32_t (&o0)[4], const uint32_t (&o1)[4]) {
  const int64_t t0 = static_cast<int64_t>(4 * gi) * a.Gc + c;   // LT f is t0 + f Gc
  // Union rows first (the rank table is written while the rest may still be
  // in flight): lane l < 32 loads dword l % 8 of LT l / 8's four words.
  const int fl = (lane >> 3) & 3;
  s.rowbits = reinterpret_cast<const uint32_t*>(a.bitmaps + (t0 + static_cast<int64_t>(fl) * a.Gc) * 4)[lane & 7];
  const int i = lane & 15;
  // The map byte of the lane's row in each LT, as vector loads: they are
  // counted in order with the slot's other loads, so the compute waits for
  // exactly this slot (scalar loads return out of order, and a wait for one
  // of them waits for all, the next slot's included).
  if (a.rowmap) {
#pragma unroll
    for (int f = 0; f < 4; ++f) s.srow[f] = a.rowmap[(t0 + static_cast<int64_t>(f) * a.Gc) * 16 + i];
  }
  const uint64_t top = a.values_alloc - 16;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    // At most 256 active positions; the clamp keeps windows inside the
    // buffer even for offsets that disagree with the union words.
    s.P[f] = min((o1[f] - o0[f]) >> 2, 256u);
    const uint64_t a0 = min(Packed<BITS>::chunk_start(o0[f]), top);
    s.delta[f] = Packed<BITS>::chunk_delta(o0[f], a0);
    const uint32_t nch = min(Packed<BITS>::chunk_count(o1[f], a0), static_cast<uint32_t>((kU16Vbuf - 16) / 16));
    const uint32_t last = min(nch > 0 ? nch - 1 : 0u, static_cast<uint32_t>((top - a0) >> 4));
    const int span = __builtin_amdgcn_readfirstlane(static_cast<int>(16 * (last + 1)));
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values + a0), 0, span, kBufferRsrcWord3);
    s.v[f] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * lane, 0, 0));
  }
  const int kb = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = min(nb * 16 + i, a.N - 1);
      s.x[ks][nb] = *reinterpret_cast<const u32x4_t*>(a.X + static_cast<size_t>(n) * a.K + c * kGT + ks * 32 + kb * 8);
    }
}

// Rank table of a column's four LTs: entry 8 f + r (r < 8) = {row r's bits,
// element position of the row's first active value in LDS (area 0's
// stream of LT f)}.  base[f]: where LT f's payload starts in LDS.
__device__ __forceinline__ void u16_tab_write(uint8_t* tab, uint32_t rowbits, const uint32_t (&base)[4], int lane) {
  const uint32_t pc = lane < 32 ? __builtin_popcount(rowbits) : 0u;
  const uint32_t excl = wave_inclusive_scan(pc) - pc;
  const uint32_t first = __shfl(excl, lane & ~7);   // the prefix at the LT's first row
  if (lane < 32) {
    const int f = lane >> 3;
    const uint32_t b = f == 0 ? base[0] : f == 1 ? base[1] : f == 2 ? base[2] : base[3];
    u32x2_t e;
    e.x = rowbits;
    e.y = b + excl - first;
    reinterpret_cast<u32x2_t*>(tab)[lane] = e;
  }
}

template <int NB, int BITS>
__device__ __forceinline__ void u16_tile_mma(const U16Slot<NB>& cur, bool mapped, const uint8_t* smem,
                                             const uint8_t* tab, const u32x2_t* lut, f32x4_t (&acc)[4][NB],
                                             f32x4_t (&corr)[NB], int lane) {
  code_offset_collect<NB>(corr, cur.x);
  const uint32_t sh = 8u * static_cast<uint32_t>(lane >> 4);
  const uint32_t pmask = (1u << sh) - 1u;
  const int i = lane & 15;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    // Stored row of the lane's row i of W: byte i of LT f's row map.
    const uint32_t srow = mapped ? (cur.srow[f] & 15u) : static_cast<uint32_t>(i);
    const u32x2_t e = reinterpret_cast<const u32x2_t*>(tab)[8 * f + (srow & 7u)];
    const uint32_t byte = __builtin_amdgcn_ubfe(e.x, sh, 8);
    const uint32_t rb = e.y + __builtin_popcount(e.x & pmask);
    const u32x2_t sel = lut[byte];
    const uint32_t q0 = 2u * (srow >> 3);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const half8_t av = expand_row_i4(Packed<BITS>::window(smem, rb + (q0 + ks) * cur.P[f]), sel);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[f][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8_t, cur.x[ks][nb]),
                                                            acc[f][nb], 0, 0, 0);
    }
  }
}

template <int NB, int BITS, bool OUT_F16, int OCC>
__global__ __launch_bounds__(kU16Threads, OCC) void union16_decode_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) u32x2_t lut[256];
  constexpr int kStage = kU16Waves * (4 * kU16Vbuf + kU16Tab);
  constexpr int kRed = kU16Waves * 4 * NB * 64 * 4 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStage > kRed ? kStage : kRed];
  __shared__ uint32_t last_flag;
  USW_LDS_POISON(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = static_cast<int>(gridDim.x);
  const int b = static_cast<int>(blockIdx.x);
  const int L = a.remap ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int gi = L / a.splits;
  const int sidx = L - gi * a.splits;

  lut[tid] = row_byte_selectors(static_cast<uint32_t>(tid));
  __syncthreads();

  // Columns of LTs this wave streams (the host keeps the count <= 15).
  const int parts = a.splits * kU16Waves;
  const int qw = sidx * kU16Waves + w;
  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * qw / parts);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (qw + 1) / parts);

  f32x4_t acc[4][NB];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[f][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t corr[NB];   // the code expansion offset's correction, same for every row
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) corr[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint8_t* vb = smem + w * 4 * kU16Vbuf;
  uint8_t* tab = smem + kU16Waves * 4 * kU16Vbuf + w * kU16Tab;
  // LT f's payload buffer, in elements (nibbles) from the start of smem.
  const uint32_t vb_elems = static_cast<uint32_t>(w * 4 * kU16Vbuf) * Packed<BITS>::kPerByte;

  // The LT offsets of the wave's columns: lane 16 f + j holds
  // offsets[(4 gi + f) Gc + c_begin + j] for j <= count.
  const int cnt = c_end - c_begin;
  const int fo = lane >> 4, jo = lane & 15;
  const uint32_t ov = a.offsets[static_cast<int64_t>(4 * gi + fo) * a.Gc + c_begin + min(jo, max(cnt, 0))];
  auto offs = [&](int c, uint32_t (&o0)[4], uint32_t (&o1)[4]) {
    const int j = min(c - c_begin, 15);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      o0[f] = __builtin_amdgcn_readlane(ov, 16 * f + j);
      o1[f] = __builtin_amdgcn_readlane(ov, 16 * f + min(j + 1, 15));
    }
  };

  const bool mapped = a.rowmap != nullptr;
  if (cnt > 0) {
    const int c_last = c_end - 1;
    auto load = [&](U16Slot<NB>& sl, int c) {
      const int cc = min(c, c_last);
      uint32_t o0[4], o1[4];
      offs(cc, o0, o1);
      u16slot_load<NB, BITS>(sl, a, gi, cc, lane, o0, o1);
    };
    auto commit = [&](const U16Slot<NB>& sl) {
#pragma unroll
      for (int f = 0; f < 4; ++f) reinterpret_cast<u32x4_t*>(vb + f * kU16Vbuf)[lane] = sl.v[f];
    };
    auto write_tab = [&](const U16Slot<NB>& sl) {
      uint32_t base[4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
        base[f] = sl.delta[f] + vb_elems + static_cast<uint32_t>(f * kU16Vbuf) * Packed<BITS>::kPerByte;
      u16_tab_write(tab, sl.rowbits, base, lane);
    };
    U16Slot<NB> s[2];
    load(s[0], c_begin);
    write_tab(s[0]);
    auto step = [&](U16Slot<NB>& cur, int c, U16Slot<NB>& nxt) {
      __builtin_amdgcn_s_setprio(2);   // loads first (see the TCA-BME decode step)
      load(nxt, c + 1);
      __builtin_amdgcn_s_setprio(0);
      commit(cur);
      wave_sync();
      u16_tile_mma<NB, BITS>(cur, mapped, smem, tab, lut, acc, corr, lane);
      wave_sync();
      write_tab(nxt);
    };
    int c = c_begin;
    for (; c + 2 <= c_end; c += 2) {
      step(s[0], c, s[1]);
      step(s[1], c + 1, s[0]);
    }
    if (c < c_end) step(s[0], c, s[1]);
  }

  // Workgroup reduction over waves (fixed order).
  code_offset_finish<NB>(corr);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [waves][4][NB][64 lanes][4]
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4_t*>(red + (((w * 4 + f) * NB + nb) * 64 + lane) * 4) =
          (acc[f][nb] + corr[nb]) * Packed<BITS>::kSumScale;
  __syncthreads();

  finish_strip<NB, true, OUT_F16>(a, gi, sidx, kU16Threads, last_flag, [&](int n, int ml) {
    // Strip rows ml .. ml+3 are D rows 4g .. 4g+3 (g = (ml / 4) % 4) of
    // LT ml / 16: registers 0-3 of lane 16 g + n % 16.
    const int f = ml >> 4;
    const int ln = 16 * ((ml >> 2) & 3) + (n & 15);
    const int nb = n >> 4;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < kU16Waves; ++ww)
      sum += *reinterpret_cast<const f32x4_t*>(red + (((ww * 4 + f) * NB + nb) * 64 + ln) * 4);
    return sum;
  });
}

// ---------------------------------------------------------------------------
// General area grids: LTs of 16, 32 or 64 rows by 64 columns, any R_A x C_A
// ---------------------------------------------------------------------------
//
// The section states IE-BME and the LSPD gather for a general R_A x C_A grid
// (Q = R_A C_A areas of (H_L / R_A) x (K_L / C_A)); the two kernels above are
// the 2 x 2 cases.  This one takes the grid at run time (powers of two, area
// width 8..64 columns, whole 64-bit words per LT) and the LT height as a
// template parameter, with or without row maps.
//
//   * One workgroup owns one 64-row strip, i.e. F = 64 / H_L stacked LTs, and
//     a range of LT columns; each wave streams its own run of columns one
//     column ahead in registers, as in the kernels above.
//   * Table row t < 64 / R_A of a column step is logical union row t % am of
//     the strip's LT t / am (am = H_L / R_A rows of ak = 64 / C_A bits): its
//     bits and the LDS element position of its first active value in area
//     stream 0 (a DPP prefix scan, segmented per LT).
//   * Fragment (fr, ks) holds strip rows 16 fr .. +15, i.e. rows of LT
//     fr / (H_L / 16); lane (i, g) holds row r of that LT and columns
//     kc = 32 ks + 8 g .. +7.  Its stored row s (rowmap, else r) lies in area
//     row s / am at logical row s % am; its columns lie in area column
//     kc / ak at logical columns kc % ak .. +7 (an area is at least 8 wide,
//     so one byte of the union row).  That byte's selectors and its rank
//     (row base + masked popcount) address stream q = (s / am) C_A + kc / ak
//     at rank + q P: one traversal and one rank for the row's values in
//     every area stream.

constexpr int kUGWaves = 4;
constexpr int kUGThreads = 64 * kUGWaves;
constexpr int kUGTab = 64 * 16;                // up to 64 table rows of {bits lo, bits hi, base, -}

// Per column step: F LTs of C 1 KB payload chunks each (payload <= H_L 64
// codes plus a 16-byte head).
template <int LTM, int BITS>
struct UGShape {
  static constexpr int F = 64 / LTM;
  static constexpr int C = (LTM * 64 * BITS / 8 + 16 + 1023) / 1024;
  static constexpr int NCH = F * C;
  static constexpr int kVbuf = NCH * 1024 + 64;   // + what a window reads past the last chunk
  static constexpr int kMaxCols = 64 / F - 1;     // LT columns per wave: offsets of F LT rows in one register
  static_assert(LTM == 16 || LTM == 32 || LTM == 64, "LT heights of 16, 32 or 64 rows");
  static_assert(NCH <= 4, "four payload chunks per step");
};

template <int NB, int NCH, int F>
struct UGSlot {
  u32x4_t v[NCH];      // lane's 16-byte piece of each payload chunk
  uint32_t lo, hi;     // lane t < 64 / R_A: table row t's union bits
  uint32_t srow[4];    // stored row of the lane's row of W, per fragment (with a rowmap)
  u32x4_t x[2][NB];
  uint32_t delta[F];   // payload elements before LT f's first one in its first piece (wave-uniform)
  uint32_t P[F];       // active union positions of LT f (wave-uniform)
};

// Issue the loads of LT column c of strip gi; o0[f], o1[f] frame LT f's
// payload elements.
template <int LTM, int NB, int BITS>
__device__ __forceinline__ void ugslot_load(UGSlot<NB, UGShape<LTM, BITS>::NCH, UGShape<LTM, BITS>::F>& s,
                                            const Args& a, int gi, int c, int lane,
                                            const uint32_t (&o0)[UGShape<LTM, BITS>::F],
                                            const uint32_t (&o1)[UGShape<LTM, BITS>::F]) {
  using S = UGShape<LTM, BITS>;
  const int64_t t0 = static_cast<int64_t>(S::F * gi) * a.Gc + c;   // LT f of the strip is t0 + f Gc
  // Union rows first (the table is written while the rest may still be in
  // flight).  Row lr of an LT is bits lr ak .. lr ak + ak - 1 of its words.
  {
    const int rows = S::F << a.lg_am;
    const int t = min(lane, rows - 1);
    const int f = t >> a.lg_am;
    const int lr = t & ((1 << a.lg_am) - 1);
    const int bit = lr << a.lg_ak;
    const int lg_wpl = a.lg_am + a.lg_ak - 6;
    uint64_t wd = a.bitmaps[((t0 + static_cast<int64_t>(f) * a.Gc) << lg_wpl) + (bit >> 6)];
    wd >>= (bit & 63);
    if (a.lg_ak < 6) wd &= (1ull << (1 << a.lg_ak)) - 1ull;
    if (lane >= rows) wd = 0;
    s.lo = static_cast<uint32_t>(wd);
    s.hi = static_cast<uint32_t>(wd >> 32);
  }
  const int i = lane & 15;
  // The map byte of the lane's row in each fragment, as vector loads (counted
  // in order with the slot's other loads).
  if (a.rowmap) {
#pragma unroll
    for (int fr = 0; fr < 4; ++fr) {
      const int f = fr / (LTM / 16);
      const int r = (fr % (LTM / 16)) * 16 + i;
      s.srow[fr] = a.rowmap[(t0 + static_cast<int64_t>(f) * a.Gc) * LTM + r];
    }
  }
  const uint64_t top = a.values_alloc - 16;
  const uint32_t pmax = static_cast<uint32_t>(LTM * 64) >> a.lg_q;
#pragma unroll
  for (int f = 0; f < S::F; ++f) {
    // The clamps keep windows inside the buffer even for offsets that
    // disagree with the union words.
    s.P[f] = min((o1[f] - o0[f]) >> a.lg_q, pmax);
    const uint64_t a0 = min(Packed<BITS>::chunk_start(o0[f]), top);
    s.delta[f] = Packed<BITS>::chunk_delta(o0[f], a0);
    const uint32_t nch = min(Packed<BITS>::chunk_count(o1[f], a0), static_cast<uint32_t>(S::C * 64));
    const uint32_t last = min(nch > 0 ? nch - 1 : 0u, static_cast<uint32_t>((top - a0) >> 4));
    const int span = __builtin_amdgcn_readfirstlane(static_cast<int>(16 * (last + 1)));
#pragma unroll
    for (int k = 0; k < S::C; ++k) {
      const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values + a0 + 1024 * k), 0,
                                                          max(span - 1024 * k, 0), kBufferRsrcWord3);
      s.v[f * S::C + k] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * lane, 0, 0));
    }
  }
  const int kb = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = min(nb * 16 + i, a.N - 1);
      s.x[ks][nb] = *reinterpret_cast<const u32x4_t*>(a.X + static_cast<size_t>(n) * a.K + c * kGT + ks * 32 + kb * 8);
    }
}

// Rank table of a column step: entry t = {row bits lo, hi, active union
// positions of its LT before the row}.  The reader adds where its LT's
// payload starts in LDS (wave-uniform), so no lane has to pick one of the
// F bases by a run-time index.
__device__ __forceinline__ void ug_tab_write(uint8_t* tab, uint32_t lo, uint32_t hi, int rows, int lg_am, int lane) {
  const uint32_t pc = __builtin_popcount(lo) + __builtin_popcount(hi);   // zero past the last row
  const uint32_t excl = wave_inclusive_scan(pc) - pc;
  const uint32_t first = __shfl(excl, lane & ~((1 << lg_am) - 1));      // the prefix at the LT's first row
  if (lane < rows) {
    u32x4_t e;
    e.x = lo;
    e.y = hi;
    e.z = excl - first;
    e.w = 0;
    reinterpret_cast<u32x4_t*>(tab)[lane] = e;
  }
}

template <int LTM, int NB, int BITS>
__device__ __forceinline__ void ug_tile_mma(const UGSlot<NB, UGShape<LTM, BITS>::NCH, UGShape<LTM, BITS>::F>& cur,
                                            const Args& a, bool mapped, const uint8_t* smem, const uint8_t* tab,
                                            const u32x2_t* lut, uint32_t vb_elems, f32x4_t (&acc)[4][NB],
                                            f32x4_t (&corr)[NB], int lane) {
  code_offset_collect<NB>(corr, cur.x);
  using S = UGShape<LTM, BITS>;
  const int i = lane & 15;
  const int g = lane >> 4;
  const uint32_t am_mask = (1u << a.lg_am) - 1u;
  const uint32_t ak_mask = (1u << a.lg_ak) - 1u;
#pragma unroll
  for (int fr = 0; fr < 4; ++fr) {
    constexpr int kFr = LTM / 16;             // fragments per LT
    const int f = fr / kFr;
    const uint32_t r = static_cast<uint32_t>((fr % kFr) * 16 + i);
    const uint32_t s = mapped ? (cur.srow[fr] & static_cast<uint32_t>(LTM - 1)) : r;
    const uint32_t ar = s >> a.lg_am;
    const u32x4_t e = reinterpret_cast<const u32x4_t*>(tab)[(f << a.lg_am) + (s & am_mask)];
    const uint64_t bits = static_cast<uint64_t>(e.x) | (static_cast<uint64_t>(e.y) << 32);
    // Where LT f's payload starts in LDS, in elements.
    const uint32_t lt_base = cur.delta[f] + vb_elems + static_cast<uint32_t>(f * S::C * 1024) * Packed<BITS>::kPerByte;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t kc = static_cast<uint32_t>(32 * ks + 8 * g);
      const uint32_t lc = kc & ak_mask;
      const uint32_t q = (ar << a.lg_ca) + (kc >> a.lg_ak);
      const uint32_t byte = static_cast<uint32_t>(bits >> lc) & 0xFFu;
      const uint64_t below = bits & ((1ull << lc) - 1ull);
      const uint32_t rb = lt_base + e.z + __builtin_popcount(static_cast<uint32_t>(below)) +
                          __builtin_popcount(static_cast<uint32_t>(below >> 32));
      const half8_t av = expand_row_i4(Packed<BITS>::window(smem, rb + q * cur.P[f]), lut[byte]);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[fr][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8_t, cur.x[ks][nb]),
                                                             acc[fr][nb], 0, 0, 0);
    }
  }
}

template <int LTM, int NB, int BITS, bool OUT_F16, int OCC>
__global__ __launch_bounds__(kUGThreads, OCC) void union_grid_decode_kernel(Args a) {
  using S = UGShape<LTM, BITS>;
  using Slot = UGSlot<NB, S::NCH, S::F>;
  __shared__ __attribute__((aligned(16))) u32x2_t lut[256];
  constexpr int kStage = kUGWaves * (S::kVbuf + kUGTab);
  constexpr int kRed = kUGWaves * 4 * NB * 64 * 4 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStage > kRed ? kStage : kRed];
  __shared__ uint32_t last_flag;
  USW_LDS_POISON(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = static_cast<int>(gridDim.x);
  const int b = static_cast<int>(blockIdx.x);
  const int L = a.remap ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int gi = L / a.splits;
  const int sidx = L - gi * a.splits;

  lut[tid] = row_byte_selectors(static_cast<uint32_t>(tid));
  __syncthreads();

  // Columns of LTs this wave streams (the host keeps the count <= kMaxCols).
  const int parts = a.splits * kUGWaves;
  const int qw = sidx * kUGWaves + w;
  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * qw / parts);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (qw + 1) / parts);

  f32x4_t acc[4][NB];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[f][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t corr[NB];   // the code expansion offset's correction, same for every row
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) corr[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint8_t* vb = smem + w * S::kVbuf;
  uint8_t* tab = smem + kUGWaves * S::kVbuf + w * kUGTab;
  // LT f's payload buffer, in elements from the start of smem.
  const uint32_t vb_elems = static_cast<uint32_t>(w * S::kVbuf) * Packed<BITS>::kPerByte;

  // The LT offsets of the wave's columns: lane (64 / F) f + j holds
  // offsets[(F gi + f) Gc + c_begin + j] for j <= count.
  constexpr int kLanesPerRow = 64 / S::F;
  const int cnt = c_end - c_begin;
  const int fo = lane / kLanesPerRow, jo = lane % kLanesPerRow;
  const uint32_t ov = a.offsets[static_cast<int64_t>(S::F * gi + fo) * a.Gc + c_begin + min(jo, max(cnt, 0))];
  auto offs = [&](int c, uint32_t (&o0)[S::F], uint32_t (&o1)[S::F]) {
    const int j = min(c - c_begin, kLanesPerRow - 1);
#pragma unroll
    for (int f = 0; f < S::F; ++f) {
      o0[f] = __builtin_amdgcn_readlane(ov, kLanesPerRow * f + j);
      o1[f] = __builtin_amdgcn_readlane(ov, kLanesPerRow * f + min(j + 1, kLanesPerRow - 1));
    }
  };

  const bool mapped = a.rowmap != nullptr;
  if (cnt > 0) {
    const int c_last = c_end - 1;
    auto load = [&](Slot& sl, int c) {
      const int cc = min(c, c_last);
      uint32_t o0[S::F], o1[S::F];
      offs(cc, o0, o1);
      ugslot_load<LTM, NB, BITS>(sl, a, gi, cc, lane, o0, o1);
    };
    auto commit = [&](const Slot& sl) {
#pragma unroll
      for (int k = 0; k < S::NCH; ++k) reinterpret_cast<u32x4_t*>(vb + k * 1024)[lane] = sl.v[k];
    };
    auto write_tab = [&](const Slot& sl) { ug_tab_write(tab, sl.lo, sl.hi, S::F << a.lg_am, a.lg_am, lane); };
    Slot s[2];
    load(s[0], c_begin);
    write_tab(s[0]);
    auto step = [&](Slot& cur, int c, Slot& nxt) {
      __builtin_amdgcn_s_setprio(2);   // loads first (see the TCA-BME decode step)
      load(nxt, c + 1);
      __builtin_amdgcn_s_setprio(0);
      commit(cur);
      wave_sync();
      ug_tile_mma<LTM, NB, BITS>(cur, a, mapped, smem, tab, lut, vb_elems, acc, corr, lane);
      wave_sync();
      write_tab(nxt);
    };
    int c = c_begin;
    for (; c + 2 <= c_end; c += 2) {
      step(s[0], c, s[1]);
      step(s[1], c + 1, s[0]);
    }
    if (c < c_end) step(s[0], c, s[1]);
  }

  // Workgroup reduction over waves (fixed order).
  code_offset_finish<NB>(corr);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [waves][4][NB][64 lanes][4]
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4_t*>(red + (((w * 4 + f) * NB + nb) * 64 + lane) * 4) =
          (acc[f][nb] + corr[nb]) * Packed<BITS>::kSumScale;
  __syncthreads();

  finish_strip<NB, true, OUT_F16>(a, gi, sidx, kUGThreads, last_flag, [&](int n, int ml) {
    // Strip rows ml .. ml+3 are D rows 4g .. 4g+3 (g = (ml / 4) % 4) of
    // fragment ml / 16: registers 0-3 of lane 16 g + n % 16.
    const int f = ml >> 4;
    const int ln = 16 * ((ml >> 2) & 3) + (n & 15);
    const int nb = n >> 4;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < kUGWaves; ++ww)
      sum += *reinterpret_cast<const f32x4_t*>(red + (((ww * 4 + f) * NB + nb) * 64 + ln) * 4);
    return sum;
  });
}

// ---------------------------------------------------------------------------
// Host dispatch
// ---------------------------------------------------------------------------

// Waves per SIMD the register allocation allows: 5 up to 16 tokens, 3 for
// 17..32 (twice the accumulators and X fragments), 2 for passes of 64
// tokens (64-row LTs with 2 x 2 areas only).
constexpr int kOcc1 = 5;
constexpr int kOcc2 = 3;
constexpr int kOcc4 = 2;

// Which kernel runs a format: the 2 x 2 kernels for their LT shapes, the
// area-grid kernel for the rest.
enum class UKind { kLt64, kLt16, kGrid };

struct UPlan {
  int splits;
  int nchunk;   // tokens per pass (16, 32, or 64 for the 64-row-LT 2 x 2 kernel)
  int rsplits;  // the same for the last pass when it is shorter (N > nchunk,
  int rchunk;   // N mod nchunk tokens in a pass of rchunk), else splits, 0
  UKind kind;
  int ltm;      // LT rows
};

// Waves per SIMD of the 16-row-LT kernel: 4 up to 16 tokens, 2 for 17..32.
constexpr int kOcc16a = 4;
constexpr int kOcc16b = 2;

// 64-row strips of the matrix (one workgroup's rows).
int64_t union_strips(const usw::UnionGeometry& g) { return g.M / 64; }

// Tokens per pass for n tokens on a kernel kind.
int union_chunk(UKind kind, int n) { return n <= 16 ? 16 : (n <= 32 || kind != UKind::kLt64) ? 32 : 64; }

// Split factor for passes of `chunk` tokens.
int union_splits(const usw::UnionGeometry& g, UKind kind, int chunk, int splits_req) {
  const int64_t strips = union_strips(g);
  // The four waves of a workgroup share its LT columns; a wave keeps the
  // offsets of at most 63 columns (64-row LTs), 31 (32-row LTs: two LT rows
  // per register) or 15 (16-row LTs: four LT rows per register).
  const int64_t per_split = kUWaves;
  const int64_t max_cols = g.lt_m - 1;
  const int occ = kind == UKind::kLt64 ? (chunk == 16 ? kOcc1 : chunk == 32 ? kOcc2 : kOcc4)
                                       : (chunk == 16 ? kOcc16a : kOcc16b);
  int64_t s = splits_req;
  if (s <= 0) {
    // About one round of resident workgroups, each wave keeping at least 3
    // LTs to stream.  Passes of 64 tokens with at most one strip per
    // compute unit: one workgroup per compute unit, as in the TCA-BME
    // decode (the split partial sums cost more than a second workgroup
    // gains).
    const int64_t target = 256 * 4 * occ / kUWaves;
    if (chunk == 64 && strips <= 256)
      s = 256 / strips;
    else
      s = std::max<int64_t>(1, (target + strips / 2) / strips);
    s = std::min<int64_t>(s, std::max<int64_t>(1, g.lc / (per_split * 3)));
  }
  const int64_t smax = std::max<int64_t>(1, g.lc / per_split);
  const int64_t smin = (g.lc + max_cols * per_split - 1) / (max_cols * per_split);
  return static_cast<int>(std::max(smin, std::max<int64_t>(1, std::min(s, smax))));
}

UPlan union_plan(const usw::UnionGeometry& g, bool mapped, int N, int splits_req) {
  UPlan p;
  p.ltm = static_cast<int>(g.lt_m);
  const bool two_by_two = g.r_a == 2 && g.c_a == 2;
  p.kind = (two_by_two && g.lt_m == 64 && !mapped) ? UKind::kLt64
           : (two_by_two && g.lt_m == 16)           ? UKind::kLt16
                                                    : UKind::kGrid;
  // One LT rebuild serves every token of a pass; the 64-row-LT kernel takes
  // passes of 64 tokens (one instead of two up to N = 64).
  p.nchunk = union_chunk(p.kind, N);
  p.splits = union_splits(g, p.kind, p.nchunk, splits_req);
  // A shorter last pass gets the split factor of its own size.
  const int rem = N > p.nchunk ? N % p.nchunk : 0;
  p.rchunk = rem > 0 ? union_chunk(p.kind, rem) : 0;
  p.rsplits = rem > 0 ? union_splits(g, p.kind, p.rchunk, splits_req) : p.splits;
  return p;
}

size_t union_counter_bytes(const usw::UnionGeometry& g) {
  return (static_cast<size_t>(4 * union_strips(g)) + 255) & ~size_t(255);
}

// Partial sums of the largest pass: splits x tokens of the pass x M fp32.
size_t union_workspace_bytes(const usw::UnionGeometry& g, const UPlan& p) {
  const size_t full = p.splits > 1 ? static_cast<size_t>(p.splits) * p.nchunk : 0;
  const size_t last = p.rchunk > 0 && p.rsplits > 1 ? static_cast<size_t>(p.rsplits) * p.rchunk : 0;
  const size_t cols = std::max(full, last);
  if (cols == 0) return 0;
  return union_counter_bytes(g) + cols * g.M * sizeof(float);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

usw_status union_check(const usw_union_fmt* f, int32_t y_type, int32_t N, usw::UnionGeometry* g) {
  if (!f) return USW_ERR_NULL_ARG;
  usw_status st = usw::make_union_geometry(f->M, f->K, f->lt_m, f->lt_k, f->r_a, f->c_a, g);
  if (st) return st;
  if (f->val_type != USW_VAL_F16 && f->val_type != USW_VAL_I4 && f->val_type != USW_VAL_I2) return USW_ERR_BAD_DTYPE;
  if (y_type != USW_OUT_F16 && y_type != USW_OUT_F32) return USW_ERR_BAD_DTYPE;
  if (f->reserved != 0) return USW_ERR_BAD_SHAPE;
  if (N < 1) return USW_ERR_BAD_N;
  // Low-bit payloads; LTs of 16, 32 or 64 rows by 64 columns stacked into
  // 64-row strips; areas at least 8 columns wide (one byte of a union row
  // per lane).  The geometry already holds R_A | H_L, C_A | 64 and whole
  // words per LT, so R_A and C_A are powers of two.
  if ((f->val_type != USW_VAL_I4 && f->val_type != USW_VAL_I2) || f->lt_k != 64) return USW_ERR_UNSUPPORTED;
  if ((f->lt_m != 16 && f->lt_m != 32 && f->lt_m != 64) || f->M % 64 || g->ak < 8) return USW_ERR_UNSUPPORTED;
  if (f->payload < 0 || f->payload >= (int64_t(1) << 32)) return USW_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(N) * g->M > (int64_t(1) << 40)) return USW_ERR_BAD_SHAPE;
  return USW_OK;
}

template <int LTM, int NB, int BITS>
void union_grid_launch(const Args& a, bool f16out, dim3 grid, hipStream_t s) {
  constexpr int occ = NB == 1 ? kOcc16a : kOcc16b;
  if (f16out)
    union_grid_decode_kernel<LTM, NB, BITS, true, occ><<<grid, kUGThreads, 0, s>>>(a);
  else
    union_grid_decode_kernel<LTM, NB, BITS, false, occ><<<grid, kUGThreads, 0, s>>>(a);
}

template <int NB, int BITS>
void union_launch(const Args& a, bool f16out, const UPlan& p, dim3 grid, hipStream_t s) {
  constexpr int occ = NB == 1 ? kOcc1 : NB == 2 ? kOcc2 : kOcc4;
  constexpr int occ16 = NB == 1 ? kOcc16a : kOcc16b;
  if constexpr (NB == 4) {
    // Passes of 64 tokens exist for the 64-row-LT 2 x 2 kernel only.
    if (f16out)
      union_decode_kernel<NB, BITS, true, occ><<<grid, kUThreads, 0, s>>>(a);
    else
      union_decode_kernel<NB, BITS, false, occ><<<grid, kUThreads, 0, s>>>(a);
  } else if (p.kind == UKind::kGrid) {
    if (p.ltm == 16) union_grid_launch<16, NB, BITS>(a, f16out, grid, s);
    else if (p.ltm == 32) union_grid_launch<32, NB, BITS>(a, f16out, grid, s);
    else union_grid_launch<64, NB, BITS>(a, f16out, grid, s);
  } else if (p.kind == UKind::kLt16) {
    if (f16out)
      union16_decode_kernel<NB, BITS, true, occ16><<<grid, kU16Threads, 0, s>>>(a);
    else
      union16_decode_kernel<NB, BITS, false, occ16><<<grid, kU16Threads, 0, s>>>(a);
  } else if (f16out) {
    union_decode_kernel<NB, BITS, true, occ><<<grid, kUThreads, 0, s>>>(a);
  } else {
    union_decode_kernel<NB, BITS, false, occ><<<grid, kUThreads, 0, s>>>(a);
  }
}

int log2i(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

}  // namespace

extern "C" {

usw_status usw_union_spmm_workspace(const usw_union_fmt* f, int32_t N, int32_t splits, size_t* bytes) {
  if (!bytes) return USW_ERR_NULL_ARG;
  usw::UnionGeometry g;
  usw_status st = union_check(f, USW_OUT_F16, N, &g);
  if (st) return st;
  *bytes = union_workspace_bytes(g, union_plan(g, f->rowmap != nullptr, N, splits < 0 ? 0 : splits));
  return USW_OK;
}

usw_status usw_union_spmm_counter_bytes(const usw_union_fmt* f, int32_t N, int32_t splits, size_t* bytes) {
  if (!bytes) return USW_ERR_NULL_ARG;
  usw::UnionGeometry g;
  usw_status st = union_check(f, USW_OUT_F16, N, &g);
  if (st) return st;
  *bytes = union_workspace_bytes(g, union_plan(g, f->rowmap != nullptr, N, splits < 0 ? 0 : splits)) > 0
               ? union_counter_bytes(g)
               : 0;
  return USW_OK;
}

usw_status usw_union_spmm(const usw_union_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N,
                          int32_t splits, void* ws, size_t ws_bytes, void* stream) {
  usw::UnionGeometry g;
  usw_status st = union_check(f, y_type, N, &g);
  if (st) return st;
  // The kernel reads whole 16-byte chunks of values even for an empty payload.
  if (!X || !Y || !f->bitmaps || !f->offsets || !f->scales || !f->values) return USW_ERR_NULL_ARG;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(f->bitmaps) || !aligned16(f->values)) return USW_ERR_MISALIGNED;
  const UPlan p = union_plan(g, f->rowmap != nullptr, N, splits < 0 ? 0 : splits);
  const size_t need = union_workspace_bytes(g, p);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return USW_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t ybytes = y_type == USW_OUT_F16 ? 2 : 4;
  const bool f16out = y_type == USW_OUT_F16;
  for (int n0 = 0; n0 < N; n0 += p.nchunk) {
    const int nc = std::min(p.nchunk, N - n0);
    // The shorter last pass of a multi-pass call has its own split factor.
    const int splits = (p.rchunk > 0 && n0 + p.nchunk > N) ? p.rsplits : p.splits;
    const int64_t nblk = union_strips(g) * splits;
    const dim3 grid(static_cast<unsigned>(nblk));
    Args a{};
    a.bitmaps = f->bitmaps;
    a.offsets = f->offsets;
    a.values = static_cast<const uint8_t*>(f->values);
    a.scales = f->scales;
    a.rowmap = f->rowmap;
    a.X = X + static_cast<size_t>(n0) * g.K;
    a.Y = static_cast<uint8_t*>(Y) + static_cast<size_t>(n0) * g.M * ybytes;
    a.counters = need ? static_cast<uint32_t*>(ws) : nullptr;
    a.part = need ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + union_counter_bytes(g)) : nullptr;
    a.values_alloc = usw::values_alloc_bytes(f->val_type, f->payload);
    a.M = static_cast<int>(g.M);
    a.K = static_cast<int>(g.K);
    a.N = nc;
    a.Gc = static_cast<int>(g.lc);
    a.splits = splits;
    a.remap = (splits > 1 && nblk % 8 == 0) ? 1 : 0;
    a.lg_am = log2i(g.am);
    a.lg_ak = log2i(g.ak);
    a.lg_ca = log2i(g.c_a);
    a.lg_q = log2i(g.Q);
    const bool i2 = f->val_type == USW_VAL_I2;
    if (nc > 32) {
      if (i2) union_launch<4, 2>(a, f16out, p, grid, s);
      else union_launch<4, 4>(a, f16out, p, grid, s);
    } else if (nc > 16) {
      if (i2) union_launch<2, 2>(a, f16out, p, grid, s);
      else union_launch<2, 4>(a, f16out, p, grid, s);
    } else {
      if (i2) union_launch<1, 2>(a, f16out, p, grid, s);
      else union_launch<1, 4>(a, f16out, p, grid, s);
    }
    if (hipGetLastError() != hipSuccess) return USW_ERR_HIP;
  }
  return USW_OK;
}

}  // extern "C"
