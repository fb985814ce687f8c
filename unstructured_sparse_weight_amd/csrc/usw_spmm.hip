// Device half of libusw: the bitmap SpMM decode kernels for gfx950 and the
// usw_spmm dispatcher.
//
// What is computed: Y[n][m] = sum_k W_sp[m][k] X[n][k], W_sp held in the
// TCA-BME bitmap format (blog "SpInfer: How bitmaps make sparse LLMs actually
// fast", section "How TCA-BME addresses the indexing overhead").  Values are
// located by masked popcount (same blog, "Shared Memory Bitmap Decoding").
//
// Two kernels: decode_ring_kernel (fp16 values, N <= 16, matrices at most
// 55% dense), in which a workgroup's waves share each GroupTile through an
// LDS ring filled by a loader wave (described where it is defined), and
// decode_kernel (everything else in decode), described here.  They share
// the rebuild and the split-K epilogue.
//
// Design of decode_kernel (gfx950, wave64):
//   * One workgroup owns one 64-row strip of GroupTiles (64x64) and a range
//     of GroupTile columns; each of its waves streams its own contiguous run
//     of GroupTiles (bitmaps and values of consecutive GroupTiles of a strip
//     are contiguous in memory), so the main loop has no workgroup barrier.
//   * Loads run one GroupTile ahead of the compute: the 16-byte global loads
//     of GroupTile c+1 (bitmaps, the value range [offsets[g], offsets[g+1])
//     from a 16-byte aligned start, and the X^T fragments) sit in registers
//     while GroupTile c, already copied into the wave's private LDS buffer,
//     is rebuilt and multiplied.  Every load is issued unconditionally
//     (clamped indices), so the compiler waits for exactly the slot in use.
//   * Rebuild: v_mfma_f32_16x16x32_f16 gives lane l 8 consecutive columns
//     8*(l/16)..+7 of one row of a 16x32 block, which is exactly one row of
//     one BitmapTile; its kept values are contiguous in the stream.  A
//     fragment is one TCTile row (16 strip rows) by four BitmapTile columns,
//     so the 32 lanes the LDS serves together read rows of a single TCTile,
//     whose values are contiguous (few bank conflicts).  Where each
//     BitmapTile's values start (GroupTile offset + a DPP wave prefix scan of
//     the BitmapTile popcounts) goes with its bitmap words into a small LDS
//     table one GroupTile ahead; a lane reads its row's word and base, adds
//     the popcount of the earlier rows, and expands the row into 8 slots with
//     two aligned LDS windows and v_perm_b32 byte selectors looked up by the
//     row's 4-bit halves (zero for clear bits).
//   * The rebuilt fragment meets the X^T fragment (X is [N][K], so each
//     lane's 8 k values are one 16-byte load) on the matrix cores with fp32
//     accumulation, which leaves the vector ALUs to the rebuild.
//   * Partial sums of the waves of a workgroup are added in LDS in a fixed
//     order.  Split K (several workgroups per strip): each writes its sums to
//     an fp32 workspace with device-coherent stores and the last workgroup of
//     the strip, found with a per-strip counter, adds them in split order, so
//     results do not depend on scheduling.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "usw.h"
#include "usw_internal.h"
#include "usw_device.h"
#include "usw_decode_common.h"

// Scratch of usw_spmm_noalloc (see scratch_address below): split-K counters
// and partial sums, one copy per GPU, kept until the process ends.
static __device__ __align__(256) uint8_t scratch[size_t(16) << 20];

namespace {

using namespace usw_dev;

// Value slot constants: CH 1 KB chunks per GroupTile, i.e. 64 lanes x 16 B
// per chunk.  fp16 takes 5 chunks (GroupTiles up to ~62% dense) when the
// matrix is at most 55% dense on average, else 6 (~74%); INT4 takes 3, which
// every GroupTile fits (<= 2 KB + head).  Denser GroupTiles are staged in two
// halves of two TCTile rows each (<= 4 KB + head).  Every chunk load is
// issued unconditionally, so the loads carry no branches and the compiler
// waits for exactly the slot being consumed.
template <bool I4, int CH>
struct ValTraits {
  static constexpr int kChunks = CH;
  // LDS value buffer per wave: one slot plus the <16 B a window reads past
  // the last value.
  static constexpr int kVbuf = CH * 1024 + 64;
  static constexpr uint32_t kFastLimit = I4 ? 4096u : (16u * 64u * CH - 32u) / 2u;   // values per GroupTile
  static_assert(I4 || kVbuf >= 16 * 257 + 16, "a half GroupTile fits");
  static_assert(!I4 || kFastLimit / 2 + 16 <= 1024 * CH, "every INT4 GroupTile fits");
};

// Registers holding one GroupTile's loads until they are copied into LDS.
template <int NB, bool I4, int CH>
struct Slot {
  u32x4_t v[CH];
  u32x2_t bm;       // lane t: bitmap word t of the GroupTile
  u32x4_t x[2][NB];
  uint32_t nch;     // 16-byte pieces of values spanned (wave-uniform)
  uint32_t delta;   // value elements before the GroupTile's first one in its first piece
  uint64_t a0;      // byte offset of the first piece
};


// Issue the loads of GroupTile c of strip gi, whose values occupy elements
// [o0, o1) of the stream.
template <int NB, bool I4, int CH>
__device__ __forceinline__ void slot_load(Slot<NB, I4, CH>& s, const Args& a, int gi, int c, int lane, uint32_t o0,
                                          uint32_t o1) {
  using VT = ValTraits<I4, CH>;
  const int64_t g = static_cast<int64_t>(gi) * a.Gc + c;
  // Bitmaps first: the bitmap table of a slot is written while its values
  // and X^T fragments may still be in flight.
  s.bm = reinterpret_cast<const u32x2_t*>(a.bitmaps + g * kBtPerGt)[lane];
  // The clamps keep every load inside the padded allocation and every store
  // inside the LDS buffer even for offsets that disagree with the bitmaps.
  const uint64_t top = a.values_alloc - 16;
  s.a0 = min(chunk_start<I4>(o0), top);
  s.delta = chunk_delta<I4>(o0, s.a0);
  s.nch = min(chunk_count<I4>(o1, s.a0), static_cast<uint32_t>((VT::kVbuf - 16) / 16));
  // The values go through buffer resources, one per chunk, that end after
  // the GroupTile's last piece (piece 0 of an empty GroupTile lies inside the
  // padded allocation): pieces past it read as zero, with no clamp per piece
  // and one vector offset (the lane's) for all chunks.
  const uint32_t last = min(s.nch > 0 ? s.nch - 1 : 0u, static_cast<uint32_t>((top - s.a0) >> 4));
  const int span = static_cast<int>(16 * (last + 1));
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.values + s.a0 + 1024 * i), 0,
                                                        max(span - 1024 * i, 0), kBufferRsrcWord3);
    s.v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, 16 * lane, 0, 0));
  }
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

template <int NB, bool I4, int CH>
__device__ __forceinline__ void slot_commit(const Slot<NB, I4, CH>& s, uint8_t* vb, int lane) {
#pragma unroll
  for (int i = 0; i < CH; ++i) reinterpret_cast<u32x4_t*>(vb)[lane + 64 * i] = s.v[i];
}

// Which rows a lane rebuilds.  Fragment (f, ks) of a GroupTile (f = 0..3,
// ks = 0, 1) is the 16 x 32 block of strip rows 16f .. 16f+15 and GroupTile
// columns 32ks .. 32ks+31.  Lane l with i = l % 16 and g = l / 16 holds row i,
// columns 8g .. 8g+7 of the block, which is row r = i % 8 of the BitmapTile
// in BitmapTile row R = 2f + i / 8 and BitmapTile column C = 4ks + g.  The
// 32 lanes that the LDS serves together (g = 0, 1 or g = 2, 3) thus read the
// rows of one TCTile, whose values are contiguous, so their windows spread
// over few bytes and few bank conflicts; and D row i of fragment f is strip
// row 16f + i.
struct LaneMap {
  uint32_t tab;     // byte offset of the lane's entry for f = ks = 0 in the bitmap table
  uint32_t sh;      // 8 (r % 4): bit offset of row r in its bitmap word
  uint32_t pmask;   // bits of the rows before r in that word
};

__device__ __forceinline__ LaneMap lane_map(int lane) {
  const int i = lane & 15, g = lane >> 4, r = i & 7;
  // BitmapTile (R, C) is number 16 (R / 2) + 4 (C / 2) + 2 (R % 2) + C % 2 in
  // storage order (TCTiles row-major, BitmapTiles row-major inside them);
  // fragment (f, ks) adds 16 f + 8 ks to the BitmapTile number below.
  const int bt = 4 * (g >> 1) + 2 * (i >> 3) + (g & 1);
  LaneMap m;
  m.tab = 16u * static_cast<uint32_t>(bt) + 8u * static_cast<uint32_t>(r >> 2);
  m.sh = 8u * static_cast<uint32_t>(r & 3);
  m.pmask = (1u << m.sh) - 1u;
  return m;
}

constexpr int kTabBytes = 16 * kBtPerGt;

// Bitmap table of a GroupTile in LDS, 16 bytes per BitmapTile, written by
// lane t for BitmapTile t: bitmap rows 0-3, where row 0's values start,
// bitmap rows 4-7, where row 4's values start (value positions counted in
// elements from the start of the staging area).  base is where the
// BitmapTile's values start.
__device__ __forceinline__ void tab_write(uint8_t* tab, u32x2_t bm, uint32_t base, int lane) {
  u32x4_t e;
  e.x = bm.x;
  e.y = base;
  e.z = bm.y;
  e.w = base + __builtin_popcount(bm.x);
  reinterpret_cast<u32x4_t*>(tab)[lane] = e;
}

// Exclusive prefix of the BitmapTile popcounts of a GroupTile from the
// slot's registers (lane t holds bitmap word t).
__device__ __forceinline__ uint32_t bitmap_prefix_reg(u32x2_t bm) {
  const uint32_t pc = __builtin_popcount(bm.x) + __builtin_popcount(bm.y);
  return wave_inclusive_scan(pc) - pc;
}

// Rebuild and multiply fragments f = F0 .. F1-1 (both ks) of a GroupTile
// whose bitmap table is at tab and whose values are in the LDS staging area
// starting at vals.  INT4 rows carry the expansion's offset: corr collects
// its correction (code_offset_collect, all four fragments of a GroupTile at once).
template <int NB, bool I4, int F0 = 0, int F1 = 4>
__device__ __forceinline__ void tile_mma(const u32x4_t (&x)[2][NB], const uint8_t* vals, const uint8_t* tab,
                                         const uint32_t* lut, f32x4_t (&acc)[4][NB], f32x4_t (&corr)[NB],
                                         const LaneMap& lm) {
  static_assert(!I4 || (F0 == 0 && F1 == 4), "the INT4 correction covers whole GroupTiles");
  if constexpr (I4) code_offset_collect<NB>(corr, x);
  u32x2_t e[F1 - F0][2];
#pragma unroll
  for (int f = F0; f < F1; ++f)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      e[f - F0][ks] = *reinterpret_cast<const u32x2_t*>(tab + lm.tab + 256 * f + 128 * ks);
#pragma unroll
  for (int f = F0; f < F1; ++f)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint32_t word = e[f - F0][ks].x;
      const uint32_t rb = e[f - F0][ks].y + __builtin_popcount(word & lm.pmask);
      const half8_t a = rebuild_row<I4>(vals, lut, rb, __builtin_amdgcn_ubfe(word, lm.sh, 8));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[f][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(half8_t, x[ks][nb]), acc[f][nb], 0,
                                                            0, 0);
    }
}

// Launch shape of the decode kernel: waves per workgroup, GroupTiles loaded
// ahead of the one being computed (1 or 2), and the minimum waves per SIMD
// the register allocation must allow.
template <int WAVES_, int DEPTH_, int OCC_>
struct Cfg {
  static constexpr int kWavesPerGroup = WAVES_;
  static constexpr int kDepth = DEPTH_;
  static constexpr int kOcc = OCC_;
  static constexpr int kThreadsPerGroup = 64 * WAVES_;
};

template <int NB, bool I4, int CH, bool OUT_F16, class C>
__global__ __launch_bounds__(C::kThreadsPerGroup, C::kOcc) void decode_kernel(Args a) {
  using VT = ValTraits<I4, CH>;
  constexpr int kW = C::kWavesPerGroup;
  constexpr int kThreads = C::kThreadsPerGroup;
  constexpr int kD = C::kDepth;
  // Row selectors: fp16 16 nibble entries of two dwords, INT4 256 byte
  // entries of two dwords.
  __shared__ __attribute__((aligned(16))) uint32_t lut[I4 ? 512 : 32];
  // Staging (per wave: values, then the bitmap table); reused for the final
  // reduction.
  constexpr int kStage = kW * (VT::kVbuf + kTabBytes);
  constexpr int kRed = kW * 4 * NB * 64 * 4 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStage > kRed ? kStage : kRed];
  __shared__ uint32_t last_flag;
  USW_LDS_POISON(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // The wave index is uniform across the wave; saying so keeps the wave's
  // GroupTile range, its offsets and the loop control scalar.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Workgroups are dealt to the 8 XCDs round robin; with remap the splits of
  // one strip land on the same XCD (one L2 for their partial sums).
  const int nblk = static_cast<int>(gridDim.x);
  const int b = static_cast<int>(blockIdx.x);
  const int L = a.remap ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int gi = L / a.splits;
  const int sidx = L - gi * a.splits;

  if (tid < 16) {
    if constexpr (!I4) {
      u32x2_t e;
      e.x = nibble_selector(tid, 0);
      e.y = nibble_selector(tid, 1);
      reinterpret_cast<u32x2_t*>(lut)[tid] = e;
    }
  }
  if constexpr (I4) {
    for (int i = tid; i < 256; i += kThreads) reinterpret_cast<u32x2_t*>(lut)[i] = row_byte_selectors(i);
  }
  __syncthreads();

  // Columns of GroupTiles this wave streams.
  const int parts = a.splits * kW;
  const int q = sidx * kW + w;
  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * q / parts);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (q + 1) / parts);

  const LaneMap lm = lane_map(lane);

  f32x4_t acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t corr[NB];   // INT4: the expansion offset's correction, same for every row
#pragma unroll
  for (int j = 0; j < NB; ++j) corr[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint8_t* vb = smem + w * VT::kVbuf;
  uint8_t* tab = smem + kW * VT::kVbuf + w * kTabBytes;
  // The rebuild addresses the wave's value buffer from smem: its offset, in
  // value elements, is folded into the BitmapTile bases.
  const uint32_t vb_elems = I4 ? static_cast<uint32_t>(w * VT::kVbuf * 2) : static_cast<uint32_t>(w * VT::kVbuf / 2);

  // The wave's GroupTile offsets, one per lane: lane i holds
  // offsets[g_begin + i] for i <= count (the host keeps count <= 63), so a
  // slot's value range comes from two v_readlane.
  const int cnt = c_end - c_begin;
  const int64_t g_begin = static_cast<int64_t>(gi) * a.Gc + c_begin;
  const uint32_t ov = a.offsets[g_begin + min(lane, max(cnt, 0))];
  auto off_at = [&](int c) -> uint32_t { return __builtin_amdgcn_readlane(ov, min(c - c_begin, 63)); };

  // A wave may own no GroupTile column (K < 64 * waves): it only joins the
  // reduction.  A GroupTile whose values span more chunks than a slot holds
  // (fp16 density above ~74%) sends the whole wave down the unpipelined path.
  const uint32_t ov_next = __shfl_down(ov, 1);
  const uint32_t widest = wave_max(lane < cnt ? ov_next - ov : 0u);

  // The bitmap table of the GroupTile in slot s.
  auto write_tab = [&](const Slot<NB, I4, CH>& s) {
    tab_write(tab, s.bm, bitmap_prefix_reg(s.bm) + s.delta + vb_elems, lane);
  };

  if (cnt <= 0) {
    // nothing to stream
  } else if (widest > VT::kFastLimit) {
    if constexpr (!I4) {
      // Unpipelined: per GroupTile, the values of TCTile rows 0-1 (fragments
      // f = 0, 1), then those of TCTile rows 2-3 (f = 2, 3), each staged in
      // the wave's buffer with its own bitmap table bases.
      const uint64_t top = a.values_alloc - 16;
      for (int c = c_begin; c < c_end; ++c) {
        const uint32_t o0 = off_at(c), o1 = off_at(c + 1);
        Slot<NB, I4, CH> s0;
        slot_load(s0, a, gi, c, lane, o0, o1);
        const uint32_t excl = bitmap_prefix_reg(s0.bm);
        const uint32_t mid = __builtin_amdgcn_readlane(excl, 32);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t hs = o0 + (h ? mid : 0u);
          const uint32_t he = h ? o1 : o0 + mid;
          const uint64_t a0 = min(chunk_start<I4>(hs), top);
          const uint32_t delta = chunk_delta<I4>(hs, a0);
          const uint32_t nch = min(chunk_count<I4>(he, a0), static_cast<uint32_t>((VT::kVbuf - 16) / 16));
          const uint32_t last = static_cast<uint32_t>((top - a0) >> 4);
          const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.values + a0);
          for (uint32_t ch = lane; ch < nch; ch += 64) reinterpret_cast<u32x4_t*>(vb)[ch] = src[min(ch, last)];
          // Entries of the other half get bases that are never read.
          tab_write(tab, s0.bm, excl - (h ? mid : 0u) + delta + vb_elems, lane);
          wave_sync();
          if (h == 0)
            tile_mma<NB, I4, 0, 2>(s0.x, smem, tab, lut, acc, corr, lm);
          else
            tile_mma<NB, I4, 2, 4>(s0.x, smem, tab, lut, acc, corr, lm);
          wave_sync();
        }
      }
    }
  } else if constexpr (kD == 0) {
    // One register slot: GroupTile c is copied into LDS, then the loads of
    // c+1 are issued into the same registers while c is rebuilt and
    // multiplied.  Fewer registers, more waves per SIMD.
    const int c_last = c_end - 1;
    Slot<NB, I4, CH> s0;
    slot_load(s0, a, gi, c_begin, lane, off_at(c_begin), off_at(c_begin + 1));
    write_tab(s0);
    for (int c = c_begin; c < c_end; ++c) {
      slot_commit(s0, vb, lane);
      u32x4_t xc[2][NB];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) xc[ks][nb] = s0.x[ks][nb];
      const int cn = min(c + 1, c_last);
      slot_load(s0, a, gi, cn, lane, off_at(cn), off_at(cn + 1));
      wave_sync();
      tile_mma<NB, I4>(xc, smem, tab, lut, acc, corr, lm);
      wave_sync();
      write_tab(s0);
    }
  } else {
    // kD + 1 register slots: GroupTile c is in LDS while c+1 .. c+kD load.
    // Loads past the wave's last GroupTile repeat it (every wave here owns at
    // least one), so each step issues the same loads and waits for exactly
    // one slot.  A step issues the loads of c+kD before it waits for c, and
    // ends by writing the bitmap table of c+1 (the bitmaps are the first
    // load of a slot, long arrived by then).
    constexpr int kS = kD + 1;
    const int c_last = c_end - 1;
    auto load = [&](Slot<NB, I4, CH>& sl, int c) {
      const int cc = min(c, c_last);
      slot_load(sl, a, gi, cc, lane, off_at(cc), off_at(cc + 1));
    };
    Slot<NB, I4, CH> s[kS];
#pragma unroll
    for (int j = 0; j < kD; ++j) load(s[j], c_begin + j);
    write_tab(s[0]);
    // The loads go out at a raised wave priority, so a wave that reaches
    // them is not held behind the other waves' rebuild work (measured on
    // MI355X: INT4 20480x5120 N = 2 19.5 -> 19.0 us, N = 32 41.4 -> 40.1,
    // 11008x4096 N = 64 30.7 -> 28.3).
    auto step = [&](Slot<NB, I4, CH>& cur, int c, Slot<NB, I4, CH>& nxt, const Slot<NB, I4, CH>& after) {
      __builtin_amdgcn_s_setprio(2);
      load(nxt, c + kD);
      __builtin_amdgcn_s_setprio(0);
      slot_commit(cur, vb, lane);
      wave_sync();
      tile_mma<NB, I4>(cur.x, smem, tab, lut, acc, corr, lm);
      wave_sync();
      write_tab(after);
    };
    int c = c_begin;
    for (; c + kS <= c_end; c += kS) {
#pragma unroll
      for (int j = 0; j < kS; ++j) step(s[j], c + j, s[(j + kD) % kS], s[(j + 1) % kS]);
    }
#pragma unroll
    for (int j = 0; j < kD; ++j)
      if (c + j < c_end) step(s[j], c + j, s[(j + kD) % kS], s[(j + 1) % kS]);
  }

  // Workgroup reduction over waves (fixed order).
  if constexpr (I4) code_offset_finish<NB>(corr);
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [waves][4][NB][64 lanes][4]
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4_t*>(red + (((w * 4 + f) * NB + nb) * 64 + lane) * 4) =
          I4 ? acc[f][nb] + corr[nb] : acc[f][nb];
  __syncthreads();

  finish_strip<NB, I4, OUT_F16>(a, gi, sidx, kThreads, last_flag, [&](int n, int ml) {
    // Strip rows ml .. ml+3 are D rows 4g .. 4g+3 (g = (ml / 4) % 4) of
    // fragment ml / 16: registers 0-3 of lane 16 g + n % 16.
    const int f = ml >> 4;
    const int ln = 16 * ((ml >> 2) & 3) + (n & 15);
    const int nb = n >> 4;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < kW; ++ww)
      sum += *reinterpret_cast<const f32x4_t*>(red + (((ww * 4 + f) * NB + nb) * 64 + ln) * 4);
    return sum;
  });
}

// ---------------------------------------------------------------------------
// Workgroup-cooperative decode: fp16 values, N <= 16, matrices at most 55%
// dense on average
// ---------------------------------------------------------------------------
//
// One workgroup is four compute waves and two loader waves over one strip's
// range of GroupTile columns; all six pass one barrier per GroupTile.
//  * Wave 4 moves each GroupTile's values and X^T column, and the bitmap
//    words of the GroupTile after, straight into a ring of R LDS slots with
//    global_load_lds_dwordx4, R - 1 GroupTiles ahead, so no register holds
//    them in flight.  It waits for its own loads with explicit vmcnt counts
//    before each barrier.
//  * Wave 5 writes the bitmap table of the next GroupTile into its slot.
//  * Compute wave q (0-3) rebuilds fragments f = 2 (q / 2) and 2 (q / 2) + 1
//    for ks = q % 2: two rows per lane per GroupTile, and multiplies them
//    with its X^T fragment, which wave 4 also stages in the slot.  The MFMA B
//    layout puts a different token in each of four consecutive lanes, so as
//    a global load every compute wave's fragment would cost four times the
//    address-unit cycles of a contiguous one; the compute waves issue no
//    global loads at all.
// A workgroup whose range holds a GroupTile too wide for a slot runs the
// range unpipelined, half a GroupTile (two TCTile rows) at a time in slot 0.

constexpr int kRingVals = 5 * 1024 + 64;                 // value bytes per slot
constexpr int kRingX = 2048;                             // X^T of one GroupTile column, 16 tokens
constexpr int kRingSlot = kRingVals + 512 + kTabBytes + kRingX;   // + bitmap words, table, X^T
constexpr uint32_t kRingPieces = 5 * 64;                 // 16-byte value pieces a slot takes
constexpr uint32_t kRingFast = (16u * kRingPieces - 32u) / 2u;   // values per GroupTile that fit a slot
constexpr int kRingThreads = 384;
static_assert(kRingSlot % 16 == 0, "slots keep 16-byte alignment");
static_assert(16 * kRingPieces + 16 <= kRingVals, "windows past the last piece stay in the slot");

template <int R, bool OUT_F16>
__global__ __launch_bounds__(kRingThreads, 5) void decode_ring_kernel(Args a) {
  constexpr int NB = 1;
  constexpr int kRed = 2 * 4 * 64 * 16;          // [ks][f][64 lanes][4] fp32
  constexpr int kRing = R * kRingSlot;
  __shared__ __attribute__((aligned(16))) uint32_t lut[32];
  __shared__ __attribute__((aligned(16))) uint8_t smem[kRing > kRed ? kRing : kRed];
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

  if (tid < 16) {
    u32x2_t e;
    e.x = nibble_selector(tid, 0);
    e.y = nibble_selector(tid, 1);
    reinterpret_cast<u32x2_t*>(lut)[tid] = e;
  }
  __syncthreads();

  // The workgroup's GroupTile columns (the host keeps 1 <= count <= 63) and
  // their offsets, lane i holding offsets[g_begin + i].
  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * sidx / a.splits);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (sidx + 1) / a.splits);
  const int cnt = c_end - c_begin;
  const int64_t g_begin = static_cast<int64_t>(gi) * a.Gc + c_begin;
  const uint32_t ov = a.offsets[g_begin + min(lane, cnt)];
  auto off_at = [&](int c) -> uint32_t { return __builtin_amdgcn_readlane(ov, min(c - c_begin, 63)); };
  // The shuffle runs in all lanes (a lane reading an inactive one gets 0).
  const uint32_t ov_next = __shfl_down(ov, 1);
  const uint32_t widest = wave_max(lane < cnt ? ov_next - ov : 0u);

  const int role = w < 4 ? 0 : w - 3;   // 0 compute, 1 loads, 2 bitmap tables
  const uint64_t top = a.values_alloc - 16;
  auto slot_vals = [&](int s) { return smem + s * kRingSlot; };
  auto slot_bm = [&](int s) { return smem + s * kRingSlot + kRingVals; };
  auto slot_tab = [&](int s) { return smem + s * kRingSlot + kRingVals + 512; };
  auto slot_x = [&](int s) { return smem + s * kRingSlot + kRingVals + 512 + kTabBytes; };

  // Loader: the bitmap words of GroupTile c (lanes 0-31, 16 bytes each) into
  // slot s; one load.
  auto issue_bm = [&](int c, int s) {
    const int64_t g = static_cast<int64_t>(gi) * a.Gc + c;
    if (lane < 32) lds_dma16_tracked(a.bitmaps + g * kBtPerGt + 2 * lane, slot_bm(s));
  };
  // Loader: value elements [e0, e1) into slot s, from the 16-byte piece
  // holding e0 on; returns the number of loads (1 KB each).  Pieces past the
  // range repeat its last one, and the range is cut to what a slot takes.
  auto issue_vals = [&](uint32_t e0, uint32_t e1, int s) -> int {
    const uint64_t a0 = min(chunk_start<false>(e0), top);
    const uint32_t pieces = min(chunk_count<false>(e1, a0), kRingPieces);
    const uint32_t last = min(pieces > 0 ? pieces - 1 : 0u, static_cast<uint32_t>((top - a0) >> 4));
    const int nl = static_cast<int>((pieces + 63) / 64);
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.values + a0);
    for (int i = 0; i < nl; ++i) lds_dma16_tracked(src + min(64u * i + lane, last), slot_vals(s) + 1024 * i);
    return nl;
  };
  // Loader: X^T of GroupTile column c (16 tokens x 64 k) into slot s, two
  // loads of 1 KB, one per k half.  Four consecutive lanes read one token's
  // 64 contiguous bytes of the half (one address-unit cycle, where the MFMA
  // B layout would take four); their pieces are rotated by token / 4 so that
  // the compute waves' 16-lane reads of B fragments fall in 16 different
  // bank groups.  Lane 4j + t holds piece (t - j/4) mod 4 of token j.
  auto issue_x = [&](int c, int s) {
    const int j = lane >> 2, t = lane & 3;
    const int piece = (t - (j >> 2)) & 3;
    const uint16_t* src = a.X + static_cast<size_t>(min(j, a.N - 1)) * a.K + c * kGT + piece * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) lds_dma16_tracked(src + 32 * i, slot_x(s) + 1024 * i);
  };
  // The bitmap table of the value range starting at element e0 whose bitmaps
  // are in slot s; `skip` values of the GroupTile precede the range.  Its LDS
  // accesses are asm, so that in the wave that issues the LDS-DMA loads they
  // do not wait for those in flight.
  auto build_tab = [&](uint32_t e0, uint32_t skip, int s) {
    const u32x2_t bm = lds_load_b64(lds_addr(slot_bm(s)) + 8 * lane);
    const uint64_t a0 = min(chunk_start<false>(e0), top);
    const uint32_t base = bitmap_prefix_reg(bm) - skip + chunk_delta<false>(e0, a0) + (s * kRingSlot) / 2;
    u32x4_t e;
    e.x = bm.x;
    e.y = base;
    e.z = bm.y;
    e.w = base + __builtin_popcount(bm.x);
    lds_store_b128(lds_addr(slot_tab(s)) + 16 * lane, e);
  };

  // Compute waves.
  const int ks = w & 1;
  const int f0 = 2 * (w >> 1);
  const LaneMap lm = lane_map(lane);
  const uint32_t toff = lm.tab + 256u * f0 + 128u * ks;
  f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  // The lane's B fragment (token n = lane % 16, k group g = lane / 16 of half
  // ks) in a slot's X^T area: position 4n + (g + n/4) mod 4 of the half.
  const uint32_t xoff = 1024u * ks + 16u * (4 * (lane & 15) + (((lane >> 4) + ((lane & 15) >> 2)) & 3));
  auto compute = [&](int s) {
    const u32x4_t x = *reinterpret_cast<const u32x4_t*>(slot_x(s) + xoff);
    const uint8_t* tab = slot_tab(s);
    u32x2_t e[2];
    e[0] = *reinterpret_cast<const u32x2_t*>(tab + toff);
    e[1] = *reinterpret_cast<const u32x2_t*>(tab + toff + 256);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t rb = e[j].y + __builtin_popcount(e[j].x & lm.pmask);
      const half8_t av = rebuild_row<false>(smem, lut, rb, __builtin_amdgcn_ubfe(e[j].x, lm.sh, 8));
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8_t, x), acc[j], 0, 0, 0);
    }
  };

  // The offsets load completes here, before the loader's first LDS-DMA: the
  // compiler does not count those, so a later wait for it would wait for
  // them too.
  asm volatile("" : : "v"(ov));
  // The roles are separate uniform paths (a branch taken by the whole wave).
  // Lowered as a divergent branch, one role's code would follow another's,
  // and the compute waves' LDS reads would wait for the loader's LDS-DMA
  // loads.  All pass the same number of barriers: two before the first
  // GroupTile, then one per GroupTile (four per GroupTile unpipelined).
  const bool fast = widest <= kRingFast;
  const int rl = __builtin_amdgcn_readfirstlane(role);
  if (rl == 1) {
    // The two loader waves run at a higher wave priority than the compute
    // waves: a step ends only when their loads are issued and their tables
    // written, so their instructions go first when several waves of a SIMD
    // are ready (measured on MI355X: 27.8 against 28.9 us on 20480x5120,
    // N = 16).
    __builtin_amdgcn_s_setprio(3);
    if (fast) {
      // Step c issues the values and X^T of c+R-1 and the bitmaps of c+R,
      // then waits until those issued R-2 steps before (values and X^T of
      // c+1, bitmaps of c+2) have landed.  pend[j]: loads issued by step
      // c-R+2+j.
      auto step_loads = [&](int c) -> int {
        const int sv = (c + R - 1 - c_begin) % R;
        int n = 0;
#ifdef USW_DEBUG
        // The areas this step loads into hold NaNs until the loads land:
        // slot sv's values and X^T, the next slot's bitmap words.
        auto poison = [&](uint8_t* p, int bytes) {
          const u32x4_t v = {kLdsPoison, kLdsPoison, kLdsPoison, kLdsPoison};
          for (int off = 16 * lane; off < bytes; off += 1024) lds_store_b128(lds_addr(p) + off, v);
        };
        if (c + R - 1 < c_end) {
          poison(slot_vals(sv), kRingVals);
          poison(slot_x(sv), kRingX);
        }
        if (c + R < c_end) poison(slot_bm(sv == R - 1 ? 0 : sv + 1), 512);
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
#endif
        if (c + R - 1 < c_end) {
          issue_x(c + R - 1, sv);
          n += 2 + issue_vals(off_at(c + R - 1), off_at(c + R), sv);
        }
        if (c + R < c_end) {
          issue_bm(c + R, sv == R - 1 ? 0 : sv + 1);
          ++n;
        }
        return n;
      };
      // Before the first GroupTile: the bitmaps of c_begin, then steps
      // c_begin-R+1 .. c_begin-1.
      issue_bm(c_begin, 0);
      int pend[R - 1];
#pragma unroll
      for (int j = 0; j < R - 1; ++j) pend[j] = step_loads(c_begin - R + 1 + j);
      int later = 0;
#pragma unroll
      for (int j = 0; j < R - 1; ++j) later += pend[j];
      wait_vm(later);                              // bitmaps of c_begin
      lds_barrier();
      later -= pend[0];
      wait_vm(later);                              // values and X^T of c_begin, bitmaps of c_begin+1
      lds_barrier();
      for (int c = c_begin; c < c_end; ++c) {
#pragma unroll
        for (int j = 0; j < R - 2; ++j) pend[j] = pend[j + 1];
        pend[R - 2] = step_loads(c);
        later = 0;
#pragma unroll
        for (int j = 1; j < R - 1; ++j) later += pend[j];
        wait_vm(later);                            // values and X^T of c+1, bitmaps of c+2
        lds_barrier();
      }
    } else {
      // Unpipelined: per GroupTile, its bitmaps, then the values of TCTile
      // rows 0-1 and of rows 2-3 in turn (each at most 4 KB + head), all in
      // slot 0; two barriers per half.
      lds_barrier();
      lds_barrier();
      for (int c = c_begin; c < c_end; ++c) {
        const uint32_t o0 = off_at(c), o1 = off_at(c + 1);
        issue_bm(c, 0);
        wait_vm(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x2_t bm = lds_load_b64(lds_addr(slot_bm(0)) + 8 * lane);
          const uint32_t mid = __builtin_amdgcn_readlane(bitmap_prefix_reg(bm), 32);
          const uint32_t hs = o0 + (h ? mid : 0u);
          if (h == 0) issue_x(c, 0);
          issue_vals(hs, h ? o1 : o0 + mid, 0);
          wait_vm(0);
          build_tab(hs, h ? mid : 0u, 0);
          lds_barrier();
          lds_barrier();
        }
      }
    }
  } else if (rl == 2) {
    __builtin_amdgcn_s_setprio(3);
    // The bitmap table of c+1 (its bitmaps landed before the barrier that
    // opened step c) goes into its slot during step c.
    lds_barrier();
    if (fast) build_tab(off_at(c_begin), 0, 0);
    lds_barrier();
    if (fast) {
      for (int c = c_begin; c < c_end; ++c) {
        if (c + 1 < c_end) build_tab(off_at(c + 1), 0, (c + 1 - c_begin) % R);
        lds_barrier();
      }
    } else {
      for (int c = c_begin; c < c_end; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          lds_barrier();
          lds_barrier();
        }
    }
  } else {
    lds_barrier();
    lds_barrier();
    if (fast) {
      int s = 0;
      for (int c = c_begin; c < c_end; ++c) {
        compute(s);
        s = s + 1 == R ? 0 : s + 1;
        lds_barrier();
      }
    } else {
      for (int c = c_begin; c < c_end; ++c) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          lds_barrier();
          if (f0 == 2 * h) compute(0);
          lds_barrier();
        }
      }
    }
  }

  // Sum the two k halves of every fragment (fixed order) and finish.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  if (role == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) *reinterpret_cast<f32x4_t*>(red + ((ks * 4 + f0 + j) * 64 + lane) * 4) = acc[j];
  }
  __syncthreads();
  finish_strip<NB, false, OUT_F16>(a, gi, sidx, kRingThreads, last_flag, [&](int n, int ml) {
    const int f = ml >> 4;
    const int ln = 16 * ((ml >> 2) & 3) + (n & 15);
    return *reinterpret_cast<const f32x4_t*>(red + (f * 64 + ln) * 4) +
           *reinterpret_cast<const f32x4_t*>(red + ((4 + f) * 64 + ln) * 4);
  });
}

// ---------------------------------------------------------------------------
// Host dispatch
// ---------------------------------------------------------------------------

// Decode launch configurations (waves per workgroup, pipeline depth,
// minimum waves per SIMD), each the measured best on MI355X for its case.
using DefaultCfg = Cfg<4, 1, 4>;
// fp16 with five-chunk value slots: 96 VGPRs, so a fifth wave per SIMD fits
// (measured 2% faster than four on the 20480x5120 layer at N = 16).
using DefaultCfgLean = Cfg<4, 1, 5>;
// 17..32 columns of N: twice the accumulators and X fragments, which do not
// fit 128 registers; three waves per SIMD leave room for them.
using DefaultCfg2 = Cfg<4, 1, 3>;
// 33..64 columns of N in one pass (four token blocks): two waves per SIMD.
using DefaultCfg4 = Cfg<4, 1, 2>;
// INT4 values, up to 16 columns of N: a third of the fp16 slot registers
// (85 VGPRs), so a fifth wave per SIMD fits and hides more of the rebuild
// latency (measured 6% faster on the 20480x5120 layer at N = 2).
using DefaultCfgI4 = Cfg<4, 1, 5>;

struct CfgInfo {
  int waves;   // waves per workgroup
  int occ;     // waves per SIMD the configuration allows
};

CfgInfo cfg_info(int nchunk, bool i4, bool lean) {
  if (nchunk > 32) return CfgInfo{DefaultCfg4::kWavesPerGroup, DefaultCfg4::kOcc};
  if (nchunk > 16) return CfgInfo{DefaultCfg2::kWavesPerGroup, DefaultCfg2::kOcc};
  if (i4) return CfgInfo{DefaultCfgI4::kWavesPerGroup, DefaultCfgI4::kOcc};
  return lean ? CfgInfo{DefaultCfgLean::kWavesPerGroup, DefaultCfgLean::kOcc}
              : CfgInfo{DefaultCfg::kWavesPerGroup, DefaultCfg::kOcc};
}

// Compute units of MI355X; the automatic split aims at one full round of
// resident workgroups on all of them.
constexpr int64_t kComputeUnits = 256;

struct Plan {
  int splits;     // workgroups per 64-row strip, passes of nchunk tokens
  int nchunk;     // columns of N per kernel pass (16, 32 or 64)
  int rsplits;    // the same for the last pass when it is shorter (N > 64,
  int rchunk;     // N mod 64 tokens in a pass of rchunk), else splits, 0
  int waves;      // waves per workgroup
  bool ring;      // the workgroup-cooperative kernel
};

// LDS slots of the workgroup-cooperative decode: two GroupTiles load while
// one is computed (measured on MI355X: 2 slots 2% slower, 4 slots, which
// leave room for four workgroups per compute unit instead of five, 24%
// slower).
constexpr int kRingDepth = 3;
// Fewest GroupTile columns the automatic split gives a ring workgroup.
constexpr int64_t kRingMinCols = 10;

void ring_launch(const Args& a, bool f16out, dim3 grid, hipStream_t s) {
  if (f16out)
    decode_ring_kernel<kRingDepth, true><<<grid, kRingThreads, 0, s>>>(a);
  else
    decode_ring_kernel<kRingDepth, false><<<grid, kRingThreads, 0, s>>>(a);
}

// Workgroups of the ring kernel resident per compute unit (registers, LDS).
int ring_resident() {
  int n = 0;
  const hipError_t e =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, decode_ring_kernel<kRingDepth, true>, kRingThreads, 0);
  return (e == hipSuccess && n > 0) ? n : 4;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// fp16 values with more than this many tokens take the prefill kernels;
// fewer take the decode kernels in passes of up to 64 tokens, which re-read
// the weight per pass but beat the 256-token prefill tiles up to 128 tokens
// on MI355X (at 128: 59.5 against 84.5 us on 11008x4096, 53.0 against 77.8
// on 4096x11008, 115.8 against 154.6 on 20480x5120; at 192 the prefill
// kernel is as fast or faster).
constexpr int kDecodeMaxN = 128;

bool use_prefill(const usw_fmt* f, int32_t N) { return f->val_type == USW_VAL_F16 && N > kDecodeMaxN; }

// Five 1 KB value chunks per slot when an fp16 matrix is at most 55% dense on
// average (a GroupTile then needs more than five only far in the tail; such
// a wave takes the two-half path), six otherwise.
bool lean_values(const usw_fmt* f, const usw::Geometry& g) {
  return f->val_type == USW_VAL_F16 &&
         static_cast<double>(f->nnz) <= 0.55 * static_cast<double>(g.M) * static_cast<double>(g.K);
}

// Pass size (16, 32 or 64 tokens) that n tokens take.
int pass_chunk(int n) { return n <= 16 ? 16 : n <= 32 ? 32 : 64; }

// Split factor of the per-wave decode kernel for passes of `chunk` tokens.
int wave_splits(const usw::Geometry& g, int chunk, int splits_req, bool i4, bool lean) {
  const CfgInfo ci = cfg_info(chunk, i4, lean);
  int64_t s = splits_req;
  if (s <= 0) {
    // About one round of resident workgroups (occ waves per SIMD, 4 SIMDs
    // per compute unit), each wave keeping at least 3 GroupTiles to stream.
    // Passes of 64 tokens on a matrix with at most one strip per compute
    // unit take as many workgroups as there are compute units, no more: the
    // split partial sums (64 x M fp32 per split, written and read back) then
    // cost more than the second workgroup per compute unit gains (measured
    // on MI355X at N = 64: 11008x4096 31.0 us with 1 split against 37.3 with
    // 3; 4096x11008 27.3 with 4 against 31.0 with 8; 15360x5120 38.1 with 1
    // against 44.5 with 2).
    const int64_t target = kComputeUnits * 4 * ci.occ / ci.waves;
    if (chunk == 64 && g.Gr <= kComputeUnits)
      s = kComputeUnits / g.Gr;
    else
      s = std::max<int64_t>(1, (target + g.Gr / 2) / g.Gr);
    s = std::min<int64_t>(s, std::max<int64_t>(1, g.Gc / (ci.waves * 3)));
  }
  const int64_t smax = std::max<int64_t>(1, g.Gc / ci.waves);
  // Each wave caches its GroupTile offsets in one register: at most 63
  // GroupTiles per wave.
  const int64_t smin = (g.Gc + 63 * ci.waves - 1) / (63 * ci.waves);
  return static_cast<int>(std::max(smin, std::max<int64_t>(1, std::min(s, smax))));
}

Plan make_plan(const usw::Geometry& g, int N, int splits_req, bool i4, bool lean) {
  Plan p;
  p.nchunk = pass_chunk(N);
  p.rchunk = 0;
  p.ring = !i4 && lean && N <= 16;
  if (p.ring) {
    // One round of resident workgroups, each keeping at most 63 GroupTiles
    // and, when the matrix has few strips, at least kRingMinCols: a
    // workgroup fills and drains its ring over the first and last steps, so
    // shorter runs lose more to that than a full round gains (measured on
    // MI355X: 5120x5120 at N = 16 13.5 us with 8 splits against 15.5 us with
    // the 16 of a full round).  The factor is clamped to K/256 like the
    // other decode kernel's.
    p.waves = 5;
    static const int resident = ring_resident();
    int64_t s = splits_req > 0 ? splits_req
                               : std::min<int64_t>((kComputeUnits * resident) / g.Gr,
                                                   std::max<int64_t>(1, g.Gc / kRingMinCols));
    const int64_t smax = std::max<int64_t>(1, g.Gc / 4);
    const int64_t smin = (g.Gc + 62) / 63;
    p.splits = static_cast<int>(std::max(smin, std::max<int64_t>(1, std::min(s, smax))));
    p.rsplits = p.splits;
    return p;
  }
  p.waves = cfg_info(p.nchunk, i4, lean).waves;
  p.splits = wave_splits(g, p.nchunk, splits_req, i4, lean);
  // A shorter last pass gets the split factor of its own size.
  const int rem = N > p.nchunk ? N % p.nchunk : 0;
  p.rchunk = rem > 0 ? pass_chunk(rem) : 0;
  p.rsplits = rem > 0 ? wave_splits(g, p.rchunk, splits_req, i4, lean) : p.splits;
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
  if (f->nnz < 0 || f->nnz >= (int64_t(1) << 32)) return USW_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(N) * g->M > (int64_t(1) << 40)) return USW_ERR_BAD_SHAPE;
  return USW_OK;
}

// Workspace: per-strip counters (4 B each, padded to 256 B) then the fp32
// partial sums of every split.
size_t counters_bytes(const usw::Geometry& g) { return (static_cast<size_t>(4 * g.Gr) + 255) & ~size_t(255); }

// Partial sums of the largest pass: splits x tokens of the pass x M fp32.
size_t workspace_bytes(const usw::Geometry& g, const Plan& p) {
  const size_t full = p.splits > 1 ? static_cast<size_t>(p.splits) * p.nchunk : 0;
  const size_t last = p.rchunk > 0 && p.rsplits > 1 ? static_cast<size_t>(p.rsplits) * p.rchunk : 0;
  const size_t cols = std::max(full, last);
  if (cols == 0) return 0;
  return counters_bytes(g) + cols * g.M * sizeof(float);
}

template <int NB, bool I4, int CH, class C>
void launch_cfg(const Args& a, bool f16out, dim3 grid, hipStream_t s) {
  if (f16out)
    decode_kernel<NB, I4, CH, true, C><<<grid, C::kThreadsPerGroup, 0, s>>>(a);
  else
    decode_kernel<NB, I4, CH, false, C><<<grid, C::kThreadsPerGroup, 0, s>>>(a);
}

template <int NB, bool I4, int CH>
void launch_decode(const Args& a, bool f16out, dim3 grid, hipStream_t s) {
  if constexpr (NB == 4)
    launch_cfg<NB, I4, CH, DefaultCfg4>(a, f16out, grid, s);
  else if constexpr (NB == 2)
    launch_cfg<NB, I4, CH, DefaultCfg2>(a, f16out, grid, s);
  else if constexpr (I4)
    launch_cfg<NB, I4, CH, DefaultCfgI4>(a, f16out, grid, s);
  else if constexpr (CH == 5)
    launch_cfg<NB, I4, CH, DefaultCfgLean>(a, f16out, grid, s);
  else
    launch_cfg<NB, I4, CH, DefaultCfg>(a, f16out, grid, s);
}

// Argument checks of a product call (nothing is written or launched).
usw_status check_call(const usw_fmt* f, const uint16_t* X, const void* Y, int32_t y_type, int32_t N,
                      usw::Geometry* g) {
  usw_status st = check_common(f, y_type, N, g);
  if (st) return st;
  if (!X || !Y || !f->bitmaps || !f->offsets || !f->values) return USW_ERR_NULL_ARG;
  if (f->val_type == USW_VAL_I4 && !f->scales) return USW_ERR_NULL_ARG;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(f->bitmaps) || !aligned16(f->values) ||
      (reinterpret_cast<uintptr_t>(f->offsets) & 3u))
    return USW_ERR_MISALIGNED;
  return USW_OK;
}

// Kernel choice, split factor and workspace of one call.
struct CallPlan {
  bool prefill;
  usw::PrefillPlan pp;   // prefill
  Plan p;                // decode
  size_t need;           // workspace bytes (0: none)
  size_t cb;             // leading counter bytes of the workspace
};

CallPlan make_call_plan(const usw_fmt* f, const usw::Geometry& g, int32_t N, int splits_req, bool tiles512 = true) {
  CallPlan c{};
  c.prefill = use_prefill(f, N);
  if (c.prefill) {
    c.pp = usw::prefill_plan(g, N, splits_req, tiles512);
    c.need = usw::prefill_workspace_bytes(g, N, c.pp);
    c.cb = usw::prefill_counter_bytes(g, c.pp);
  } else {
    c.p = make_plan(g, N, splits_req, f->val_type == USW_VAL_I4, lean_values(f, g));
    c.need = workspace_bytes(g, c.p);
    c.cb = c.need > 0 ? counters_bytes(g) : 0;
  }
  return c;
}

// Enqueue a planned call.  counters (c.cb bytes, zero at the start) and part
// (c.need - c.cb bytes) are used only when c.need > 0.
usw_status launch_call(const usw_fmt* f, const usw::Geometry& g, const CallPlan& c, const uint16_t* X, void* Y,
                       int32_t y_type, int32_t N, uint32_t* counters, float* part, void* stream) {
  if (c.prefill) return usw::prefill_launch(f, g, X, Y, y_type == USW_OUT_F16, N, counters, part, c.pp, stream);
  const Plan& p = c.p;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = static_cast<int>(g.M), K = static_cast<int>(g.K), Gc = static_cast<int>(g.Gc);
  const size_t ybytes = y_type == USW_OUT_F16 ? 2 : 4;
  const bool f16out = y_type == USW_OUT_F16;
  const bool i4 = f->val_type == USW_VAL_I4;
  const bool lean = lean_values(f, g);

  for (int n0 = 0; n0 < N; n0 += p.nchunk) {
    const int nc = std::min(p.nchunk, N - n0);
    // The shorter last pass of a multi-pass call has its own split factor.
    const int splits = (p.rchunk > 0 && n0 + p.nchunk > N) ? p.rsplits : p.splits;
    const int64_t nblk = g.Gr * splits;
    const dim3 grid(static_cast<unsigned>(nblk));
    Args a{};
    a.bitmaps = f->bitmaps;
    a.offsets = f->offsets;
    a.values = static_cast<const uint8_t*>(f->values);
    a.scales = i4 ? f->scales : nullptr;
    a.X = X + static_cast<size_t>(n0) * K;
    a.Y = static_cast<uint8_t*>(Y) + static_cast<size_t>(n0) * M * ybytes;
    a.counters = c.need ? counters : nullptr;
    a.part = c.need ? part : nullptr;
    a.values_alloc = usw::values_alloc_bytes(f->val_type, f->nnz);
    a.M = M;
    a.K = K;
    a.N = nc;
    a.Gc = Gc;
    a.splits = splits;
    a.remap = (splits > 1 && nblk % 8 == 0) ? 1 : 0;
    const int nb = nc > 32 ? 4 : nc > 16 ? 2 : 1;   // 16-token blocks of this pass
    if (p.ring) {
      ring_launch(a, f16out, grid, s);
    } else if (i4) {
      if (nb == 4) launch_decode<4, true, 3>(a, f16out, grid, s);
      else if (nb == 2) launch_decode<2, true, 3>(a, f16out, grid, s);
      else launch_decode<1, true, 3>(a, f16out, grid, s);
    } else if (lean) {
      if (nb == 4) launch_decode<4, false, 5>(a, f16out, grid, s);
      else if (nb == 2) launch_decode<2, false, 5>(a, f16out, grid, s);
      else launch_decode<1, false, 5>(a, f16out, grid, s);
    } else {
      if (nb == 4) launch_decode<4, false, 6>(a, f16out, grid, s);
      else if (nb == 2) launch_decode<2, false, 6>(a, f16out, grid, s);
      else launch_decode<1, false, 6>(a, f16out, grid, s);
    }
    if (hipGetLastError() != hipSuccess) return USW_ERR_HIP;
  }
  return USW_OK;
}

usw_status spmm_impl(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N, void* ws,
                     size_t ws_bytes, void* stream, int splits_req) {
  usw::Geometry g;
  usw_status st = check_call(f, X, Y, y_type, N, &g);
  if (st) return st;
  const CallPlan c = make_call_plan(f, g, N, splits_req);
  if (c.need > 0) {
    if (!ws || ws_bytes < c.need) return USW_ERR_WORKSPACE;
    if (!aligned16(ws)) return USW_ERR_MISALIGNED;
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  return launch_call(f, g, c, X, Y, y_type, N, reinterpret_cast<uint32_t*>(w),
                     c.need ? reinterpret_cast<float*>(w + c.cb) : nullptr, stream);
}

// ---------------------------------------------------------------------------
// Scratch-backed calls (usw_spmm_noalloc)
// ---------------------------------------------------------------------------
//
// The split-K counters and partial sums of usw_spmm_noalloc live in one
// statically allocated device array per GPU instead of a caller workspace:
// counters in its first kScratchCounterBytes, partial sums after them.  In
// host code the array's name is only a stand-in; its device address on the
// current GPU comes from hipGetSymbolAddress, taken once per device and kept.

constexpr size_t kScratchBytes = size_t(16) << 20;          // the whole array: 16 MiB
constexpr size_t kScratchCounterBytes = size_t(16) << 10;   // counters: up to 4096 tiles
constexpr int kMaxDevices = 64;
static_assert(sizeof(scratch) == kScratchBytes, "the scratch array has the stated size");

// Clears n 32-bit words (the counters a call needs at zero) with ordinary
// vector stores; a kernel, so that the call can be captured in a HIP graph.
__global__ __launch_bounds__(256) void scratch_clear_kernel(uint32_t* __restrict__ p, uint32_t n) {
  for (uint32_t i = threadIdx.x + blockIdx.x * 256u; i < n; i += 256u * gridDim.x) p[i] = 0u;
}

std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the current device.
usw_status scratch_address(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return USW_ERR_HIP;
  if (dev >= kMaxDevices) return USW_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return USW_ERR_HIP;
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return USW_OK;
}

usw_status spmm_noalloc_impl(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N,
                             int32_t splits, void* stream) {
  usw::Geometry g;
  usw_status st = check_call(f, X, Y, y_type, N, &g);
  if (st) return st;
  auto fits = [](const CallPlan& c) {
    return c.cb <= kScratchCounterBytes && c.need - c.cb <= kScratchBytes - kScratchCounterBytes;
  };
  CallPlan c = make_call_plan(f, g, N, splits < 0 ? 0 : splits);
  // The automatic factor falls back to 1 when its partial sums do not fit,
  // and N > 256 to the 256-token prefill kernel when the 512-token kernel's
  // copy of X does not.
  if (splits <= 0 && !fits(c)) c = make_call_plan(f, g, N, 1);
  if (splits <= 1 && c.prefill && !fits(c)) c = make_call_plan(f, g, N, 1, false);
  if (!fits(c)) return USW_ERR_WORKSPACE;
  uint8_t* base = nullptr;
  if (c.need > 0) {
    st = scratch_address(&base);
    if (st) return st;
    // The counters must be zero when the kernels start.  Every call leaves
    // them zero, but a call that overlapped another on this GPU may not.
    hipStream_t s = static_cast<hipStream_t>(stream);
    scratch_clear_kernel<<<1, 256, 0, s>>>(reinterpret_cast<uint32_t*>(base), static_cast<uint32_t>(c.cb / 4));
    if (hipGetLastError() != hipSuccess) return USW_ERR_HIP;
  }
  return launch_call(f, g, c, X, Y, y_type, N, reinterpret_cast<uint32_t*>(base),
                     c.need ? reinterpret_cast<float*>(base + kScratchCounterBytes) : nullptr, stream);
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
  const int sr = splits < 0 ? 0 : splits;
  if (use_prefill(f, N))
    *bytes = usw::prefill_workspace_bytes(g, N, usw::prefill_plan(g, N, sr));
  else
    *bytes = workspace_bytes(g, make_plan(g, N, sr, f->val_type == USW_VAL_I4, lean_values(f, g)));
  return USW_OK;
}

usw_status usw_spmm_counter_bytes(const usw_fmt* f, int32_t N, int32_t splits, size_t* bytes) {
  if (!bytes) return USW_ERR_NULL_ARG;
  usw::Geometry g;
  usw_status st = check_common(f, USW_OUT_F16, N, &g);
  if (st) return st;
  const int sr = splits < 0 ? 0 : splits;
  if (use_prefill(f, N)) {
    *bytes = usw::prefill_counter_bytes(g, usw::prefill_plan(g, N, sr));
  } else {
    const Plan p = make_plan(g, N, sr, f->val_type == USW_VAL_I4, lean_values(f, g));
    *bytes = workspace_bytes(g, p) > 0 ? counters_bytes(g) : 0;
  }
  return USW_OK;
}

usw_status usw_spmm_ex(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N, int32_t splits,
                       void* ws, size_t ws_bytes, void* stream) {
  return spmm_impl(f, X, Y, y_type, N, ws, ws_bytes, stream, splits < 0 ? 0 : splits);
}

usw_status usw_spmm_noalloc(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N, int32_t splits,
                            void* stream) {
  return spmm_noalloc_impl(f, X, Y, y_type, N, splits, stream);
}

}  // extern "C"
