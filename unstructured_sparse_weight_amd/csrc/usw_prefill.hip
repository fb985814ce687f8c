// Prefill kernel of libusw (fp16 values, N > 32): Y[n][m] = sum_k W_sp[m][k] X[n][k]
// with W_sp in the TCA-BME bitmap format (blog "SpInfer: How bitmaps make
// sparse LLMs actually fast", section "How TCA-BME addresses the indexing
// overhead"), fed to the fp16 matrix cores.
//
// At large N the product is a dense contraction: every rebuilt 64x64
// GroupTile meets many tokens, so the cost that matters is the matrix-core
// work plus the rebuild, which is paid once per GroupTile per workgroup.
// Design (gfx950, wave64):
//   * A workgroup owns one 64-row strip of GroupTiles and 64 tokens per wave
//     (256 or 512 tokens), and walks a range of GroupTile columns.
//   * Per GroupTile the workgroup stages the value range [offsets[g],
//     offsets[g+1]) in LDS with 16-byte loads issued ahead; the bitmap
//     words stay in registers, where each wave derives the BitmapTile bases
//     of its fragments a step before the rebuild.  Each wave rebuilds 8 /
//     waves of the 8 A fragments
//     (16 rows x 32 columns each; lane l holds row l%16, columns
//     8*(l/16)..+7, i.e. one row of one BitmapTile) by masked popcount and
//     writes them to a double-buffered LDS tile that every wave reads.
//   * Each wave multiplies the 64x64 tile with its 64 tokens: 32
//     v_mfma_f32_16x16x32_f16 per GroupTile, fp32 accumulators in VGPRs.  Its
//     slice of X (X is [N][K]: 64 tokens x 128 B) is loaded a GroupTile
//     ahead in whole cache lines and staged in the wave's own LDS region,
//     from which the X^T fragments are read (no other wave uses them).
//   * Split K (more workgroups than strips x token tiles): fp32 partial sums
//     go to the workspace and the last workgroup of a tile adds them in
//     split order, so the result does not depend on scheduling.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "usw.h"
#include "usw_internal.h"
#include "usw_device.h"

namespace {

using namespace usw_dev;

constexpr int kMaxCols = 1024;      // GroupTile columns per workgroup (offsets table in LDS)
constexpr int kStageChunks = 520;   // >= 513 16-byte chunks: a dense GroupTile plus a partial first chunk

struct PArgs {
  const uint64_t* __restrict__ bitmaps;
  const uint32_t* __restrict__ offsets;
  const uint8_t* __restrict__ values;
  const uint16_t* __restrict__ X;
  const u32x4_t* __restrict__ xf;   // prefill_ws_kernel: X in fragment order (xfrag_kernel)
  void* __restrict__ Y;
  float* __restrict__ part;         // partial sums: [splits][N][M], or slots of 512 x 64 (prefill_ws_kernel)
  uint32_t* __restrict__ counters;  // per (strip, token tile): workgroups done; kept at 0 between calls
  uint64_t values_alloc;            // padded size of the values buffer in bytes
  int M, K, N, Gc, splits, ntiles;
  int tiles;                        // strips x token tiles
  int wgs;                          // prefill_ws_kernel: > 0 stream-K over this many workgroups
  int remap;                        // 1: keep consecutive tiles (and a tile's splits) on one XCD
  int kb32;                         // K / 32
};

template <int WAVES>
struct PTraits {
  static constexpr int kThreads = 64 * WAVES;
  static constexpr int kCpt = (kStageChunks + kThreads - 1) / kThreads;  // value chunks per thread
  static constexpr int kFrags = 8 / WAVES;                                // A fragments each wave rebuilds
  static constexpr int kStageBytes = kThreads * kCpt * 16 + 16;
  static constexpr int kBN = 64 * WAVES;                                  // tokens per workgroup
};

template <int CPT>
struct VSlot {
  u32x4_t v[CPT];
  u32x2_t bm;       // lane t: bitmap word t of the GroupTile
};

// What a lane needs from a GroupTile's bitmaps to rebuild its fragments:
// the value base and the bitmap word of each of its BitmapTiles.  Computed
// from the slot's registers when the GroupTile is copied into LDS, a step
// before its rebuild, so the rebuild itself waits on one LDS round trip.
template <int FRAGS>
struct RbIn {
  uint32_t base[FRAGS];
  uint32_t lo[FRAGS], hi[FRAGS];
};

template <int WAVES, bool OUT_F16>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void prefill_kernel(PArgs a) {
  using T = PTraits<WAVES>;
  constexpr int kThreads = T::kThreads;
  constexpr int kCpt = T::kCpt;

  __shared__ __attribute__((aligned(16))) uint8_t stage[2][T::kStageBytes];
  __shared__ __attribute__((aligned(16))) u32x4_t abuf[2][8 * 64];   // two rebuilt 64x64 tiles, fragment order
  __shared__ __attribute__((aligned(16))) u32x4_t xs[WAVES][64 * 8];   // per wave: its 64 tokens x 64 k of X
  __shared__ __attribute__((aligned(16))) uint32_t lut[32];
  __shared__ uint32_t offtab[kMaxCols + 1];
  __shared__ uint32_t last_flag;
  USW_LDS_POISON(stage);
  USW_LDS_POISON(abuf);
  USW_LDS_POISON(xs);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int nblk = static_cast<int>(gridDim.x);
  const int b = static_cast<int>(blockIdx.x);
  const int L = a.remap ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int tile = L / a.splits;
  const int sidx = L - tile * a.splits;
  const int gi = tile / a.ntiles;
  const int nt = tile - gi * a.ntiles;
  const int m0 = gi * kGT;
  const int nw = nt * T::kBN + 64 * w;   // first token of this wave

  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * sidx / a.splits);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (sidx + 1) / a.splits);
  const int cnt = c_end - c_begin;        // >= 1: the host keeps splits <= Gc
  const int c_last = c_end - 1;
  const int64_t g_row = static_cast<int64_t>(gi) * a.Gc;

  if (tid < 16) {
    u32x2_t e;
    e.x = nibble_selector(tid, 0);
    e.y = nibble_selector(tid, 1);
    reinterpret_cast<u32x2_t*>(lut)[tid] = e;
  }
  for (int i = tid; i <= cnt; i += kThreads) offtab[i] = a.offsets[g_row + c_begin + i];
  __syncthreads();

  const uint64_t top = a.values_alloc - 16;
  auto load_v = [&](VSlot<kCpt>& s, int c) {
    const uint32_t o0 = offtab[c - c_begin], o1 = offtab[c - c_begin + 1];
    const uint64_t a0 = min(chunk_start<false>(o0), top);
    const uint32_t nch = min(chunk_count<false>(o1, a0), static_cast<uint32_t>(kThreads * kCpt));
    const uint32_t last = min(nch > 0 ? nch - 1 : 0u, static_cast<uint32_t>((top - a0) >> 4));
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.values + a0);
#pragma unroll
    for (int i = 0; i < kCpt; ++i) s.v[i] = src[min(static_cast<uint32_t>(tid + kThreads * i), last)];
    s.bm = reinterpret_cast<const u32x2_t*>(a.bitmaps + (g_row + c) * kBtPerGt)[lane];
  };
  auto commit_v = [&](const VSlot<kCpt>& s, int buf) {
#pragma unroll
    for (int i = 0; i < kCpt; ++i) reinterpret_cast<u32x4_t*>(stage[buf])[tid + kThreads * i] = s.v[i];
  };

  // X for this wave's 64 tokens and GroupTile column c: 64 rows of 128 B,
  // loaded 8 lanes per row (whole cache lines) and kept in the wave's LDS
  // region, 16-byte chunk q of row r at slot 8r + (q ^ ((r >> 1) & 7)) so
  // that both these row writes and the fragment reads below (16 rows, one
  // chunk) touch 16 distinct bank groups.  Tokens past N repeat token N-1;
  // their products land in columns never stored.
  const int row = lane & 15, kb = lane >> 4;
  auto xslot = [](int r, int q) { return 8 * r + (q ^ ((r >> 1) & 7)); };
  auto load_x = [&](u32x4_t (&x)[8], int c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = min(nw + (lane >> 3) + 8 * j, a.N - 1);
      x[j] = *reinterpret_cast<const u32x4_t*>(a.X + static_cast<size_t>(n) * a.K + c * kGT + (lane & 7) * 8);
    }
  };
  auto store_x = [&](const u32x4_t (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) xs[w][xslot((lane >> 3) + 8 * j, lane & 7)] = x[j];
  };

  // Lane constants of the 16x32 A fragment.
  const int r8 = row & 7;
  const int bt_lane = 4 * (kb >> 1) + 2 * (row >> 3) + (kb & 1);
  const uint64_t rowmask = (1ull << (8 * r8)) - 1ull;

  // Rebuild inputs of GroupTile column c from its slot: DPP prefix scan of
  // the BitmapTile popcounts (lane t <-> BitmapTile t, plus the value
  // elements before the GroupTile's first one in its first chunk), then each
  // fragment's BitmapTile base and bitmap word via ds_bpermute.
  auto prep = [&](const VSlot<kCpt>& s, int c) {
    RbIn<T::kFrags> in;
    const uint32_t o0 = offtab[c - c_begin];
    const uint64_t a0 = min(chunk_start<false>(o0), top);
    const uint32_t pc = __builtin_popcount(s.bm.x) + __builtin_popcount(s.bm.y);
    const uint32_t ebase = wave_inclusive_scan(pc) - pc + chunk_delta<false>(o0, a0);
#pragma unroll
    for (int j = 0; j < T::kFrags; ++j) {
      const int f = w * T::kFrags + j;
      const int bt = 16 * (f >> 1) + 8 * (f & 1) + bt_lane;
      in.base[j] = __builtin_amdgcn_ds_bpermute(bt << 2, ebase);
      in.lo[j] = __builtin_amdgcn_ds_bpermute(bt << 2, s.bm.x);
      in.hi[j] = __builtin_amdgcn_ds_bpermute(bt << 2, s.bm.y);
    }
    return in;
  };

  // Rebuild this wave's fragments of GroupTile column c, staged in
  // stage[c&1], into abuf[c&1].
  auto rebuild = [&](int c, const RbIn<T::kFrags>& in) {
    const int buf = c & 1;
    const uint8_t* vb = stage[buf];
#pragma unroll
    for (int j = 0; j < T::kFrags; ++j) {
      const int f = w * T::kFrags + j;
      const uint64_t bm = (static_cast<uint64_t>(in.hi[j]) << 32) | in.lo[j];
      const uint32_t rb = in.base[j] + __popcll(bm & rowmask);
      const uint32_t byte = static_cast<uint32_t>(bm >> (8 * r8)) & 0xFFu;
      abuf[buf][f * 64 + lane] = __builtin_bit_cast(u32x4_t, rebuild_row<false>(vb, lut, rb, byte));
    }
  };

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // X^T fragment (ks, nb): lane l holds token 16nb + l%16, k = 32ks + 8(l/16) .. +7.
  auto mma = [&](int buf) {
    u32x4_t af[8];
#pragma unroll
    for (int f = 0; f < 8; ++f) af[f] = abuf[buf][f * 64 + lane];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const u32x4_t bf = xs[w][xslot(16 * nb + row, 4 * ks + kb)];
#pragma unroll
        for (int rs = 0; rs < 4; ++rs)
          acc[rs][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, af[rs * 2 + ks]),
                                                               __builtin_bit_cast(half8_t, bf), acc[rs][nb], 0, 0, 0);
      }
  };

  // Pipeline, one barrier per GroupTile column c, loads two columns ahead.
  // A step issues the loads of X(c+2) and of the values of c+3 into one
  // register slot, rebuilds tile c+1 (staged in stage[(c+1)&1]) into
  // abuf[(c+1)&1] while multiplying tile c (abuf[c&1], X(c) in the wave's
  // LDS region), then moves the other slot, loaded a step earlier, into LDS:
  // X(c+1) replaces X(c), and the values of c+2 go to stage[c&1], rebuilt in
  // the step before.  Loads past the last column repeat it.
  VSlot<kCpt> vs0, vs1;
  u32x4_t xr0[8], xr1[8];
  load_x(xr0, c_begin);
  load_v(vs0, c_begin);
  commit_v(vs0, c_begin & 1);
  const RbIn<T::kFrags> rin0 = prep(vs0, c_begin);
  load_v(vs0, min(c_begin + 1, c_last));
  commit_v(vs0, (c_begin + 1) & 1);
  RbIn<T::kFrags> rin = prep(vs0, min(c_begin + 1, c_last));
  store_x(xr0);
  load_x(xr1, min(c_begin + 1, c_last));
  load_v(vs1, min(c_begin + 2, c_last));
  __syncthreads();
  rebuild(c_begin, rin0);
  __syncthreads();

  // rin holds the rebuild inputs of column c+1 when step c starts.
  auto step = [&](int c, u32x4_t (&xl)[8], VSlot<kCpt>& vl, const u32x4_t (&xu)[8], const VSlot<kCpt>& vu) {
    load_x(xl, min(c + 2, c_last));
    load_v(vl, min(c + 3, c_last));
    // Keep the loads ahead of the compute they are meant to overlap.
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < c_end) rebuild(c + 1, rin);
    mma(c & 1);
    // The wave's own LDS operations run in order: the fragment reads above
    // see X(c), the stores below replace it with X(c+1).
    store_x(xu);
    commit_v(vu, c & 1);
    rin = prep(vu, min(c + 2, c_last));
    __syncthreads();
  };
  int c = c_begin;
  for (; c + 2 <= c_end; c += 2) {
    step(c, xr0, vs0, xr1, vs1);
    step(c + 1, xr1, vs1, xr0, vs0);
  }
  if (c < c_end) step(c, xr0, vs0, xr1, vs1);

  // Epilogue: lane l of block (rs, nb) holds rows 16rs + 4(l/16) + i and
  // token 16nb + l%16.
  auto store_y4 = [&](int n, int m, f32x4_t v) {
    const size_t yi = static_cast<size_t>(n) * a.M + m;
    if constexpr (OUT_F16) {
      typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
      half4_t h;
      h.x = static_cast<_Float16>(v.x);
      h.y = static_cast<_Float16>(v.y);
      h.z = static_cast<_Float16>(v.z);
      h.w = static_cast<_Float16>(v.w);
      *reinterpret_cast<half4_t*>(reinterpret_cast<_Float16*>(a.Y) + yi) = h;
    } else {
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.Y) + yi) = v;
    }
  };
#pragma unroll
  for (int rs = 0; rs < 4; ++rs)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = nw + nb * 16 + row;
      const int m = m0 + rs * 16 + 4 * kb;
      if (n >= a.N) continue;
      if (a.splits > 1) {
        float* p = a.part + (static_cast<size_t>(sidx) * a.N + n) * a.M + m;
#pragma unroll
        for (int i = 0; i < 4; ++i) __hip_atomic_store(p + i, acc[rs][nb][i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        store_y4(n, m, acc[rs][nb]);
      }
    }
  if (a.splits <= 1) return;

  // Split K: the last workgroup of the tile adds the partial sums of all its
  // splits in split order (device-coherent stores, completed before the
  // barrier that precedes the counter increment) and resets the counter.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0)
    last_flag = __hip_atomic_fetch_add(&a.counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                static_cast<uint32_t>(a.splits - 1);
  __syncthreads();
  if (!last_flag) return;
  const int n_base = nt * T::kBN;
  for (int e = tid; e < T::kBN * 16; e += kThreads) {
    const int n = n_base + (e >> 4);
    const int m = m0 + 4 * (e & 15);
    if (n >= a.N) continue;
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < a.splits; ++p) {
      const float* q = a.part + (static_cast<size_t>(p) * a.N + n) * a.M + m;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += __hip_atomic_load(q + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    store_y4(n, m, s);
  }
  if (tid == 0) __hip_atomic_store(&a.counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Builder-side barrier: wait until at most n (wave-uniform, 0..4) of this
// wave's LDS-DMA loads are in flight, then a workgroup barrier; a larger n
// waits as for 4 (never for fewer loads than asked).
__device__ __forceinline__ void builder_barrier(int n) {
  switch (__builtin_amdgcn_readfirstlane(n)) {
    case 0: USW_PRODUCER_BARRIER(0); break;
    case 1: USW_PRODUCER_BARRIER(1); break;
    case 2: USW_PRODUCER_BARRIER(2); break;
    case 3: USW_PRODUCER_BARRIER(3); break;
    default: USW_PRODUCER_BARRIER(4); break;
  }
}

// X in the order of the MFMA B fragments of prefill_ws_kernel, written once
// per call before it: the 16-byte unit u = ((nt * K/32 + j) * 32 + tb) * 64 + l
// holds X[n][k0 .. k0 + 7] with n = 512 nt + 16 tb + (l % 16) and
// k0 = 32 j + 8 (l / 16) -- lane l's register of fragment tb of k-block j --
// or zeros for n >= N.  A wave's eight fragments of one half GroupTile column
// are then 8 KB in a row, and a 512-token tile's X for that half column 32 KB.
// A thread writes the units of k-blocks 2jj and 2jj + 1 of one lane slot (its
// two reads lie in one 128-byte line of X); 32-bit index arithmetic (the host
// keeps the unit count below 2^31).
__global__ __launch_bounds__(256) void xfrag_kernel(const uint16_t* __restrict__ X, u32x4_t* __restrict__ xf, int N,
                                                    int K, uint32_t pairs) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  if (t >= pairs) return;
  const uint32_t l = t & 63u, tb = (t >> 6) & 31u;
  const uint32_t blk = t >> 11;             // nt * K/64 + jj
  const uint32_t kp = static_cast<uint32_t>(K) / 64u;
  const uint32_t nt = blk / kp, jj = blk - nt * kp;
  const uint32_t n = 512u * nt + 16u * tb + (l & 15u);
  u32x4_t v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
  if (n < static_cast<uint32_t>(N)) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(X + static_cast<size_t>(n) * K + 64u * jj + 8u * (l >> 4));
    v0 = src[0];
    v1 = src[4];
  }
  const size_t u0 = ((static_cast<size_t>(nt) * (2u * kp) + 2u * jj) * 32u + tb) * 64u + l;
  xf[u0] = v0;
  xf[u0 + 32 * 64] = v1;
}

// Warp-specialised variant for N > 256: a tile is 64 rows (one GroupTile
// strip) by 512 tokens, and eight waves in two roles pass the same barriers,
// one per GroupTile column.
//  - Waves 0-3 (consumers) multiply: each owns 128 tokens (64 rows x 128
//    tokens of fp32 accumulators) and per half column reads 4 A fragments
//    from LDS and 8 X^T fragments straight from the fragment-ordered copy of
//    X (xfrag_kernel) into registers, a half column ahead, for 32 MFMAs.
//    X never passes through LDS: every 64-row strip re-reads the whole X
//    tile, and staging it in LDS made LDS the bound.
//  - Waves 4-7 (builders) rebuild the A tile of the next column (two
//    fragments each) from the staged values, and bring the values and
//    bitmap words of a GroupTile three columns ahead into LDS with
//    global_load_lds_dwordx4 (no register round trip).  Before each barrier
//    a builder waits until the loads that the next column's rebuild reads
//    have landed (s_waitcnt vmcnt).
//
// Work split.  The (tile, GroupTile column) units are numbered tile-major.
// With a.wgs > 0 (stream-K) every compute unit gets the same number of
// columns whatever the tile count: workgroup p of P = a.wgs takes R whole
// tiles p, p + P, ... and an even share [B + U p / P, B + U (p + 1) / P) of
// the units of the tiles left over (B = R P Gc; R = 0 when there are fewer
// tiles than workgroups).  Otherwise (split-K) workgroup L takes split
// L % splits of tile L / splits.  A workgroup first runs the pieces of its
// range (one per tile it touches) from the last to the first -- the
// workgroups that share a tile then start its columns at both ends at once,
// and the partial sums are added while whole tiles still run -- then its
// whole tiles.  A piece that covers its whole tile stores Y; otherwise it
// stores fp32 partial sums in a slot of its own, and the workgroup that
// completes the tile's count adds the tile's slots in a fixed order (that of
// the ranges), so results do not depend on timing.
template <bool OUT_F16>
__global__ __launch_bounds__(512, 1) void prefill_ws_kernel(PArgs a) {
  constexpr int kBN = 512;
  constexpr int kThreads = 512;
  constexpr int kPThreads = 256;                                      // builder threads
  constexpr int kCpt = (kStageChunks + kPThreads - 1) / kPThreads;   // value chunks per builder thread
  constexpr int kStageBytes = kPThreads * kCpt * 16 + 16;
  constexpr int kSlot = kBN * kGT;                                    // floats per partial-sum slot
  static_assert(kCpt + 1 <= 4, "builder_barrier counts at most 4 loads per column");

  __shared__ __attribute__((aligned(16))) uint8_t stage[3][kStageBytes];   // values of columns c .. c+2 (by c % 3)
  __shared__ __attribute__((aligned(16))) u32x4_t abuf[2][8 * 64];
  __shared__ __attribute__((aligned(16))) uint32_t lut[32];
  __shared__ __attribute__((aligned(16))) u32x2_t bmw[3][64];   // their bitmap words
  __shared__ uint32_t offtab[kMaxCols + 1];
  __shared__ uint32_t last_flag;
  USW_LDS_POISON(stage);
  USW_LDS_POISON(abuf);
  USW_LDS_POISON(bmw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 15, kb = lane >> 4;

  const int nblk = static_cast<int>(gridDim.x);
  const int b = static_cast<int>(blockIdx.x);
  const int L = a.remap ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int64_t Gc = a.Gc;
  // Stream-K: R whole rounds of tiles L, L + P, ..., and the units of the
  // remaining tiles, [B, B + U) with B = R P Gc, split evenly.  R is
  // tiles / P, one less when the remainder would give some workgroup no
  // unit (the host keeps tiles * Gc >= P): an empty range between two owners
  // of a tile would leave its count short.
  int R = a.wgs > 0 ? a.tiles / nblk : 0;
  if (R > 0 && a.tiles % nblk != 0 && static_cast<int64_t>(a.tiles - R * nblk) * Gc < nblk) --R;
  const int64_t B = static_cast<int64_t>(R) * nblk * Gc;
  const int64_t U = static_cast<int64_t>(a.tiles) * Gc - B;
  int64_t r0, r1;
  if (a.wgs > 0) {
    r0 = B + U * L / nblk;
    r1 = B + U * (L + 1) / nblk;
  } else {
    const int tile = L / a.splits, sidx = L - tile * a.splits;
    r0 = tile * Gc + Gc * sidx / a.splits;
    r1 = tile * Gc + Gc * (sidx + 1) / a.splits;
  }

  if (tid < 16) {
    u32x2_t e;
    e.x = nibble_selector(tid, 0);
    e.y = nibble_selector(tid, 1);
    reinterpret_cast<u32x2_t*>(lut)[tid] = e;
  }


  auto store_y4 = [&](int n, int m, f32x4_t v) {
    const size_t yi = static_cast<size_t>(n) * a.M + m;
    if constexpr (OUT_F16) {
      typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
      half4_t h;
      h.x = static_cast<_Float16>(v.x);
      h.y = static_cast<_Float16>(v.y);
      h.z = static_cast<_Float16>(v.z);
      h.w = static_cast<_Float16>(v.w);
      *reinterpret_cast<half4_t*>(reinterpret_cast<_Float16*>(a.Y) + yi) = h;
    } else {
      *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.Y) + yi) = v;
    }
  };

  // One piece: columns [c_begin, c_end) of one tile.
  struct Piece {
    int tile, c_begin, c_end, cnt, m0, n_base, slot;
    int64_t t0, g_row;
    bool full;
  };

  // Split tile: after every wave's partial-sum stores have completed, count
  // the piece; the tile's last piece (the one whose count completes it) then
  // has the consumers add the tile's slots in range order.  Returns the first
  // owner and the number of pieces in *q0, *np.
  auto count_split = [&](const Piece& pc, int* q0, int* np) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();
    if (a.wgs > 0) {
      // Owners of the tile: workgroups p with B + U p / P <= t0 + Gc - 1
      // and B + U (p + 1) / P > t0.
      const int64_t x0 = pc.t0 - B;
      *q0 = static_cast<int>(((x0 + 1) * nblk + U - 1) / U) - 1;
      *np = static_cast<int>(((x0 + Gc) * nblk + U - 1) / U) - *q0;
    } else {
      *q0 = pc.tile * a.splits;
      *np = a.splits;
    }
    if (tid == 0)
      last_flag = __hip_atomic_fetch_add(&a.counters[pc.tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  static_cast<uint32_t>(*np - 1);
    __syncthreads();
    return last_flag != 0;
  };
  // Partial-sum slot of owner q of a split tile.
  auto slot_of = [&](const Piece& pc, int q) {
    return a.wgs > 0 ? 2 * q + (B + U * q / nblk >= pc.t0 ? 0 : 1) : q;
  };
  // The tile's sum, owner by owner in range order, by all threads: thread
  // tid takes slot elements e = tid + kThreads j, element e being 4 floats
  // of token 128 wv + 16 nb + ln % 16, rows 16 rs + 4 (ln / 16) .. +3 for
  // e = ((wv * 4 + rs) * 8 + nb) * 64 + ln.  Loads reach the device-coherent
  // level (sc1), where the owners' stores went.
  auto reduce_tile = [&](const Piece& pc, int q0, int np) {
    constexpr int kE = kSlot / 4;                       // float4 elements per slot
    constexpr int kJ = (kE + kThreads - 1) / kThreads;
    // The thread index through an empty asm: what is derived from it is
    // recomputed here instead of being hoisted out of the piece loop, where
    // it would stay live in every role's registers.
    int me = tid;
    asm volatile("" : "+v"(me));
    // The first two slots' loads go out together; the sum keeps range
    // order, starting from +0 as a plain running sum would (x + 0 is x,
    // except that -0 becomes +0).
    auto slot_rsrc = [&](int k) {
      return __builtin_amdgcn_make_buffer_rsrc(a.part + static_cast<size_t>(slot_of(pc, q0 + k)) * kSlot, 0,
                                               kSlot * 4, kBufferRsrcWord3);
    };
    auto load_slot = [&](int k, f32x4_t* d) {
      const auto r = slot_rsrc(k);
#pragma unroll
      for (int j = 0; j < kJ; ++j)
        d[j] = __builtin_bit_cast(f32x4_t,
                                  __builtin_amdgcn_raw_buffer_load_b128(r, (me + kThreads * j) * 16, 0, kCacheSc1));
    };
    f32x4_t sum[kJ], u[kJ];
    load_slot(0, sum);
    if (np > 1) load_slot(1, u);
#pragma unroll
    for (int j = 0; j < kJ; ++j) sum[j] += f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int k = 1; k < np; ++k) {
      if (k > 1) load_slot(k, u);
#pragma unroll
      for (int j = 0; j < kJ; ++j) sum[j] += u[j];
    }
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int e = me + kThreads * j;
      if (e >= kE) break;
      const int ln = e & 63, nb = (e >> 6) & 7, rs = (e >> 9) & 3, wv = e >> 11;
      const int n = pc.n_base + 128 * wv + 16 * nb + (ln & 15);
      if (n < a.N) store_y4(n, pc.m0 + 16 * rs + 4 * (ln >> 4), sum[j]);
    }
  };

  auto run_piece = [&](auto&& body, int tile, int c_begin, int c_end) {
    Piece pc;
    pc.tile = tile;
    pc.t0 = tile * Gc;
    pc.c_begin = c_begin;
    pc.c_end = c_end;
    pc.full = c_begin == 0 && c_end == a.Gc;
    // Partial-sum slot: stream-K, 2p for the piece that opens workgroup p's
    // range, 2p + 1 for the one that closes it; split-K, L.
    pc.slot = a.wgs > 0 ? 2 * L + (pc.t0 + c_begin == r0 ? 0 : 1) : L;
    const int gi = tile / a.ntiles;
    pc.m0 = gi * kGT;
    pc.n_base = (tile - gi * a.ntiles) * kBN;
    pc.cnt = c_end - c_begin;           // >= 1
    pc.g_row = static_cast<int64_t>(gi) * a.Gc;

    const uint32_t* otab = a.offsets + pc.g_row + c_begin;
    for (int i = tid; i <= pc.cnt; i += kThreads) offtab[i] = otab[i];
    __syncthreads();
    body(pc);
    if (!pc.full) {
      int q0, np;
      if (count_split(pc, &q0, &np)) {
        reduce_tile(pc, q0, np);
        if (tid == 0) __hip_atomic_store(&a.counters[pc.tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();   // LDS buffers and offtab are reused by the next piece
  };
  // Runs body(piece) for every piece of this workgroup: first the pieces of
  // its range [r0, r1) from the last to the first, then (stream-K) its whole
  // tiles.  Each role calls it with its own body, so that the values a role
  // keeps across pieces are only live in that role's code.  All roles pass
  // the same barriers: the offset table fill, the body's, and those of the
  // split-tile count.
  auto for_pieces = [&](auto&& body) {
    for (int64_t u1 = r1; u1 > r0;) {
      const int tile = static_cast<int>((u1 - 1) / Gc);
      const int64_t t0 = tile * Gc;
      const int c_begin = static_cast<int>(max(r0, t0) - t0);
      run_piece(body, tile, c_begin, static_cast<int>(u1 - t0));
      u1 = t0 + c_begin;
    }
    for (int r = 0; r < R; ++r) run_piece(body, L + r * nblk, 0, a.Gc);
  };

  if (w < 4) {
    // ---------------- consumer ----------------
    const int nl = 128 * w;               // first token of this wave inside the tile
    for_pieces([&](const Piece& pc) {
      f32x4_t acc[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // This wave's 8 X^T fragments of half column h of column c: lane l of
      // fragment nb holds token nl + 16 nb + l % 16, k 64 c + 32 h + 8 (l / 16) .. +7.
      const u32x4_t* xw = a.xf + (static_cast<size_t>(pc.n_base / kBN) * a.kb32 * 32 + 8 * w) * 64 + lane;
      auto xload = [&](int c, int h, u32x4_t* d) {
        const u32x4_t* src = xw + static_cast<size_t>(2 * c + h) * (32 * 64);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) d[nb] = src[64 * nb];
      };
      auto mma = [&](int c, int h, const u32x4_t* bf) {
        u32x4_t af[4];
#pragma unroll
        for (int rs = 0; rs < 4; ++rs) af[rs] = abuf[c & 1][(rs * 2 + h) * 64 + lane];
#pragma unroll
        for (int rs = 0; rs < 4; ++rs)
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
            acc[rs][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, af[rs]),
                                                                 __builtin_bit_cast(half8_t, bf[nb]), acc[rs][nb], 0,
                                                                 0, 0);
      };
      // Two register sets, each loaded a half column before its use; the
      // scheduling barriers keep the compiler from sinking the loads to
      // their use.
      u32x4_t xa[8], xb[8];
      xload(pc.c_begin, 0, xa);
      __syncthreads();   // builders: first three columns' values and bitmap words landed
      __syncthreads();   // builders: first column's A tile rebuilt
      for (int c = pc.c_begin; c < pc.c_end; ++c) {
        xload(c, 1, xb);
        __builtin_amdgcn_sched_barrier(0);
        mma(c, 0, xa);
        __builtin_amdgcn_sched_barrier(0);
        if (c + 1 < pc.c_end) xload(c + 1, 0, xa);
        __builtin_amdgcn_sched_barrier(0);
        mma(c, 1, xb);
        __syncthreads();   // builders: column c+1's A tile rebuilt; abuf[c & 1] free
      }
      // lane l of block (rs, nb): rows 16rs + 4(l/16) + i, token 16nb + l%16.
      if (pc.full) {
#pragma unroll
        for (int rs = 0; rs < 4; ++rs)
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
            const int n = pc.n_base + nl + nb * 16 + row;
            if (n < a.N) store_y4(n, pc.m0 + rs * 16 + 4 * kb, acc[rs][nb]);
          }
      } else {
        // Stores that reach the device-coherent level (sc1), as agent-scope
        // atomic stores do, 16 bytes at a time; the slot keeps the
        // accumulators in register order, [wave][rs][nb][lane][i].
        const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(a.part + static_cast<size_t>(pc.slot) * kSlot + w * (kSlot / 4),
                                                            0, kSlot, kBufferRsrcWord3);
#pragma unroll
        for (int rs = 0; rs < 4; ++rs)
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc[rs][nb]), rsrc,
                                                   ((rs * 8 + nb) * 64 + lane) * 16, 0, kCacheSc1);
      }
    });
  } else {
    // ---------------- builder ----------------
    for_pieces([&](const Piece& pc) {
      const int bw = w - 4;               // A fragments 2bw, 2bw+1: rows 16bw .. +15; value chunk slots 64bw + 256i + lane
      const uint64_t top = a.values_alloc - 16;
      const int r8 = row & 7;
      const int bt_lane = 4 * (kb >> 1) + 2 * (row >> 3) + (kb & 1);
      const uint64_t rowmask = (1ull << (8 * r8)) - 1ull;
      // Values of column c into stage[c % 3]: slot 64bw + lane + 256i of
      // the buffer takes chunk slot of the GroupTile's range; an instruction
      // whose 64 slots all lie past the range is not issued.  Returns how
      // many were.
      auto dma_v = [&](int c) {
        const uint32_t o0 = offtab[c - pc.c_begin], o1 = offtab[c - pc.c_begin + 1];
        const uint64_t a0 = min(chunk_start<false>(o0), top);
        const uint32_t nch = __builtin_amdgcn_readfirstlane(
            min(chunk_count<false>(o1, a0), static_cast<uint32_t>((top - a0) >> 4) + 1u));
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.values + a0);
        const uint32_t dst = lds_addr(stage[c % 3]) + 16 * 64 * bw;
        int issued = 0;
#pragma unroll
        for (int i = 0; i < kCpt; ++i) {
          const uint32_t slot0 = static_cast<uint32_t>(64 * bw + kPThreads * i);
          if (slot0 < nch) {
            lds_dma16(src + min(slot0 + lane, nch - 1), dst + 16 * kPThreads * i);
            ++issued;
          }
        }
        return issued;
      };
      // The 64 bitmap words of column c into bmw[c % 3] (builder 0, lanes
      // 0-31, two words each).  Returns how many loads this wave issued.
      auto dma_bm = [&](int c) {
        if (bw != 0) return 0;
        if (lane < 32) lds_dma16(a.bitmaps + (pc.g_row + c) * kBtPerGt + 2 * lane, lds_addr(bmw[c % 3]));
        return 1;
      };
      // Rebuild inputs of column c for this wave's two fragments: for the
      // BitmapTile row a lane rebuilds, the bitmap and the element index of
      // the tile's first value inside the staged chunk range.
      auto prep = [&](int c) {
        const u32x2_t bmv = reinterpret_cast<const u32x2_t*>(bmw[c % 3])[lane];
        RbIn<2> in;
        const uint32_t o0 = offtab[c - pc.c_begin];
        const uint64_t a0 = min(chunk_start<false>(o0), top);
        const uint32_t pc = __builtin_popcount(bmv.x) + __builtin_popcount(bmv.y);
        const uint32_t ebase = wave_inclusive_scan(pc) - pc + chunk_delta<false>(o0, a0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = 2 * bw + j;
          const int bt = 16 * (f >> 1) + 8 * (f & 1) + bt_lane;
          in.base[j] = __builtin_amdgcn_ds_bpermute(bt << 2, ebase);
          in.lo[j] = __builtin_amdgcn_ds_bpermute(bt << 2, bmv.x);
          in.hi[j] = __builtin_amdgcn_ds_bpermute(bt << 2, bmv.y);
        }
        return in;
      };
      auto rebuild = [&](int c, const RbIn<2>& in) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int f = 2 * bw + j;
          const uint64_t bm = (static_cast<uint64_t>(in.hi[j]) << 32) | in.lo[j];
          const uint32_t rb = in.base[j] + __popcll(bm & rowmask);
          const uint32_t byte = static_cast<uint32_t>(bm >> (8 * r8)) & 0xFFu;
          abuf[c & 1][f * 64 + lane] = __builtin_bit_cast(u32x4_t, rebuild_row<false>(stage[c % 3], lut, rb, byte));
        }
      };

      for (int c = pc.c_begin; c < min(pc.c_begin + 3, pc.c_end); ++c) {
        dma_bm(c);
        dma_v(c);
      }
      USW_PRODUCER_BARRIER(0);   // first three columns' values and bitmap words landed
      rebuild(pc.c_begin, prep(pc.c_begin));
      __syncthreads();
      // Column c: rebuild column c+1 (staged at least a column before), then
      // stage column c+3 into the buffers column c used.  At the barrier
      // everything but those loads has landed: column c+2's values and
      // bitmap words, which the next column's rebuild reads.
      for (int c = pc.c_begin; c < pc.c_end; ++c) {
        if (c + 1 < pc.c_end) rebuild(c + 1, prep(c + 1));
        int n = 0;
        if (c + 3 < pc.c_end) {
          n += dma_bm(c + 3);
          n += dma_v(c + 3);
        }
        builder_barrier(n);
      }
      __builtin_amdgcn_s_waitcnt(0);   // no LDS write of this wave outlives the piece
    });
  }
}

constexpr int64_t kComputeUnits = 256;
constexpr int64_t kMinStreamCols = 8;   // fewest GroupTile columns a stream-K workgroup takes

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

namespace usw {

PrefillPlan prefill_plan(const Geometry& g, int N, int splits_req, bool tiles512) {
  PrefillPlan p;
  p.waves = (N > 256 && tiles512) ? 8 : 4;
  const int bn = 64 * p.waves;
  p.ntiles = (N + bn - 1) / bn;
  p.wgs = 0;
  const int64_t tiles = g.Gr * p.ntiles;
  const int64_t smin = (g.Gc + kMaxCols - 1) / kMaxCols;
  if (p.waves == 8 && splits_req <= 0 && smin == 1) {
    // Stream-K: every compute unit takes the same number of GroupTile
    // columns (at least kMinStreamCols, unless the whole problem is smaller).
    const int64_t units = tiles * g.Gc;
    p.wgs = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(kComputeUnits, units / kMinStreamCols)));
    p.splits = 1;
    return p;
  }
  int64_t s = splits_req;
  if (s <= 0) {
    // One workgroup per compute unit is resident.  Split K only when the
    // tiles leave more than half of the compute units idle; each split keeps
    // at least 16 GroupTile columns.
    s = 1;
    if (tiles * 2 <= kComputeUnits) s = std::min<int64_t>((kComputeUnits + tiles - 1) / tiles, std::max<int64_t>(1, g.Gc / 16));
  }
  p.splits = static_cast<int>(std::max(smin, std::max<int64_t>(1, std::min<int64_t>(s, g.Gc))));
  return p;
}

static bool uses_slots(const PrefillPlan& p) { return p.waves == 8 && (p.wgs > 0 || p.splits > 1); }

size_t prefill_counter_bytes(const Geometry& g, const PrefillPlan& p) {
  return (p.splits > 1 || p.wgs > 0) ? align256(static_cast<size_t>(4) * g.Gr * p.ntiles) : 0;
}
// Slot bytes of the 512-token kernel's split tiles (0 without them): slots
// of 512 tokens x 64 rows, two per stream-K workgroup (the pieces that open
// and close its range), one per split-K workgroup.
static size_t slot_bytes(const Geometry& g, const PrefillPlan& p) {
  if (!uses_slots(p)) return 0;
  const size_t slots = p.wgs > 0 ? static_cast<size_t>(2) * p.wgs : static_cast<size_t>(g.Gr) * p.ntiles * p.splits;
  return align256(slots * 512 * kGT * sizeof(float));
}
// Bytes of the fragment-ordered copy of X the 512-token kernel reads (0 for
// the 256-token kernel).
static size_t xfrag_bytes(const Geometry& g, const PrefillPlan& p) {
  return p.waves == 8 ? align256(static_cast<size_t>(p.ntiles) * 512 * g.K * sizeof(uint16_t)) : 0;
}
size_t prefill_workspace_bytes(const Geometry& g, int N, const PrefillPlan& p) {
  const size_t cb = prefill_counter_bytes(g, p);
  if (p.waves == 8) return cb + slot_bytes(g, p) + xfrag_bytes(g, p);
  if (cb == 0) return 0;
  return cb + static_cast<size_t>(p.splits) * N * g.M * sizeof(float);
}
usw_status prefill_launch(const usw_fmt* f, const Geometry& g, const uint16_t* X, void* Y, bool f16out, int N,
                          uint32_t* counters, float* part, const PrefillPlan& p, void* stream) {
  PArgs a;
  a.bitmaps = f->bitmaps;
  a.offsets = f->offsets;
  a.values = static_cast<const uint8_t*>(f->values);
  a.X = X;
  a.Y = Y;
  const bool shared = prefill_counter_bytes(g, p) > 0;
  a.counters = shared ? counters : nullptr;
  a.part = shared ? part : nullptr;
  // Workspace after the counters: the slots, then the copy of X.
  a.xf = p.waves == 8 ? reinterpret_cast<const u32x4_t*>(reinterpret_cast<uint8_t*>(part) + slot_bytes(g, p)) : nullptr;
  a.kb32 = static_cast<int>(g.K / 32);
  a.values_alloc = values_alloc_bytes(f->val_type, f->nnz);
  a.M = static_cast<int>(g.M);
  a.K = static_cast<int>(g.K);
  a.N = N;
  a.Gc = static_cast<int>(g.Gc);
  a.splits = p.splits;
  a.ntiles = p.ntiles;
  a.tiles = static_cast<int>(g.Gr * p.ntiles);
  a.wgs = p.wgs;
  const int64_t nblk = p.wgs > 0 ? p.wgs : g.Gr * p.ntiles * p.splits;
  a.remap = nblk % 8 == 0 ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(nblk));
  if (p.waves == 8) {
    const int64_t pairs = static_cast<int64_t>(p.ntiles) * (a.kb32 / 2) * 32 * 64;
    if (pairs >= (int64_t(1) << 31)) return USW_ERR_UNSUPPORTED;
    xfrag_kernel<<<dim3(static_cast<unsigned>((pairs + 255) / 256)), 256, 0, s>>>(
        X, const_cast<u32x4_t*>(a.xf), N, a.K, static_cast<uint32_t>(pairs));
    if (f16out) prefill_ws_kernel<true><<<grid, 512, 0, s>>>(a);
    else prefill_ws_kernel<false><<<grid, 512, 0, s>>>(a);
  } else {
    if (f16out) prefill_kernel<4, true><<<grid, 256, 0, s>>>(a);
    else prefill_kernel<4, false><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError() == hipSuccess ? USW_OK : USW_ERR_HIP;
}

}  // namespace usw
