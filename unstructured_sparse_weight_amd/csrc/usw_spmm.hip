// Device half of libusw: the bitmap SpMM kernels for gfx950 and the
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
//   * Per GroupTile a wave loads the 512 B of bitmaps and the value range
//     [offsets[g], offsets[g+1]) with 16-byte loads from a 16-byte aligned
//     start into a private LDS buffer, then rebuilds dense fp16 fragments of
//     the MFMA A operand.  v_mfma_f32_16x16x32_f16 gives lane l the row
//     l%16 and the 8 consecutive columns 8*(l/16)..+7 of a 16x32 block; that
//     is exactly one row of one BitmapTile, whose kept values are contiguous
//     in the value stream.  The lane finds where they start (GroupTile offset
//     + popcounts of earlier BitmapTiles, from a wave prefix scan, + popcount
//     of the earlier rows of its own BitmapTile) and expands them into 8
//     slots with two aligned LDS windows and v_perm_b32 byte selectors looked
//     up by the row's 8-bit mask (zero for clear bits).
//   * The rebuilt 16x32 fragment is multiplied by the X^T fragment (X is
//     [N][K], so each lane's 8 k values are one 16-byte load) on the matrix
//     cores with fp32 accumulation; for N <= 32 this keeps the vector ALUs
//     free for the rebuild, which is what bounds the kernel after HBM.
//   * Partial sums of the waves of a workgroup are added in LDS in a fixed
//     order; across workgroups (split K) they go through an fp32 workspace and
//     a second kernel adds them in a fixed order, so results are
//     deterministic.

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
// Per-wave value buffer: a dense GroupTile (4096 fp16), the <16 B head before
// the first value, and the <16 B a window may read past the last value.
constexpr int kVbufF16 = 8192 + 64;
constexpr int kVbufI4 = 2048 + 64;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// v_perm_b32 byte selectors that expand the packed values of one 4-bit
// nibble of a BitmapTile row into 4 fp16 slots.  Packed value k of the
// window occupies bytes 2k, 2k+1 (window dword 0 = selector bytes 0-3, dword
// 1 = bytes 4-7); a clear bit selects 0x0C, which v_perm turns into 0x00.
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

// Two dwords holding packed fp16 values e and e+1, e+2, e+3 of an LDS
// buffer (element e starts at byte 2e; buffers are dword aligned).
__device__ __forceinline__ u32x2_t lds_window_f16(const uint8_t* buf, uint32_t e) {
  const uint32_t ba = 2u * e;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(buf + (ba & ~3u));
  const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
  u32x2_t w;
  w.x = __builtin_amdgcn_alignbyte(d1, d0, ba & 3u);
  w.y = __builtin_amdgcn_alignbyte(d2, d1, ba & 3u);
  return w;
}

template <int NB>
struct Frags {
  u32x4_t b[2][NB];  // X^T fragments for the two 32-column halves of a GroupTile
};

// X^T fragment for MFMA B: lane l holds X[n0 + l%16][k0 + 8*(l/16) .. +7].
__device__ __forceinline__ u32x4_t load_x_frag(const uint16_t* __restrict__ X, int K, int N, int n, int k) {
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (n < N) v = *reinterpret_cast<const u32x4_t*>(X + static_cast<size_t>(n) * K + k);
  return v;
}

// ---------------------------------------------------------------------------
// fp16 values, N <= 16*NB, NB in {1, 2}
// ---------------------------------------------------------------------------
template <int NB, bool OUT_F16>
__global__ __launch_bounds__(kThreads) void decode_f16_kernel(
    const uint64_t* __restrict__ bitmaps, const uint32_t* __restrict__ offsets,
    const uint8_t* __restrict__ values, const uint16_t* __restrict__ X, void* __restrict__ Y,
    float* __restrict__ ws, int M, int K, int N, int Gc, int splits) {
  __shared__ u32x4_t lut[256];
  // Staging (per wave: values, then bitmaps); reused for the final reduction.
  constexpr int kStage = kWaves * (kVbufF16 + 8 * kBtPerGt);
  constexpr int kRed = kWaves * 4 * NB * 64 * 4 * 4;
  static_assert(kRed <= kStage, "reduction fits the staging area");
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int gi = blockIdx.x / splits;
  const int sidx = blockIdx.x - gi * splits;

  for (int b = tid; b < 256; b += kThreads) {
    u32x4_t e;
    e.x = nibble_selector(b & 15, 0);
    e.y = nibble_selector(b & 15, 1);
    e.z = nibble_selector(b >> 4, 0);
    e.w = nibble_selector(b >> 4, 1);
    lut[b] = e;
  }
  __syncthreads();

  // Columns of GroupTiles this wave streams.
  const int parts = splits * kWaves;
  const int q = sidx * kWaves + w;
  const int c_begin = static_cast<int>(static_cast<int64_t>(Gc) * q / parts);
  const int c_end = static_cast<int>(static_cast<int64_t>(Gc) * (q + 1) / parts);

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

  uint8_t* vb = smem + w * kVbufF16;
  uint64_t* bb = reinterpret_cast<uint64_t*>(smem + kWaves * kVbufF16) + w * kBtPerGt;

  for (int c = c_begin; c < c_end; ++c) {
    const int64_t g = static_cast<int64_t>(gi) * Gc + c;
    const uint32_t o0 = offsets[g];
    const uint32_t o1 = offsets[g + 1];
    const uint64_t a0 = (2ull * o0) & ~15ull;               // 16-byte aligned start (bytes)
    const uint32_t nch = static_cast<uint32_t>((2ull * o1 - a0 + 15ull) >> 4);
    const uint32_t delta = static_cast<uint32_t>((2ull * o0 - a0) >> 1);   // elements before the first value

    // Stage bitmaps and values of GroupTile g in LDS.
    if (lane < 32) {
      const u32x4_t v = reinterpret_cast<const u32x4_t*>(bitmaps + g * kBtPerGt)[lane];
      reinterpret_cast<u32x4_t*>(bb)[lane] = v;
    }
    for (uint32_t ch = lane; ch < nch; ch += 64) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(values + a0 + 16ull * ch);
      *reinterpret_cast<u32x4_t*>(vb + 16 * ch) = v;
    }
    Frags<NB> fr;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        fr.b[ks][nb] = load_x_frag(X, K, N, nb * 16 + row, c * kGT + ks * 32 + kb * 8);
    wave_sync();

    // Exclusive prefix of BitmapTile popcounts: lane i <-> BitmapTile i.
    const uint32_t pc = __popcll(bb[lane]);
    uint32_t inc = pc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t t = __shfl_up(inc, d);
      if (lane >= d) inc += t;
    }
    const uint32_t ebase = inc - pc;

#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int bt = 16 * rs + 8 * ks + bt_lane;
        const uint64_t bm = bb[bt];
        const uint32_t base = __shfl(ebase, bt);
        const uint32_t rb = base + __popcll(bm & rowmask) + delta;
        const uint32_t byte = static_cast<uint32_t>(bm >> (8 * r8)) & 0xFFu;
        const uint32_t pcl = __builtin_popcount(byte & 0xFu);
        const u32x4_t sel = lut[byte];
        const u32x2_t lo = lds_window_f16(vb, rb);
        const u32x2_t hi = lds_window_f16(vb, rb + pcl);
        u32x4_t a;
        a.x = __builtin_amdgcn_perm(lo.y, lo.x, sel.x);
        a.y = __builtin_amdgcn_perm(lo.y, lo.x, sel.y);
        a.z = __builtin_amdgcn_perm(hi.y, hi.x, sel.z);
        a.w = __builtin_amdgcn_perm(hi.y, hi.x, sel.w);
        const half8_t ah = __builtin_bit_cast(half8_t, a);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[rs][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(half8_t, fr.b[ks][nb]),
                                                               acc[rs][nb], 0, 0, 0);
      }
    }
    wave_sync();
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
    if (n >= N) continue;
    const int rs = ml >> 4, r16 = ml & 15;
    const int ln = ((r16 >> 2) << 4) | (n & 15);
    const int i = r16 & 3;
    const int nb = n >> 4;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s += red[(((ww * 4 + rs) * NB + nb) * 64 + ln) * 4 + i];
    const size_t yi = static_cast<size_t>(n) * M + m0 + ml;
    if (splits > 1) {
      ws[static_cast<size_t>(sidx) * N * M + yi] = s;
    } else if (OUT_F16) {
      reinterpret_cast<_Float16*>(Y)[yi] = static_cast<_Float16>(s);
    } else {
      reinterpret_cast<float*>(Y)[yi] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// INT4 values with per-row fp16 scales, N <= 16*NB
// ---------------------------------------------------------------------------

// v_perm selectors that expand the 8 packed nibbles of one BitmapTile row
// into 8 byte slots.  Packed nibble k sits in byte k/2 of `lo4` (k even) or
// of `hi4` (k odd), where lo4 = w & 0x0F0F0F0F and hi4 = (w >> 4) & 0x0F0F0F0F;
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

template <int NB, bool OUT_F16>
__global__ __launch_bounds__(kThreads) void decode_i4_kernel(
    const uint64_t* __restrict__ bitmaps, const uint32_t* __restrict__ offsets,
    const uint8_t* __restrict__ values, const uint16_t* __restrict__ scales, const uint16_t* __restrict__ X,
    void* __restrict__ Y, float* __restrict__ ws, int M, int K, int N, int Gc, int splits) {
  __shared__ u32x2_t lut[256];
  constexpr int kStage = kWaves * (kVbufI4 + 8 * kBtPerGt);
  constexpr int kRed = kWaves * 4 * NB * 64 * 4 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStage > kRed ? kStage : kRed];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int gi = blockIdx.x / splits;
  const int sidx = blockIdx.x - gi * splits;

  for (int b = tid; b < 256; b += kThreads) {
    u32x2_t e;
    e.x = nibble_byte_selector(b, 0);
    e.y = nibble_byte_selector(b, 1);
    lut[b] = e;
  }
  __syncthreads();

  const int parts = splits * kWaves;
  const int q = sidx * kWaves + w;
  const int c_begin = static_cast<int>(static_cast<int64_t>(Gc) * q / parts);
  const int c_end = static_cast<int>(static_cast<int64_t>(Gc) * (q + 1) / parts);

  const int row = lane & 15;
  const int kb = lane >> 4;
  const int r8 = row & 7;
  const int bt_lane = 4 * (kb >> 1) + 2 * (row >> 3) + (kb & 1);
  const uint64_t rowmask = (1ull << (8 * r8)) - 1ull;

  f32x4_t acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint8_t* vb = smem + w * kVbufI4;
  uint64_t* bb = reinterpret_cast<uint64_t*>(smem + kWaves * kVbufI4) + w * kBtPerGt;
  const _Float16 kBias = static_cast<_Float16>(-1032.0f);

  for (int c = c_begin; c < c_end; ++c) {
    const int64_t g = static_cast<int64_t>(gi) * Gc + c;
    const uint32_t o0 = offsets[g];
    const uint32_t o1 = offsets[g + 1];
    const uint64_t a0 = (static_cast<uint64_t>(o0) >> 1) & ~15ull;     // byte address, 16-aligned
    const uint64_t bend = (static_cast<uint64_t>(o1) + 1) >> 1;         // first byte past the last nibble
    const uint32_t nch = static_cast<uint32_t>((bend - a0 + 15ull) >> 4);
    const uint32_t delta = static_cast<uint32_t>(o0 - 2 * a0);         // nibbles before the first value

    if (lane < 32) {
      const u32x4_t v = reinterpret_cast<const u32x4_t*>(bitmaps + g * kBtPerGt)[lane];
      reinterpret_cast<u32x4_t*>(bb)[lane] = v;
    }
    for (uint32_t ch = lane; ch < nch; ch += 64) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(values + a0 + 16ull * ch);
      *reinterpret_cast<u32x4_t*>(vb + 16 * ch) = v;
    }
    Frags<NB> fr;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        fr.b[ks][nb] = load_x_frag(X, K, N, nb * 16 + row, c * kGT + ks * 32 + kb * 8);
    wave_sync();

    const uint32_t pc = __popcll(bb[lane]);
    uint32_t inc = pc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t t = __shfl_up(inc, d);
      if (lane >= d) inc += t;
    }
    const uint32_t ebase = inc - pc;

#pragma unroll
    for (int rs = 0; rs < 4; ++rs) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int bt = 16 * rs + 8 * ks + bt_lane;
        const uint64_t bm = bb[bt];
        const uint32_t base = __shfl(ebase, bt);
        const uint32_t rb = base + __popcll(bm & rowmask) + delta;      // nibble index in vbuf
        const uint32_t byte = static_cast<uint32_t>(bm >> (8 * r8)) & 0xFFu;
        const u32x2_t sel = lut[byte];
        // 8 packed nibbles starting at nibble rb.
        const uint32_t ba = rb >> 1;
        const uint32_t* p = reinterpret_cast<const uint32_t*>(vb + (ba & ~3u));
        const uint32_t sh = ((ba & 3u) << 3) | ((rb & 1u) << 2);
        const uint32_t win = __builtin_amdgcn_alignbit(p[1], p[0], sh);
        const uint32_t lo4 = win & 0x0F0F0F0Fu;
        const uint32_t hi4 = (win >> 4) & 0x0F0F0F0Fu;
        // Slots as bytes; xor 8 maps two's-complement nibble q to q + 8 in [0, 15]
        // (an empty slot's 0 becomes 8, i.e. q = 0).
        const uint32_t e0 = __builtin_amdgcn_perm(hi4, lo4, sel.x) ^ 0x08080808u;
        const uint32_t e1 = __builtin_amdgcn_perm(hi4, lo4, sel.y) ^ 0x08080808u;
        // fp16 bit pattern 0x6400 | u is 1024 + u exactly; subtracting 1032 leaves q.
        u32x4_t a;
        a.x = __builtin_amdgcn_perm(0x64646464u, e0, 0x04010400u);
        a.y = __builtin_amdgcn_perm(0x64646464u, e0, 0x04030402u);
        a.z = __builtin_amdgcn_perm(0x64646464u, e1, 0x04010400u);
        a.w = __builtin_amdgcn_perm(0x64646464u, e1, 0x04030402u);
        half8_t ah = __builtin_bit_cast(half8_t, a);
        ah += kBias;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[rs][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, __builtin_bit_cast(half8_t, fr.b[ks][nb]),
                                                               acc[rs][nb], 0, 0, 0);
      }
    }
    wave_sync();
  }

  __syncthreads();
  float* redbuf = reinterpret_cast<float*>(smem);   // [kWaves][4][NB][64 lanes][4]
#pragma unroll
  for (int rs = 0; rs < 4; ++rs)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      *reinterpret_cast<f32x4_t*>(redbuf + (((w * 4 + rs) * NB + nb) * 64 + lane) * 4) = acc[rs][nb];
  __syncthreads();

  const int m0 = gi * kGT;
  for (int e = tid; e < 64 * 16 * NB; e += kThreads) {
    const int n = e >> 6;
    const int ml = e & 63;
    if (n >= N) continue;
    const int rs = ml >> 4, r16 = ml & 15;
    const int ln = ((r16 >> 2) << 4) | (n & 15);
    const int i = r16 & 3;
    const int nb = n >> 4;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) s += redbuf[(((ww * 4 + rs) * NB + nb) * 64 + ln) * 4 + i];
    const size_t yi = static_cast<size_t>(n) * M + m0 + ml;
    if (splits > 1) {
      // Partial sums stay unscaled; the reduction applies the row scale.
      ws[static_cast<size_t>(sidx) * N * M + yi] = s;
    } else {
      const _Float16 sh16 = __builtin_bit_cast(_Float16, scales[m0 + ml]);
      const float v = s * static_cast<float>(sh16);
      if (OUT_F16)
        reinterpret_cast<_Float16*>(Y)[yi] = static_cast<_Float16>(v);
      else
        reinterpret_cast<float*>(Y)[yi] = v;
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
  s = std::max(1, std::min<int>(s, static_cast<int>(g.Gc / kWaves > 0 ? g.Gc / kWaves : 1)));
  p.splits = s;
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
  if (g->M > INT32_MAX / 64 || static_cast<int64_t>(N) * g->M > (int64_t(1) << 40)) return USW_ERR_BAD_SHAPE;
  return USW_OK;
}

size_t workspace_bytes(const usw::Geometry& g, const Plan& p) {
  if (p.splits <= 1) return 0;
  return static_cast<size_t>(p.splits) * p.nchunk * g.M * sizeof(float);
}

usw_status spmm_impl(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N, void* ws,
                     size_t ws_bytes, void* stream, int splits_req) {
  usw::Geometry g;
  usw_status st = check_common(f, y_type, N, &g);
  if (st) return st;
  if (!X || !Y || !f->bitmaps || !f->offsets || !f->values) return USW_ERR_NULL_ARG;
  if (f->val_type == USW_VAL_I4 && !f->scales) return USW_ERR_NULL_ARG;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(f->bitmaps) || !aligned16(f->values) ||
      (f->offsets && (reinterpret_cast<uintptr_t>(f->offsets) & 3u)))
    return USW_ERR_MISALIGNED;
  const Plan p = make_plan(g, N, splits_req);
  const size_t need = workspace_bytes(g, p);
  if (need > 0) {
    if (!ws || ws_bytes < need) return USW_ERR_WORKSPACE;
    if (!aligned16(ws)) return USW_ERR_MISALIGNED;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(g.Gr * p.splits));
  const dim3 block(kThreads);
  const int M = static_cast<int>(g.M), K = static_cast<int>(g.K), Gc = static_cast<int>(g.Gc);
  const size_t ybytes = y_type == USW_OUT_F16 ? 2 : 4;
  const bool f16out = y_type == USW_OUT_F16;
  const uint8_t* vals = static_cast<const uint8_t*>(f->values);
  float* wsf = static_cast<float*>(ws);

  for (int n0 = 0; n0 < N; n0 += p.nchunk) {
    const int nc = std::min(p.nchunk, N - n0);
    const uint16_t* Xc = X + static_cast<size_t>(n0) * K;
    void* Yc = static_cast<uint8_t*>(Y) + static_cast<size_t>(n0) * M * ybytes;
    const bool two = nc > 16;
    if (f->val_type == USW_VAL_F16) {
      if (two) {
        if (f16out)
          decode_f16_kernel<2, true><<<grid, block, 0, s>>>(f->bitmaps, f->offsets, vals, Xc, Yc, wsf, M, K, nc, Gc, p.splits);
        else
          decode_f16_kernel<2, false><<<grid, block, 0, s>>>(f->bitmaps, f->offsets, vals, Xc, Yc, wsf, M, K, nc, Gc, p.splits);
      } else {
        if (f16out)
          decode_f16_kernel<1, true><<<grid, block, 0, s>>>(f->bitmaps, f->offsets, vals, Xc, Yc, wsf, M, K, nc, Gc, p.splits);
        else
          decode_f16_kernel<1, false><<<grid, block, 0, s>>>(f->bitmaps, f->offsets, vals, Xc, Yc, wsf, M, K, nc, Gc, p.splits);
      }
    } else {
      if (two) {
        if (f16out)
          decode_i4_kernel<2, true><<<grid, block, 0, s>>>(f->bitmaps, f->offsets, vals, f->scales, Xc, Yc, wsf, M, K, nc, Gc, p.splits);
        else
          decode_i4_kernel<2, false><<<grid, block, 0, s>>>(f->bitmaps, f->offsets, vals, f->scales, Xc, Yc, wsf, M, K, nc, Gc, p.splits);
      } else {
        if (f16out)
          decode_i4_kernel<1, true><<<grid, block, 0, s>>>(f->bitmaps, f->offsets, vals, f->scales, Xc, Yc, wsf, M, K, nc, Gc, p.splits);
        else
          decode_i4_kernel<1, false><<<grid, block, 0, s>>>(f->bitmaps, f->offsets, vals, f->scales, Xc, Yc, wsf, M, K, nc, Gc, p.splits);
      }
    }
    if (hipGetLastError() != hipSuccess) return USW_ERR_HIP;
    if (p.splits > 1) {
      const size_t total = static_cast<size_t>(M) * nc;
      const unsigned rg = static_cast<unsigned>(std::min<size_t>((total + 255) / 256, 4096));
      const uint16_t* sc = f->val_type == USW_VAL_I4 ? f->scales : nullptr;
      if (f16out)
        splitk_reduce_kernel<true><<<rg, 256, 0, s>>>(wsf, Yc, sc, M, nc, p.splits);
      else
        splitk_reduce_kernel<false><<<rg, 256, 0, s>>>(wsf, Yc, sc, M, nc, p.splits);
      if (hipGetLastError() != hipSuccess) return USW_ERR_HIP;
    }
  }
  return USW_OK;
}

}  // namespace

extern "C" {

usw_status usw_spmm_workspace(const usw_fmt* f, int32_t N, size_t* bytes) {
  if (!bytes) return USW_ERR_NULL_ARG;
  usw::Geometry g;
  usw_status st = check_common(f, USW_OUT_F16, N, &g);
  if (st) return st;
  *bytes = workspace_bytes(g, make_plan(g, N, 0));
  return USW_OK;
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
  *bytes = workspace_bytes(g, make_plan(g, N, splits));
  return USW_OK;
}

usw_status usw_spmm_ex(const usw_fmt* f, const uint16_t* X, void* Y, int32_t y_type, int32_t N, int32_t splits,
                       void* ws, size_t ws_bytes, void* stream) {
  return spmm_impl(f, X, Y, y_type, N, ws, ws_bytes, stream, splits < 0 ? 0 : splits);
}

}  // extern "C"
