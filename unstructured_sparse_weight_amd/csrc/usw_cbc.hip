// Device half of the Tiled-CBC path: the dynamically pruned spMspV kernel
// for gfx950 and the usw_cbc_spmspv dispatcher.
//
// What is computed: y[m] = sum_k W_sp[m][k] x_k over the columns with
// |x_k| >= tau ("Unified Static-Dynamic Pruning for Efficient LLM
// Inference", section 2.2 dynamic pruning, section 4.1 Tiled-CBC, section
// 4.2 decode phase), N = 1, fp32 accumulation on the vector ALUs (one token
// leaves nothing for the matrix cores).
//
// Design (wave64):
//   * One workgroup of four waves owns one 256-row strip of GTiles and a
//     range of GTile columns; each wave streams its own run of GTiles over
//     all 256 rows (lane l holds rows 4l .. 4l+3), with its own LDS staging
//     area, so the main loop has no workgroup barrier.  The four waves' row
//     sums are added in LDS at the end, in a fixed order.
//   * Per GTile: lane j (mod 16) reads column j's ColInfo and x_j, and the
//     wave ballots |x_j| >= tau into a 16-bit mask of active columns.  The
//     padded runs of the active columns are loaded (16 bytes per load; lane
//     4c + q takes pieces q, q + 4, ... of column c) into registers one
//     GTile ahead and copied into LDS just before the next GTile's loads
//     reuse those registers; inactive columns cost neither bitmap nor value
//     bytes.  ColInfo, x and TileOffset run two GTiles ahead, since the
//     value loads depend on them.
//   * The active columns' bitmap words load with the values (lane 4c + q:
//     word q of column c).  At the copy, lane 4c + q also writes a table
//     entry: the word and the set bits of the column's earlier words.
//   * Per active column (a scalar loop over the mask) every lane reads the
//     entry of its word, takes its rank (the set bits below its first row)
//     by masked popcount, and expands the values of its four rows from one
//     LDS window with v_perm byte selectors indexed by its 4-bit nibble of
//     the bitmap (a clear bit selects 0), then four fp32 FMAs with x_k.
//   * Split K: each workgroup writes its row sums to an fp32 workspace with
//     device-coherent stores; the last workgroup of the strip (a per-strip
//     counter) adds them in split order and writes y.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "usw.h"
#include "usw_internal.h"
#include "usw_device.h"

namespace {

using namespace usw_dev;

constexpr int kTM = usw::kCbcTM;    // GTile rows
constexpr int kTK = usw::kCbcTK;    // GTile columns
constexpr int kWpc = usw::kCbcWpc;  // bitmap words per column
constexpr int kCWaves = 4;
constexpr int kCThreads = 64 * kCWaves;
constexpr int kColBytes = 2 * kTM;          // LDS bytes of one column's run (at most 256 values)
constexpr int kWaveBuf = kTK * kColBytes;   // a wave's staging area: 8 KB
constexpr int kLoads = kTM / 8 / 4;         // 16-byte loads per lane per GTile: 32 pieces, 4 lanes per column
static_assert(kTK == 16 && kWpc == 4 && kTM == 256, "lane 4c + q serves column c; words 0-3 cover 256 rows");
// A buffer offset past any values array the host accepts (< 2^31 - 16 bytes).
constexpr uint32_t kPastValues = 0x7FFFFFF0u;

struct CArgs {
  const uint64_t* __restrict__ bitmaps;
  const uint32_t* __restrict__ toff;
  const uint32_t* __restrict__ colinfo;
  const uint16_t* __restrict__ values;
  const uint16_t* __restrict__ x;
  void* __restrict__ y;
  float* __restrict__ part;          // split partial sums [splits][M] (splits > 1)
  uint32_t* __restrict__ counters;   // per strip: workgroups done (splits > 1), kept at 0 between calls
  uint64_t nvals;                    // stored values (elements)
  float tau;
  int M, Gc, splits;
  int remap;                         // 1: keep the splits of a strip on one XCD
};

// Metadata of one GTile: lane j (mod 16) holds column j's ColInfo and x_j;
// tbase is the GTile's TileOffset.
struct CMeta {
  uint32_t ci;
  float xf;
  uint32_t tbase;
};

// One GTile's loads, held in registers until they are copied into LDS.
struct CData {
  u32x4_t v[kLoads];   // lane 4c + q: pieces q + 4i of column c
  u32x2_t bw;          // lane 4c + q: bitmap word q of column c (0 when inactive)
  float xf;            // lane j: x_j
  uint32_t amask;      // active columns (wave-uniform)
};

__device__ __forceinline__ CMeta cbc_meta(const CArgs& a, int gi, int c, int lane) {
  const int64_t t = static_cast<int64_t>(gi) * a.Gc + c;
  CMeta m;
  m.ci = a.colinfo[t * kTK + (lane & 15)];
  m.xf = static_cast<float>(__builtin_bit_cast(_Float16, a.x[c * kTK + (lane & 15)]));
  m.tbase = a.toff[t];
  return m;
}

__device__ __forceinline__ void cbc_load(CData& d, const CArgs& a, int gi, int c, const CMeta& m, int lane) {
  const int64_t t = static_cast<int64_t>(gi) * a.Gc + c;
  d.xf = m.xf;
  d.amask = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(fabsf(m.xf) >= a.tau)) & 0xFFFFu;
  const uint32_t tbase = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(m.tbase));
  const int bc = lane >> 2, bq = lane & 3;
  const bool active = (d.amask >> bc) & 1u;
  const uint32_t cib = __shfl(m.ci, bc);
  const uint32_t pieces = active ? ((cib & 0xFFFFu) + 7u) >> 3 : 0u;
  // The GTile's bitmap words through a buffer descriptor of their 512
  // bytes: an inactive column's lanes take an offset past it and read zeros
  // without a fetch, and without a branch.
  const auto brs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint64_t*>(a.bitmaps + t * kTK * kWpc), 0,
                                                     kTK * kWpc * 8, kBufferRsrcWord3);
  const uint32_t boff = active ? 8u * static_cast<uint32_t>(bc * kWpc + bq) : 2u * kTK * kWpc * 8;
  d.bw = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(brs, static_cast<int>(boff), 0, 0));
  // Buffer loads over the whole values array: a lane past its column's run
  // (or on an inactive column) gets an offset beyond the array, which the
  // hardware answers with zeros without a fetch, so no branch is needed;
  // the same bound keeps a corrupt ColInfo inside the array.
  const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.values), 0,
                                                      static_cast<int>(2 * a.nvals), kBufferRsrcWord3);
  const uint32_t src0 = 2u * (tbase + (cib >> 16));
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const uint32_t q = static_cast<uint32_t>(bq + 4 * i);
    const uint32_t off = q < pieces ? src0 + 16u * q : kPastValues;
    d.v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc, static_cast<int>(off), 0, 0));
  }
}

// Every lane stores its pieces, zeros past the run included.  Lane 4c + q
// also writes table entry 4c + q: word q of column c (0 when inactive) and
// the set bits of words 0 .. q-1, a prefix over the lane's quad by DPP.
__device__ __forceinline__ void cbc_commit(const CData& d, uint8_t* buf, u32x4_t* tab, int lane) {
  const int bc = lane >> 2, bq = lane & 3;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) *reinterpret_cast<u32x4_t*>(buf + bc * kColBytes + 16 * (bq + 4 * i)) = d.v[i];
  const uint32_t pc = __builtin_popcount(d.bw.x) + __builtin_popcount(d.bw.y);
  uint32_t inc = pc;
  const uint32_t t1 = __builtin_amdgcn_update_dpp(0u, inc, 0x111, 0xf, 0xf, false);   // row_shr:1
  if (bq >= 1) inc += t1;
  const uint32_t t2 = __builtin_amdgcn_update_dpp(0u, inc, 0x112, 0xf, 0xf, false);   // row_shr:2
  if (bq >= 2) inc += t2;
  tab[lane] = u32x4_t{d.bw.x, d.bw.y, inc - pc, 0u};
}

// What a lane needs to find its four rows 4l .. 4l+3 in a column: they are
// bits sh .. sh+3 of word l / 16 (sh = 4 (l mod 16)); the masks keep the
// word's bits below sh.
struct CLane {
  uint32_t mlo, mhi;   // bits of the word's low / high half below sh
  uint32_t sh;         // sh mod 32
  bool hi;             // the nibble is in the high half
};

__device__ __forceinline__ CLane cbc_lane(int lane) {
  const uint32_t sh = 4u * static_cast<uint32_t>(lane & 15);
  CLane c;
  c.hi = sh >= 32u;
  c.sh = sh & 31u;
  c.mlo = c.hi ? 0xFFFFFFFFu : (1u << sh) - 1u;
  c.mhi = c.hi ? (1u << c.sh) - 1u : 0u;
  return c;
}

// Accumulate a staged GTile over its active columns.  Per column: the
// lane's table entry gives its rank (bits below its first row); its four
// rows' values are the kept ones among window values rank .. rank+3, placed
// by the 16-entry nibble selector table (clear bits select 0).
__device__ __forceinline__ void cbc_compute(float xf, uint32_t amask, const uint8_t* buf, const u32x4_t* tab,
                                            const uint32_t* lut, const CLane& cl, float (&acc)[4], int lane) {
  typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
  typedef uint32_t u32x3_t __attribute__((ext_vector_type(3)));
  const u32x4_t* mytab = tab + (lane >> 4);
  // A column's window and selectors, then its four FMAs.
  struct Col {
    u32x2_t w, sel;
    float xc;
  };
  auto fetch = [&](int cc) {
    Col c;
    c.xc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xf), cc));
    const u32x3_t e = *reinterpret_cast<const u32x3_t*>(mytab + kWpc * cc);
    const uint32_t rank = __builtin_popcount(e.y & cl.mhi) + __builtin_popcount(e.x & cl.mlo) + e.z;
    const uint32_t nib = __builtin_amdgcn_ubfe(cl.hi ? e.y : e.x, cl.sh, 4);
    c.w = lds_window_f16(buf + cc * kColBytes, rank);
    c.sel = reinterpret_cast<const u32x2_t*>(lut)[nib];
    return c;
  };
  auto accumulate = [&](const Col& c) {
    const half2_t v01 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(c.w.y, c.w.x, c.sel.x));
    const half2_t v23 = __builtin_bit_cast(half2_t, __builtin_amdgcn_perm(c.w.y, c.w.x, c.sel.y));
    acc[0] = fmaf(static_cast<float>(v01.x), c.xc, acc[0]);
    acc[1] = fmaf(static_cast<float>(v01.y), c.xc, acc[1]);
    acc[2] = fmaf(static_cast<float>(v23.x), c.xc, acc[2]);
    acc[3] = fmaf(static_cast<float>(v23.y), c.xc, acc[3]);
  };
  // Two columns per pass, so that their chains of LDS round trips overlap;
  // the sums are still added in column order.
  uint32_t m = amask;
  while (m != 0) {
    const int c0 = __builtin_ctz(m);
    m &= m - 1;
    if (m == 0) {
      accumulate(fetch(c0));
      break;
    }
    const int c1 = __builtin_ctz(m);
    m &= m - 1;
    const Col a0 = fetch(c0);
    const Col a1 = fetch(c1);
    accumulate(a0);
    accumulate(a1);
  }
}

template <bool OUT_F16>
__global__ __launch_bounds__(kCThreads, 4) void cbc_spmspv_kernel(CArgs a) {
  // Staging areas (then the wave reduction), 16 bytes that a window at the
  // end of the last column may read, and the word tables.
  __shared__ __attribute__((aligned(16))) uint8_t smem[kCWaves * kWaveBuf + 16];
  __shared__ __attribute__((aligned(16))) u32x4_t tabs[kCWaves][kTK * kWpc];
  __shared__ __attribute__((aligned(16))) uint32_t lut[32];
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
  const int parts = a.splits * kCWaves;
  const int qw = sidx * kCWaves + w;
  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * qw / parts);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (qw + 1) / parts);

  if (tid < 16) {
    u32x2_t e;
    e.x = nibble_selector(tid, 0);
    e.y = nibble_selector(tid, 1);
    reinterpret_cast<u32x2_t*>(lut)[tid] = e;
  }
  __syncthreads();
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  uint8_t* buf = smem + w * kWaveBuf;
  u32x4_t* tab = tabs[w];
  const CLane cl = cbc_lane(lane);
  if (c_begin < c_end) {
    // One register slot: a step copies GTile c's values into LDS, then
    // issues c+1's value loads into the same registers (and c+2's metadata)
    // and multiplies c while they are in flight.  Loads past the wave's last
    // GTile repeat it, so every step issues the same loads.
    const int c_last = c_end - 1;
    CMeta m1 = cbc_meta(a, gi, min(c_begin + 1, c_last), lane);
    CData d;
    cbc_load(d, a, gi, c_begin, cbc_meta(a, gi, c_begin, lane), lane);
    for (int c = c_begin; c < c_end; ++c) {
      // Loads go out at a raised wave priority (as in the TCA-BME decode).
      __builtin_amdgcn_s_setprio(2);
      const CMeta m2 = cbc_meta(a, gi, min(c + 2, c_last), lane);
      __builtin_amdgcn_s_setprio(0);
      cbc_commit(d, buf, tab, lane);
      const float xf = d.xf;
      const uint32_t amask = d.amask;
      __builtin_amdgcn_s_setprio(2);
      cbc_load(d, a, gi, min(c + 1, c_last), m1, lane);
      __builtin_amdgcn_s_setprio(0);
      wave_sync();
      cbc_compute(xf, amask, buf, tab, lut, cl, acc, lane);
      wave_sync();
      m1 = m2;
    }
  }

  // The waves' sums of strip row tid, added in wave order.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);   // [waves][256]
  *reinterpret_cast<f32x4_t*>(red + w * kTM + 4 * lane) = f32x4_t{acc[0], acc[1], acc[2], acc[3]};
  __syncthreads();
  float rsum = 0.f;
#pragma unroll
  for (int ww = 0; ww < kCWaves; ++ww) rsum += red[ww * kTM + tid];

  const int m = gi * kTM + tid;
  auto store_y = [&](float v) {
    if constexpr (OUT_F16)
      reinterpret_cast<_Float16*>(a.y)[m] = static_cast<_Float16>(v);
    else
      reinterpret_cast<float*>(a.y)[m] = v;
  };
  if (a.splits <= 1) {
    store_y(rsum);
    return;
  }
  auto part_rsrc = [&](int s) {
    return __builtin_amdgcn_make_buffer_rsrc(a.part + static_cast<size_t>(s) * a.M, 0, a.M * 4, kBufferRsrcWord3);
  };
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, rsum), part_rsrc(sidx), m * 4, 0, kCacheSc1);
  // Every thread's partial store has completed (s_waitcnt) before the
  // barrier that precedes the counter increment; the last workgroup reads
  // the partials with device-coherent loads after it has seen the count.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0)
    last_flag = __hip_atomic_fetch_add(&a.counters[gi], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                static_cast<uint32_t>(a.splits - 1);
  __syncthreads();
  if (!last_flag) return;
  float sum = 0.f;
  for (int s = 0; s < a.splits; ++s)
    sum += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(part_rsrc(s), m * 4, 0, kCacheSc1));
  store_y(sum);
  if (tid == 0) __hip_atomic_store(&a.counters[gi], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int cbc_splits(const usw::CbcGeometry& g, int splits_req) {
  int64_t s = splits_req;
  if (s <= 0) s = std::max<int64_t>(1, 1024 / g.gr);   // one round of four resident workgroups per compute unit
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, g.gc)));
}

size_t cbc_counter_bytes(const usw::CbcGeometry& g) { return (static_cast<size_t>(4 * g.gr) + 255) & ~size_t(255); }

size_t cbc_workspace_bytes(const usw::CbcGeometry& g, int splits) {
  if (splits <= 1) return 0;
  return cbc_counter_bytes(g) + static_cast<size_t>(splits) * g.M * sizeof(float);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

usw_status cbc_check(const usw_cbc_fmt* f, int32_t y_type, usw::CbcGeometry* g) {
  if (!f) return USW_ERR_NULL_ARG;
  usw_status st = usw::make_cbc_geometry(f->M, f->K, g);
  if (st) return st;
  if (f->reserved != 0) return USW_ERR_BAD_SHAPE;
  if (f->val_type != USW_VAL_F16 && f->val_type != USW_VAL_I4) return USW_ERR_BAD_DTYPE;
  if (y_type != USW_OUT_F16 && y_type != USW_OUT_F32) return USW_ERR_BAD_DTYPE;
  if (f->val_type != USW_VAL_F16 || f->tile_m != kTM || f->tile_k != kTK) return USW_ERR_UNSUPPORTED;
  if (f->nnz_padded < 0 || f->nnz_padded >= (int64_t(1) << 32)) return USW_ERR_BAD_SHAPE;
  if (g->M > (int64_t(1) << 28)) return USW_ERR_BAD_SHAPE;   // split partial sums are addressed in 32 bits
  // Values are read through one buffer descriptor with 32-bit byte offsets.
  if (2 * f->nnz_padded > static_cast<int64_t>(kPastValues)) return USW_ERR_BAD_SHAPE;
  return USW_OK;
}

}  // namespace

extern "C" {

usw_status usw_cbc_spmspv_workspace(const usw_cbc_fmt* f, int32_t splits, size_t* bytes, size_t* counter_bytes) {
  if (!bytes) return USW_ERR_NULL_ARG;
  usw::CbcGeometry g;
  usw_status st = cbc_check(f, USW_OUT_F16, &g);
  if (st) return st;
  const int s = cbc_splits(g, splits);
  *bytes = cbc_workspace_bytes(g, s);
  if (counter_bytes) *counter_bytes = s > 1 ? cbc_counter_bytes(g) : 0;
  return USW_OK;
}

usw_status usw_cbc_spmspv(const usw_cbc_fmt* f, const uint16_t* x, void* y, int32_t y_type, float tau,
                          int32_t splits, void* ws, size_t ws_bytes, void* stream) {
  usw::CbcGeometry g;
  usw_status st = cbc_check(f, y_type, &g);
  if (st) return st;
  if (!(tau >= 0.f)) return USW_ERR_UNSUPPORTED;
  if (!x || !y || !f->bitmaps || !f->tile_offsets || !f->colinfo || (f->nnz_padded > 0 && !f->values))
    return USW_ERR_NULL_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(f->bitmaps) || !aligned16(f->values) ||
      !aligned16(f->colinfo) || !aligned16(f->tile_offsets))
    return USW_ERR_MISALIGNED;
  const int s = cbc_splits(g, splits);
  const size_t need = cbc_workspace_bytes(g, s);
  if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws))) return USW_ERR_WORKSPACE;
  CArgs a;
  a.bitmaps = f->bitmaps;
  a.toff = f->tile_offsets;
  a.colinfo = f->colinfo;
  a.values = f->values;
  a.x = x;
  a.y = y;
  a.counters = need ? static_cast<uint32_t*>(ws) : nullptr;
  a.part = need ? reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + cbc_counter_bytes(g)) : nullptr;
  a.nvals = static_cast<uint64_t>(f->nnz_padded);
  a.tau = tau;
  a.M = static_cast<int>(g.M);
  a.Gc = static_cast<int>(g.gc);
  a.splits = s;
  const int64_t nblk = g.gr * s;
  a.remap = (s > 1 && nblk % 8 == 0) ? 1 : 0;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(nblk));
  if (y_type == USW_OUT_F16)
    cbc_spmspv_kernel<true><<<grid, kCThreads, 0, hs>>>(a);
  else
    cbc_spmspv_kernel<false><<<grid, kCThreads, 0, hs>>>(a);
  return hipGetLastError() == hipSuccess ? USW_OK : USW_ERR_HIP;
}

}  // extern "C"
