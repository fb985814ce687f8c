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
//     range of GTile columns; thread t owns strip row t, so no reduction
//     across waves is needed.
//   * Per GTile: lane j (mod 16) reads column j's ColInfo and x_j and the
//     wave ballots |x_j| >= tau into a 16-bit mask of active columns (the
//     same in every wave).  Wave w copies the padded runs of its active
//     columns 4w..4w+3 into LDS (16-byte loads, at most 32 per column);
//     inactive columns cost neither bitmap nor value bytes.
//   * The active columns' bitmap words arrive as one 8-byte load per lane
//     (lane 4c + q: word q of column c) with the popcounts of the words
//     before them in the column.  For each active column (a scalar loop over
//     the mask) the wave takes word w and its base with v_readlane, and each
//     lane whose bit is set takes its value at base + v_mbcnt of the word
//     (the masked popcount of the bits below it) from LDS and multiplies it
//     with x_k.
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
constexpr int kCThreads = kTM;      // one strip row per thread
static_assert(kCThreads == 256 && kTK == 16 && kWpc == 4, "four waves of 64 rows, four columns each to stage");

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

template <bool OUT_F16>
__global__ __launch_bounds__(kCThreads, 2) void cbc_spmspv_kernel(CArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 vals[kTK * kTM];   // column c's run at [256 c, 256 c + 256)
  __shared__ uint32_t last_flag;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = static_cast<int>(gridDim.x);
  const int b = static_cast<int>(blockIdx.x);
  const int L = a.remap ? (b & 7) * (nblk >> 3) + (b >> 3) : b;
  const int gi = L / a.splits;
  const int sidx = L - gi * a.splits;
  const int c_begin = static_cast<int>(static_cast<int64_t>(a.Gc) * sidx / a.splits);
  const int c_end = static_cast<int>(static_cast<int64_t>(a.Gc) * (sidx + 1) / a.splits);

  const int j = lane & 15;      // the column whose metadata this lane reads
  const int cs = 4 * w + (lane >> 4);   // the column whose run this lane helps to stage
  float acc = 0.f;
  for (int c = c_begin; c < c_end; ++c) {
    const int64_t t = static_cast<int64_t>(gi) * a.Gc + c;
    const uint32_t ci = a.colinfo[t * kTK + j];
    const float xf = static_cast<float>(__builtin_bit_cast(_Float16, a.x[c * kTK + j]));
    const uint32_t amask = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(fabsf(xf) >= a.tau)) & 0xFFFFu;
    const uint32_t tbase = __builtin_amdgcn_readfirstlane(a.toff[t]);

    // Stage the runs of the active columns 4w .. 4w+3 (lanes 16 q .. 16 q + 15
    // copy column 4w + q, pieces p and p + 16 of 16 bytes).  The bound on the
    // stored values keeps a corrupt ColInfo inside the buffer.
    const uint32_t cci = __shfl(ci, cs);
    if ((amask >> cs) & 1u) {
      const uint32_t pieces = ((cci & 0xFFFFu) + 7u) >> 3;
      const uint64_t src0 = static_cast<uint64_t>(tbase) + (cci >> 16);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t p = static_cast<uint32_t>(lane & 15) + 16u * h;
        if (p < pieces && src0 + 8u * p + 8u <= a.nvals)
          *reinterpret_cast<u32x4_t*>(vals + cs * kTM + 8 * p) =
              *reinterpret_cast<const u32x4_t*>(a.values + src0 + 8u * p);
      }
    }
    // The active columns' bitmap words, one per lane: lane 4 c + q holds word
    // q of column c, and the set bits of words 0..q-1 (a prefix inside each
    // group of four lanes).
    const int bc = lane >> 2, bq = lane & 3;
    u32x2_t bw = {0u, 0u};
    if ((amask >> bc) & 1u) bw = reinterpret_cast<const u32x2_t*>(a.bitmaps)[(t * kTK + bc) * kWpc + bq];
    const uint32_t pc = __builtin_popcount(bw.x) + __builtin_popcount(bw.y);
    const int q0 = lane & ~3;
    const uint32_t p0 = __shfl(pc, q0), p1 = __shfl(pc, q0 + 1), p2 = __shfl(pc, q0 + 2);
    const uint32_t before = (bq > 0 ? p0 : 0u) + (bq > 1 ? p1 : 0u) + (bq > 2 ? p2 : 0u);
    __syncthreads();

    // Each active column: word w holds this wave's 64 rows; the rank of a
    // kept row is the set bits of words 0..w-1 plus those below it in word w.
    for (uint32_t m = amask; m != 0; m &= m - 1) {
      const int cc = __builtin_ctz(m);
      const int src = 4 * cc + w;
      const uint32_t lo = __builtin_amdgcn_readlane(bw.x, src);
      const uint32_t hi = __builtin_amdgcn_readlane(bw.y, src);
      const uint32_t base = __builtin_amdgcn_readlane(before, src);
      const float xc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xf), cc));
      const uint64_t word = (static_cast<uint64_t>(hi) << 32) | lo;
      if ((word >> lane) & 1ull) {
        const uint32_t rank = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, base));
        acc = fmaf(static_cast<float>(vals[cc * kTM + (rank & (kTM - 1))]), xc, acc);
      }
    }
    __syncthreads();
  }

  // Row gi * 256 + tid.
  const int m = gi * kTM + tid;
  auto store_y = [&](float v) {
    if constexpr (OUT_F16)
      reinterpret_cast<_Float16*>(a.y)[m] = static_cast<_Float16>(v);
    else
      reinterpret_cast<float*>(a.y)[m] = v;
  };
  if (a.splits <= 1) {
    store_y(acc);
    return;
  }
  auto part_rsrc = [&](int s) {
    return __builtin_amdgcn_make_buffer_rsrc(a.part + static_cast<size_t>(s) * a.M, 0, a.M * 4, kBufferRsrcWord3);
  };
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc), part_rsrc(sidx), m * 4, 0, kCacheSc1);
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
  if (s <= 0) s = (2048 + g.gr / 2) / g.gr;   // about eight resident workgroups per compute unit
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
