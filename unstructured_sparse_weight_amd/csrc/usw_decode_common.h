// Kernel arguments and the split-K epilogue shared by the decode kernels of
// both formats (TCA-BME and IE-BME).  A workgroup owns one 64-row strip of
// tiles and a range of tile columns; with split K its sums go to an fp32
// workspace and the last workgroup of the strip adds them in split order.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "usw_device.h"

namespace usw_dev {

struct Args {
  const uint64_t* __restrict__ bitmaps;
  const uint32_t* __restrict__ offsets;
  const uint8_t* __restrict__ values;
  const uint16_t* __restrict__ scales;
  const uint16_t* __restrict__ X;
  void* __restrict__ Y;
  float* __restrict__ part;       // split-K partial sums [splits][N][M] (splits > 1)
  uint32_t* __restrict__ counters;  // per 64-row strip: workgroups done (splits > 1), kept at 0 between calls
  const uint8_t* __restrict__ rowmap;  // IE-BME with reordered LTs: [NLT][lt_m] stored row of each row of W
  uint64_t values_alloc;           // padded size of the values buffer in bytes (>= 16)
  int M, K, N, Gc, splits;
  int remap;                       // 1: keep the splits of a strip on one XCD
  // IE-BME area grid (union_grid_decode_kernel): log2 of the area (= union
  // mask) rows and columns, of the area columns C_A and of Q = R_A C_A.
  int lg_am, lg_ak, lg_ca, lg_q;
};

// Writes a strip's sums to Y or, with split K, to split sidx's partial sums.
// sum_of(n, ml) gives token n's sums for strip rows ml .. ml+3.  Split K:
// the last workgroup of the strip to finish adds the partial sums of all its
// splits, in split order, and writes Y; the counter goes back to 0 for the
// next call.
template <int NB, bool I4, bool OUT_F16, class SumFn>
__device__ __forceinline__ void finish_strip(const Args& a, int gi, int sidx, int nthreads, uint32_t& last_flag,
                                             SumFn sum_of) {
  const int tid = threadIdx.x;
  const int m0 = gi * kGT;
  // Y[n][m0 + ml .. +3] from four consecutive row sums.
  auto store_y4 = [&](int n, int ml, f32x4_t v) {
    if constexpr (I4) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] *= static_cast<float>(__builtin_bit_cast(_Float16, a.scales[m0 + ml + j]));
    }
    const size_t yi = static_cast<size_t>(n) * a.M + m0 + ml;
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
  // Partial sums of split s: [N][M] fp32 at part + s N M, read and written
  // with device-coherent (sc1) 16-byte accesses.
  auto part_rsrc = [&](int s) {
    return __builtin_amdgcn_make_buffer_rsrc(a.part + static_cast<size_t>(s) * a.N * a.M, 0, a.N * a.M * 4,
                                             kBufferRsrcWord3);
  };
  // Thread element e: token n = e / 16, strip rows ml = 4 (e % 16) .. +3.
  for (int e = tid; e < 16 * 16 * NB; e += nthreads) {
    const int n = e >> 4;
    const int ml = 4 * (e & 15);
    if (n >= a.N) continue;
    const f32x4_t sum = sum_of(n, ml);
    if (a.splits > 1)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, sum), part_rsrc(sidx),
                                             (n * a.M + m0 + ml) * 4, 0, kCacheSc1);
    else
      store_y4(n, ml, sum);
  }
  if (a.splits <= 1) return;

  // Every thread's partial stores have completed
  // (s_waitcnt) before the barrier that precedes the counter increment, and
  // the last workgroup reads the partials with device-coherent loads issued
  // after it has seen the final count.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0)
    last_flag = __hip_atomic_fetch_add(&a.counters[gi], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                static_cast<uint32_t>(a.splits - 1);
  __syncthreads();
  if (!last_flag) return;
  for (int e = tid; e < 16 * a.N; e += nthreads) {
    const int n = e >> 4;
    const int ml = 4 * (e & 15);
    const int off = (n * a.M + m0 + ml) * 4;
    f32x4_t sum = {0.f, 0.f, 0.f, 0.f};
    // Up to four splits' loads in flight at once; added in split order.
    for (int p0 = 0; p0 < a.splits; p0 += 4) {
      f32x4_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (p0 + j < a.splits)
          v[j] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(part_rsrc(p0 + j), off, 0, kCacheSc1));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (p0 + j < a.splits) sum += v[j];
    }
    store_y4(n, ml, sum);
  }
  if (tid == 0) __hip_atomic_store(&a.counters[gi], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace usw_dev
