// Device helpers shared by the bitmap SpMM kernels (gfx950, wave64): lane
// scans, the byte selectors and LDS windows that expand one BitmapTile row
// of packed values into the 8 dense slots of an MFMA A fragment, and the
// 16-byte chunk arithmetic of the value stream.
//
// Format: TCA-BME (blog "SpInfer: How bitmaps make sparse LLMs actually
// fast", section "How TCA-BME addresses the indexing overhead"); a value is
// found by masked popcount (same blog, "Shared Memory Bitmap Decoding").
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace usw_dev {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kGT = 64;                   // GroupTile side the kernels are built for
constexpr int kBtPerGt = 64;              // BitmapTiles per 64x64 GroupTile

// Buffer resource word 3 for raw byte-addressed buffers on this target, and
// the cache-policy operand that sets sc1: the access goes to the level that
// is coherent across the device (all XCDs), as agent-scope atomics do.
// Partial sums shared between workgroups travel this way, 16 bytes at a time.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kCacheSc1 = 16;

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// global_load_lds_dwordx4: lane l's 16 bytes at src land at LDS byte address
// lds + 16 l (lds the same in every lane; it goes to M0), counted by vmcnt
// like any vector load.  Issued through asm so that the compiler, which
// cannot tell which LDS bytes such a load writes, does not wait for every
// one in flight before each LDS read and barrier; the caller waits with an
// explicit vmcnt before the barrier that publishes the data.
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) T*)p));
}

// Wait until at most N of this wave's vector memory operations are in flight
// and its LDS operations are done, then a workgroup barrier.
#define USW_PRODUCER_BARRIER(N) asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" : : : "memory")

// The same load through the compiler's builtin, which counts it in vmcnt
// like any load (the LDS address is wave-uniform).  A wave that uses it must
// keep its own LDS accesses out of the compiler's sight (below), or the
// compiler waits for every such load before each of them.
template <typename T>
__device__ __forceinline__ void lds_dma16_tracked(const void* src, T* lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// LDS accesses of a wave that keeps LDS-DMA loads in flight, written as asm:
// before an LDS access the compiler would itself place an s_waitcnt vmcnt(0),
// i.e. wait for every load in flight (it cannot tell which LDS bytes they
// write).  The read waits for its own result.
__device__ __forceinline__ u32x2_t lds_load_b64(uint32_t addr) {
  u32x2_t v;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ void lds_store_b128(uint32_t addr, u32x4_t v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

// Wait until at most n of this wave's vector memory operations are in
// flight (n wave-uniform; above 15 it waits as for 15, i.e. never for fewer
// operations than asked).
#define USW_WAIT_VM(N) asm volatile("s_waitcnt vmcnt(" #N ")" : : : "memory")
__device__ __forceinline__ void wait_vm(int n) {
  switch (__builtin_amdgcn_readfirstlane(n)) {
    case 0: USW_WAIT_VM(0); break;
    case 1: USW_WAIT_VM(1); break;
    case 2: USW_WAIT_VM(2); break;
    case 3: USW_WAIT_VM(3); break;
    case 4: USW_WAIT_VM(4); break;
    case 5: USW_WAIT_VM(5); break;
    case 6: USW_WAIT_VM(6); break;
    case 7: USW_WAIT_VM(7); break;
    case 8: USW_WAIT_VM(8); break;
    case 9: USW_WAIT_VM(9); break;
    case 10: USW_WAIT_VM(10); break;
    case 11: USW_WAIT_VM(11); break;
    case 12: USW_WAIT_VM(12); break;
    case 13: USW_WAIT_VM(13); break;
    case 14: USW_WAIT_VM(14); break;
    default: USW_WAIT_VM(15); break;
  }
}

// Wait for this wave's LDS operations, then a workgroup barrier (vector
// memory loads stay in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

// Debug builds (-DUSW_DEBUG) fill LDS staging buffers with fp16 NaNs
// (0x7E00) at kernel entry, and the ring decode kernel refills each ring slot
// before its next loads are issued: a read of LDS that no stage wrote, or
// one that runs ahead of the load that fills it, then turns the product into
// NaN instead of a plausible stale value.  Release builds compile none of it.
constexpr uint32_t kLdsPoison = 0x7E007E00u;
#ifdef USW_DEBUG
__device__ __forceinline__ void lds_poison_all(void* p, uint32_t bytes) {
  uint32_t* q = static_cast<uint32_t*>(p);
  for (uint32_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) q[i] = kLdsPoison;
}
#define USW_LDS_POISON(buf)                                        \
  do {                                                             \
    ::usw_dev::lds_poison_all((void*)(buf), sizeof(buf));          \
    __syncthreads();                                               \
  } while (0)
#else
#define USW_LDS_POISON(buf) \
  do {                      \
  } while (0)
#endif

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

// Maximum over the 64 lanes (DPP), returned in every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false)));
  return __builtin_amdgcn_readlane(v, 63);
}

// v_perm_b32 byte selectors that expand the packed fp16 values of one 4-bit
// nibble of a BitmapTile row into 4 slots (two output dwords, j = 0, 1).
// Packed value k of the window occupies bytes 2k, 2k+1 (window dword 0 =
// selector bytes 0-3, dword 1 = bytes 4-7); a clear bit selects 0x0C, which
// v_perm turns into 0x00.  16 entries of 8 bytes: the table's 32 dwords sit
// in distinct LDS banks, so any pattern of lookups is conflict-free.
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

// v_perm selectors that expand the packed nibbles of an 8-nibble window into
// the 8 slots of a BitmapTile row with mask byte b: slot p takes nibble
// k = (set bits of b below p) when bit p is set, else zero.  Nibble k sits in
// byte k/2 of lo4 (k even) or of hi4 (k odd), as lds_window_i4 splits a
// window, and v_perm(hi4, lo4, sel) numbers lo4's bytes 0-3 and hi4's bytes
// 4-7.  .x serves slots 0-3, .y slots 4-7; a table of all 256 mask bytes
// lives in LDS.
__device__ __forceinline__ u32x2_t row_byte_selectors(uint32_t b) {
  u32x2_t sel = {0u, 0u};
  for (int p = 0; p < 8; ++p) {
    uint32_t v = 0x0Cu;
    if ((b >> p) & 1u) {
      const uint32_t k = __builtin_popcount(b & ((1u << p) - 1u));
      v = (k & 1u) ? 4u + (k >> 1) : (k >> 1);
    }
    if (p < 4)
      sel.x |= v << (8 * p);
    else
      sel.y |= v << (8 * (p - 4));
  }
  return sel;
}

// Two dwords holding packed fp16 values e, e+1, e+2, e+3 of an LDS buffer
// (element e starts at byte 2e; the buffer is dword aligned).  v_alignbyte
// uses only the low two bits of its shift operand.
__device__ __forceinline__ u32x2_t lds_window_f16(const uint8_t* buf, uint32_t e) {
  const uint32_t ba = 2u * e;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(buf + (ba & ~3u));
  const uint32_t d0 = p[0], d1 = p[1], d2 = p[2];
  u32x2_t w;
  w.x = __builtin_amdgcn_alignbyte(d1, d0, ba);
  w.y = __builtin_amdgcn_alignbyte(d2, d1, ba);
  return w;
}

// 8 packed nibbles starting at nibble e of an LDS buffer, split into the
// even (lo4) and odd (hi4) nibbles, one per byte, each in the upper half of
// its byte.  v_alignbit uses only the low five bits of its shift operand,
// here 4 * (e mod 8).
__device__ __forceinline__ u32x2_t lds_window_i4(const uint8_t* buf, uint32_t e) {
  const uint32_t ba = e >> 1;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(buf + (ba & ~3u));
  const uint32_t win = __builtin_amdgcn_alignbit(p[1], p[0], e << 2);
  u32x2_t r;
  r.x = (win << 4) & 0xF0F0F0F0u;
  r.y = win & 0xF0F0F0F0u;
  return r;
}

// 8 packed 2-bit codes starting at code e of an LDS buffer, split into the
// even (lo4) and odd (hi4) codes, one per byte in the byte's top two bits,
// where expand_row_i4 reads them as the top of a nibble: a code c becomes
// the slot 4c + 72 (the row is 4 times the codes, plus the offset; the
// kernels scale the sum by 1/4).  v_alignbit uses only the low five bits of
// its shift operand, here 2 * (e mod 16).
__device__ __forceinline__ u32x2_t lds_window_i2(const uint8_t* buf, uint32_t e) {
  const uint32_t ba = e >> 2;
  const uint32_t* p = reinterpret_cast<const uint32_t*>(buf + (ba & ~3u));
  uint32_t t = __builtin_amdgcn_alignbit(p[1], p[0], e << 1) & 0xFFFFu;
  t = (t | (t << 8)) & 0x00FF00FFu;   // codes 0-3 in byte 0, 4-7 in byte 2
  t = (t | (t << 4)) & 0x0F0F0F0Fu;   // two codes per byte
  t = (t | (t << 2)) & 0x33333333u;   // code k in bits 0-1 of nibble k
  u32x2_t r;
  r.x = (t << 6) & 0xC0C0C0C0u;
  r.y = (t << 2) & 0xC0C0C0C0u;
  return r;
}

// Offset of the code rows expand_row_i4 returns: a slot holds code + 72.
constexpr float kCodeOffset = 72.0f;

// The 8 fp16 slots of a code row, each holding its code plus kCodeOffset
// (empty slots kCodeOffset; 2-bit rows four times the code plus
// kCodeOffset), from its 8-nibble window (split into lo4 / hi4, nibbles in
// the upper half of each byte, by lds_window_i4 / _i2) and its selectors.
// The offset keeps the expansion to byte permutes: the kernels take it out
// with code_offset_collect, once per X^T fragment.
__device__ __forceinline__ half8_t expand_row_i4(u32x2_t w8, u32x2_t sel) {
  // Slots as bytes, the nibble in the upper half; xor 0x80 maps the
  // two's-complement nibble q to u = q + 8 in [0, 15] (an empty slot's 0
  // becomes 8, i.e. q = 0).
  const uint32_t e0 = __builtin_amdgcn_perm(w8.y, w8.x, sel.x) ^ 0x80808080u;
  const uint32_t e1 = __builtin_amdgcn_perm(w8.y, w8.x, sel.y) ^ 0x80808080u;
  // fp16 bit pattern 0x5400 | (u << 4) is 64 (1 + u / 64) = 64 + u exactly,
  // i.e. q + 72.
  u32x4_t a;
  a.x = __builtin_amdgcn_perm(0x54545454u, e0, 0x04010400u);
  a.y = __builtin_amdgcn_perm(0x54545454u, e0, 0x04030402u);
  a.z = __builtin_amdgcn_perm(0x54545454u, e1, 0x04010400u);
  a.w = __builtin_amdgcn_perm(0x54545454u, e1, 0x04030402u);
  return __builtin_bit_cast(half8_t, a);
}

// Takes the expansion's offset out of a tile: every slot of a rebuilt
// fragment carries kCodeOffset, so fragment A times X^T fragment x exceeds
// the true product by kCodeOffset times x's column sums, the same for every
// row.  corr[nb] collects -kCodeOffset times those sums; code_offset_finish
// puts them in the accumulator layout, and the kernel adds them to every row block's
// accumulators before the reduction.  With one token block the sums come
// from one MFMA with a constant A per X^T fragment (the matrix cores are
// mostly idle in decode); with two, from v_dot2 on the vector ALUs (the
// MFMA form measured slower there), each lane summing its 8 k of its token
// in corr[nb].x.  With integer-valued inputs every product and partial sum
// is an integer, exact while its magnitude stays below 2^24.
template <int NB>
__device__ __forceinline__ void code_offset_collect(f32x4_t (&corr)[NB], const u32x4_t (&x)[2][NB]) {
  const _Float16 m = static_cast<_Float16>(-kCodeOffset);
  if constexpr (NB == 1) {
    const half8_t neg = {m, m, m, m, m, m, m, m};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      corr[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(neg, __builtin_bit_cast(half8_t, x[ks][0]), corr[0], 0, 0, 0);
  } else {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    const half2_t neg2 = {m, m};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // Through a scalar: bit-casting the vector element itself made
          // the compiler take element 0 for every d.
          const uint32_t pair = x[ks][nb][d];
          corr[nb].x = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pair), neg2, corr[nb].x, false);
        }
  }
}

// The collected corrections in the MFMA D layout (lane l: token l % 16 of
// its block, four rows): with v_dot2 the four lanes of a token (l % 16
// equal) add their partial sums.
template <int NB>
__device__ __forceinline__ void code_offset_finish(f32x4_t (&corr)[NB]) {
  if constexpr (NB > 1) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float t = corr[nb].x;
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
      corr[nb] = f32x4_t{t, t, t, t};
    }
  }
}

// The 8 dense fp16 slots (one BitmapTile row) of a lane's A fragment: the
// row's kept values start at element rb of the LDS buffer; `byte` is the
// row's mask.
//  * fp16: slots 0-3 come from a window at rb, slots 4-7 from a window at
//    rb + popcount(low nibble), with selectors from a 16-entry table (two
//    dwords per nibble) indexed by each half of the mask.
//  * INT4: a row's at most 8 values are the 8 nibbles from rb on, so one
//    window holds them all; selectors from the 256-entry table of
//    row_byte_selectors indexed by the whole mask.
template <bool I4>
__device__ __forceinline__ half8_t rebuild_row(const uint8_t* vb, const uint32_t* lut, uint32_t rb, uint32_t byte) {
  if constexpr (!I4) {
    const uint32_t pcl = __builtin_popcount(byte & 0xFu);
    const u32x2_t slo = reinterpret_cast<const u32x2_t*>(lut)[byte & 0xFu];
    const u32x2_t shi = reinterpret_cast<const u32x2_t*>(lut)[byte >> 4];
    const u32x2_t lo = lds_window_f16(vb, rb);
    const u32x2_t hi = lds_window_f16(vb, rb + pcl);
    u32x4_t a;
    a.x = __builtin_amdgcn_perm(lo.y, lo.x, slo.x);
    a.y = __builtin_amdgcn_perm(lo.y, lo.x, slo.y);
    a.z = __builtin_amdgcn_perm(hi.y, hi.x, shi.x);
    a.w = __builtin_amdgcn_perm(hi.y, hi.x, shi.y);
    return __builtin_bit_cast(half8_t, a);
  } else {
    return expand_row_i4(lds_window_i4(vb, rb), reinterpret_cast<const u32x2_t*>(lut)[byte]);
  }
}

// Packed-code payloads of BITS = 4 or 2 bits per element: the 16-byte chunk
// arithmetic of chunk_start / chunk_delta / chunk_count below, and the
// 8-element window of a row.
template <int BITS>
struct Packed {
  static_assert(BITS == 4 || BITS == 2, "4- or 2-bit codes");
  static constexpr uint32_t kPerByte = 8 / BITS;
  static constexpr int kShift = BITS == 4 ? 1 : 2;   // log2(kPerByte)
  // Byte offset of the 16-byte chunk holding element e.
  __device__ static uint64_t chunk_start(uint32_t e) { return (static_cast<uint64_t>(e) >> kShift) & ~15ull; }
  // Elements of the first chunk that precede element e.
  __device__ static uint32_t chunk_delta(uint32_t e, uint64_t a0) {
    return static_cast<uint32_t>(e - kPerByte * a0);
  }
  // 16-byte chunks spanned by elements [e0, e1) counted from a0.
  __device__ static uint32_t chunk_count(uint32_t e1, uint64_t a0) {
    const uint64_t end = (static_cast<uint64_t>(e1) + kPerByte - 1) >> kShift;
    return static_cast<uint32_t>((end - a0 + 15ull) >> 4);
  }
  __device__ static u32x2_t window(const uint8_t* buf, uint32_t e) {
    if constexpr (BITS == 4)
      return lds_window_i4(buf, e);
    else
      return lds_window_i2(buf, e);
  }
  // What a row's expanded slots count each code as (window above): the
  // corrected sums are multiplied by this, exactly.
  static constexpr float kSumScale = BITS == 4 ? 1.0f : 0.25f;
};

// Byte offset of the 16-byte chunk holding value element e (fp16: 2 B per
// element; INT4: 4 bits per element).
template <bool I4>
__device__ __forceinline__ uint64_t chunk_start(uint32_t e) {
  return I4 ? ((static_cast<uint64_t>(e) >> 1) & ~15ull) : ((2ull * e) & ~15ull);
}

// Elements of the first chunk that precede element e.
template <bool I4>
__device__ __forceinline__ uint32_t chunk_delta(uint32_t e, uint64_t a0) {
  return I4 ? static_cast<uint32_t>(e - 2 * a0) : static_cast<uint32_t>((2ull * e - a0) >> 1);
}

// 16-byte chunks spanned by elements [e0, e1) counted from a0.
template <bool I4>
__device__ __forceinline__ uint32_t chunk_count(uint32_t e1, uint64_t a0) {
  const uint64_t end = I4 ? ((static_cast<uint64_t>(e1) + 1) >> 1) : 2ull * e1;   // first byte past the values
  return static_cast<uint32_t>((end - a0 + 15ull) >> 4);
}

}  // namespace usw_dev
