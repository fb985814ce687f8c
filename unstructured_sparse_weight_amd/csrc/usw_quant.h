// fp16 <-> fp64 conversions and the b-bit (INT4, 2-bit) round-to-nearest
// quantiser, used by
// both the host encoder and the device encoder so that the two write the
// same bytes.
//
// b-bit rule (per output row m of W, over the kept weights only; INT4 is
// b = 4, the 2-bit payload b = 2, qmax = 2^(b-1) - 1): scale_m is
// max |w| / qmax computed in fp64 and rounded once to fp16; a kept weight w
// gets the code clamp(round_half_even(w / scale_m), -qmax - 1, qmax) in
// fp64, or 0 when the scale is 0 (a row with nothing kept, or only zeros
// kept).  Non-finite
// weights: a kept NaN makes the row maximum, and so the scale, NaN (fp16
// 0x7E00), and every code of that row 0; a NaN quotient (an infinite weight
// under an infinite scale) gives code 0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace usw {

// fp16 bits -> double (exact; NaN stays NaN, infinities stay infinite).  On
// the GPU the two hardware conversions fp16 -> fp32 -> fp64, each exact; on
// the host the bits are placed directly.
__host__ __device__ inline double f16_to_f64(uint16_t h) {
#if defined(__HIP_DEVICE_COMPILE__)
  return static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, h)));
#else
  const uint64_t sign = static_cast<uint64_t>(h >> 15) << 63;
  const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
  if (e == 0) {  // zero or subnormal: m units of 2^-24
    const double v = static_cast<double>(m) * 0x1p-24;
    return sign ? -v : v;
  }
  const uint64_t be = e == 31 ? 0x7FFull : static_cast<uint64_t>(e) - 15 + 1023;
  return __builtin_bit_cast(double, sign | (be << 52) | (static_cast<uint64_t>(m) << 42));
#endif
}

// double -> fp16 bits with a single round-to-nearest-even, from the IEEE
// binary16 layout (1 sign, 5 exponent bits with bias 15, 10 fraction bits;
// subnormal unit 2^-24; values at or above 65520 round to infinity).
__host__ __device__ inline uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000u);
  const int exp = static_cast<int>((b >> 52) & 0x7FF);
  const uint64_t frac = b & ((1ull << 52) - 1);
  if (exp == 0x7FF) return sign | (frac ? 0x7E00 : 0x7C00);
  if (exp == 0) return sign;  // fp64 subnormals are far below half the fp16 subnormal unit
  const int e = exp - 1023;   // x = sig * 2^(e - 52), sig in [2^52, 2^53)
  const uint64_t sig = frac | (1ull << 52);
  int shift;                  // bits of sig dropped
  if (e >= -14) {
    shift = 42;               // keep 11 significant bits
  } else {
    shift = 28 - e;           // express in units of 2^-24
    if (shift > 53) return sign;  // below 2^-25: rounds to zero
  }
  uint64_t r = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (r & 1))) ++r;
  if (e >= -14) {
    int ee = e;
    if (r == 2048) {          // carried into the next binade
      r = 1024;
      ++ee;
    }
    if (ee > 15) return sign | 0x7C00;
    return sign | static_cast<uint16_t>(((ee + 15) << 10) | (r & 0x3FF));
  }
  // subnormal result (r == 1024 is the smallest normal, encoded the same way)
  return sign | static_cast<uint16_t>(r);
}

// Row scale bits of a b-bit code (qmax = 2^(b-1) - 1) from the largest kept
// magnitude, as fp16 bits with the sign cleared (integer order is magnitude
// order, with NaN above infinity).
__host__ __device__ inline uint16_t int_scale_bits(uint16_t amax_bits, int qmax) {
  return f64_to_f16_rne(f16_to_f64(amax_bits) / static_cast<double>(qmax));
}

// b-bit code of fp16 weight w under scale s (fp64): clamp to
// [-qmax - 1, qmax] of the quotient rounded half to even.
__host__ __device__ inline int8_t int_code(uint16_t w, double s, int qmax) {
  if (!(s > 0.0)) return 0;  // zero or NaN scale
  double v = __builtin_rint(f16_to_f64(w) / s);
  if (v != v) return 0;      // inf / inf
  const double lo = -static_cast<double>(qmax) - 1.0, hi = static_cast<double>(qmax);
  v = (lo < v) ? v : lo;
  v = (v < hi) ? v : hi;
  return static_cast<int8_t>(v);
}

// INT4 (b = 4): scale max / 7, codes in [-8, 7].
__host__ __device__ inline uint16_t i4_scale_bits(uint16_t amax_bits) { return int_scale_bits(amax_bits, 7); }
__host__ __device__ inline int8_t i4_code(uint16_t w, double s) { return int_code(w, s, 7); }

}  // namespace usw
