// codec.hpp -- device lane codecs of the packed optimizer state (gfx950).
//
// Formats (Packed AdamW Reference README, introduction; project page,
// Release scope): a 32-bit state word per parameter whose low half is a
// signed finite E4M11 first moment and whose high half is an unsigned finite
// E4M12 uncorrected RMS.  Exponent bias 15 in both lanes (a reading: the
// pages never print it), gradual underflow at exponent field 0, every
// exponent field finite.  Encoding rounds to nearest with ties to even and
// saturates at the largest finite value; NaN encodes as 0; the RMS lane maps
// any input with the sign bit set to 0.
//
// Everything here is integer work on FP32 bit patterns plus one exact FP32
// scaling, so a value costs a handful of VALU instructions:
//
//   decode: put the lane's exponent and mantissa fields in the float's
//     exponent/mantissa positions (exponent field e lands at float exponent
//     field e) and multiply by 2^112, which moves float bias 127 to lane
//     bias 15.  Exponent field 0 becomes an FP32 denormal whose product with
//     2^112 is the lane's subnormal value, exactly.
//   encode, normal range (|x| >= 2^-14): subtract 112 from the float
//     exponent, add half a lane step minus one plus the lowest kept bit
//     (round to nearest, ties to even), shift the dropped mantissa bits out.
//     A carry out of the mantissa bumps the exponent, as it should.
//   encode, subnormal range (|x| < 2^-14): add the power of two whose FP32
//     last place equals the lane's subnormal step (2^-2 for E4M11, 2^-3 for
//     E4M12); the FP32 addition performs the round-to-nearest-even, and the
//     code is the sum's bit pattern minus that power of two's.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Bit patterns of the lane limits.
constexpr uint32_t kMinNormalBits = 0x38800000u;   // 2^-14, both lanes
constexpr uint32_t kRebias = 0x38000000u;          // 112 << 23
constexpr uint32_t kMMaxBits = 0x3FFFF000u;        // 2 - 2^-11, E4M11 largest finite
constexpr uint32_t kRMaxBits = 0x3FFFF800u;        // 2 - 2^-12, E4M12 largest finite
constexpr uint32_t kInfBits = 0x7F800000u;

__device__ __forceinline__ float e4_decode_m(uint32_t word) {
  const float mag = __uint_as_float((word & 0x7FFFu) << 12) * 0x1p112f;
  return __uint_as_float(__float_as_uint(mag) | ((word & 0x8000u) << 16));
}

// The first moment's fields in place but without the 2^112 scale: the value
// times 2^-112, an FP32 denormal or small normal.  A product c * m with a
// binary32 c equals (c * 2^112) * e4_decode_m_unscaled(word) exactly, since
// c * 2^112 is exact and the product is rounded once either way.
__device__ __forceinline__ float e4_decode_m_unscaled(uint32_t word) {
  return __uint_as_float(((word & 0x7FFFu) << 12) | ((word & 0x8000u) << 16));
}

__device__ __forceinline__ float e4_decode_r(uint32_t word) {
  return __uint_as_float((word >> 16) << 11) * 0x1p112f;
}

__device__ __forceinline__ uint32_t e4_encode_m(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t mag_bits = b & 0x7FFFFFFFu;
  // |x| at or above the largest finite value (Inf too) encodes as that value.
  const uint32_t a = min(mag_bits, kMMaxBits);
  const uint32_t nrm = (a - kRebias + 0x7FFu + ((a >> 12) & 1u)) >> 12;
  const uint32_t sub = __float_as_uint(__uint_as_float(a) + 0.25f) - 0x3E800000u;
  const uint32_t mag = a < kMinNormalBits ? sub : nrm;
  const uint32_t code = mag | ((b >> 16) & 0x8000u);
  return mag_bits > kInfBits ? 0u : code;
}

__device__ __forceinline__ uint32_t e4_encode_r(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t a = min(b, kRMaxBits);
  const uint32_t nrm = (a - kRebias + 0x3FFu + ((a >> 11) & 1u)) >> 11;
  const uint32_t sub = __float_as_uint(__uint_as_float(a) + 0.125f) - 0x3E000000u;
  const uint32_t code = a < kMinNormalBits ? sub : nrm;
  return b > kInfBits ? 0u : code;   // NaN, and every input with its sign bit set
}

// IEEE binary16 lanes: the hardware conversions round to nearest even and
// overflow to Inf under the default float mode.
__device__ __forceinline__ float f16_decode(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
}

__device__ __forceinline__ uint32_t f16_encode(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// bfloat16, round to nearest even: the bit pattern plus 0x7FFF plus its own
// bit 16, shifted down (a carry out of the mantissa moves to the next binade
// and past the largest finite value to Inf; binary32 subnormals round like
// any other pattern); NaN stays a quiet NaN with the input's sign and top
// payload bits.  gfx950's conversion instruction computes exactly this with
// the FP32 denormals this library keeps; the tests compare it with the
// oracle's bfloat16 rounding on every binary32 bit pattern.
__device__ __forceinline__ uint32_t bf16_encode(float x) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

// Two values in one word, `lo` in the low half (one conversion instruction).
__device__ __forceinline__ uint32_t bf16_encode2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 v;
  v.x = lo;
  v.y = hi;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

}  // namespace pa
