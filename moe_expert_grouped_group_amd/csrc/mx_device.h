// Device helpers shared by the MXFP8 kernels (gfx950).
//
// MXFP8 block rule (OCP Microscaling Formats v1.0, section 6.3; E4M3 and
// E8M0 encodings from its section 5): a block of 32 values takes the shared
// exponent X = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest value),
// clamped to [-127, 127], stored as the E8M0 byte X + 127; each element is the
// E4M3 value nearest to v / 2^X (ties to even), saturated to +-448.
//
// For a bf16 amax with biased exponent field e (0..254), floor(log2 amax) is
// e - 127 for e >= 1, so the scale byte is max(e - 8, 0): every quantity the
// kernels need is an integer operation on bit fields.  The element encoder
// below rounds with integer arithmetic on the fp32 bit pattern, which is exact
// by construction (no dependence on the hardware converter's rounding or
// overflow behaviour).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

constexpr int kBlock = 32;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// E8M0 scale byte from the biased exponent field of the block's amax.
__device__ __forceinline__ uint32_t scale_byte_from_exp(uint32_t amax_exp) {
  return amax_exp > 8u ? amax_exp - 8u : 0u;
}

// 2^-X as an fp32, for X = byte - 127 (byte in 0..254): bits (254 - byte) << 23.
// Valid for byte <= 253 (X <= 126); bf16 inputs give byte <= 246.
__device__ __forceinline__ float inv_scale_from_byte(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

// Encode an fp32 y that is exactly v / 2^X (|y| < 512) as an E4M3 byte:
// round to nearest even, saturate to 448, keep the sign (also of zero).
//  - |y| >= 2^-6: normal E4M3.  With fp32 exponent field E32 the E4M3
//    exponent field is E32 - 120; subtracting 120 << 23 leaves
//    (E4 << 23 | mantissa23); rounding the low 20 bits to nearest even
//    (carry may bump the exponent) and shifting gives (E4 << 3 | m3).
//    Codes above 0x7E (480, NaN slot, or an exponent overflow) become 0x7E.
//  - |y| < 2^-6: subnormal E4M3, code = rint(|y| * 2^9) in 0..8 (8 is the
//    smallest normal 0x08); the multiply is exact and rint is ties-to-even.
__device__ __forceinline__ uint32_t encode_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t t = a - (120u << 23);
  t = t + 0x7FFFFu + ((t >> 20) & 1u);
  uint32_t code_n = t >> 20;
  code_n = code_n < 0x7Eu ? code_n : 0x7Eu;
  const uint32_t code_s = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  const uint32_t code = a >= 0x3C800000u ? code_n : code_s;
  return sign | code;
}

// E4M3 byte -> fp32 value (exact), NaN codes not expected.
__device__ __forceinline__ float decode_e4m3(uint32_t c) {
  const uint32_t mag = c & 0x7Fu;
  // normal: exponent field e4 -> fp32 exponent e4 + 120, mantissa m3 << 20
  const uint32_t nbits = (mag << 20) + (120u << 23);
  const float sub = (float)mag * 0.001953125f;  // m * 2^-9 for e4 == 0 (mag < 8)
  float v = mag >= 8u ? __uint_as_float(nbits) : sub;
  return (c & 0x80u) ? -v : v;
}

// floor(log2(|value|)) of a non-zero E4M3 magnitude code (1..126), as an int:
// normal e4 - 7; subnormal floor(log2(m)) - 9.
__device__ __forceinline__ int e4m3_floor_log2(uint32_t mag) {
  return mag >= 8u ? (int)(mag >> 3) - 7 : (31 - __builtin_clz(mag)) - 9;
}

// Pack four bytes (low 8 bits of each) into a u32, byte 0 = a.
__device__ __forceinline__ uint32_t pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return a | (b << 8) | (c << 16) | (d << 24);
}

}  // namespace mx
