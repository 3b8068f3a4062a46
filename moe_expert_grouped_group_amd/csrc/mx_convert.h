// gfx950 scaled FP8 conversions (E4M3 elements with an E8M0 scale) used by
// the streaming quantize kernels.
//
// The scale operand is an fp32 whose exponent field is read as the E8M0 byte,
// so byte << 23 passes 2^(byte - 127) (byte 0 passes 2^-127).  Behaviour, as
// established by an exhaustive sweep of every (value, scale) pair against the
// integer encoder of mx_device.h (mxfp8_convert_sweep repeats that sweep on
// the device it runs on):
//  * decode: code * 2^X, exact for every code and X <= 119 (fp32 denormals
//    included); X >= 120 can overflow to infinity.
//  * encode: the E4M3 value nearest to v / 2^X, ties to even, sign of zero
//    kept, fp32 denormal inputs handled exactly; a quotient that rounds above
//    448 yields the NaN code 0x7F instead of saturating, so every encoded
//    word passes through sat_e4m3x4.
#pragma once

#include "mx_device.h"

namespace mx {


typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float e8m0_operand(uint32_t byte) { return __uint_as_float(byte << 23); }

// Four E4M3 codes in a u32: each byte whose low 7 bits are all ones (the NaN
// code, produced only by an overflowing conversion) becomes 0x7E / 0xFE, the
// largest finite magnitude with the same sign.  The +1 cannot carry out of a
// byte because the low 7 bits are at most 0x7F.
__device__ __forceinline__ uint32_t sat_e4m3x4(uint32_t w) {
  const uint32_t nan = (((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) >> 7;
  return w - nan;
}

// Four bf16 values (two packed pairs, element 0 in the low half of `lo`) ->
// four saturated E4M3 codes of v / 2^X, byte i = element i.
__device__ __forceinline__ uint32_t cvt4_bf16_e4m3(uint32_t lo, uint32_t hi, float scale) {
  i16x2_t r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, lo), scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, hi), scale, true);
  return sat_e4m3x4(__builtin_bit_cast(uint32_t, r));
}

// Four fp32 values -> four saturated E4M3 codes of v / 2^X, byte i = element i.
__device__ __forceinline__ uint32_t cvt4_f32_e4m3(float a, float b, float c, float d,
                                                  float scale) {
  i16x2_t r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, a, b, scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, scale, true);
  return sat_e4m3x4(__builtin_bit_cast(uint32_t, r));
}

// The two E4M3 codes in bytes 0 and 1 of `src` -> code * 2^X as fp32.
__device__ __forceinline__ f32x2_t cvt2_e4m3_f32(uint32_t src, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(src, scale, false);
}

// Largest scale byte whose decode cannot overflow fp32 (448 * 2^119 < 2^128);
// bf16 data never produces a larger one.
constexpr uint32_t kMaxFastScaleByte = 246;

}  // namespace mx
