// quant.h -- FP32 -> narrow-format encoders for the in-kernel re-quantisation
// of the MoE's h (MXFP8 and NVFP4), nearest even, saturating.
#pragma once
#include "common.h"

namespace mg {

// FP32 -> E4M3-FN byte, nearest even, saturating at +-448 (NaN -> 0x7F).
// Written with selects only, so that a wave converting many values runs
// them back to back: below 2^-6 the code is the value in steps of 2^-9
// (8 is the smallest normal, code 0x08); above, the FP32 bits rounded to 3
// mantissa bits with the exponent rebased.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t au = u & 0x7FFFFFFFu;
  const float a = __builtin_bit_cast(float, au);
  const uint32_t sub = (uint32_t)__builtin_rintf(fminf(a, 0.015625f) * 512.0f);
  const uint32_t nrm = ((au + 0x7FFFFu + ((au >> 20) & 1u)) >> 20) - (120u << 3);
  uint32_t c = a < 0.015625f ? sub : nrm;
  c = a < 448.0f ? c : 0x7Eu;
  return au > 0x7F800000u ? 0x7Fu : (sign | c);
}

// Two values at once on gfx950's converter (v_cvt_scalef32_pk_fp8_f32 at
// scale 1): it rounds to nearest even like f32_to_e4m3_rne_sat but does not
// saturate (at 464 and above it gives the NaN code) and gives NaN the sign
// bit, so the inputs are clamped to +-448 first and NaN is mapped to 0x7F.
// The result equals f32_to_e4m3_rne_sat on both values (a device sweep of
// every FP32 pattern with |v| in [2^-30, 2^34) of both signs, plus zeros,
// infinities, NaNs and tiny values, found no difference).  Codes of a and b
// in bits 0..7 and 8..15.
typedef short mg_v2i16 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_e4m3_rne_sat(float a, float b) {
  const float ca = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  const float cb = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  mg_v2i16 o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, ca, cb, 1.0f, false);
  const uint32_t lo = a != a ? 0x7Fu : (uint32_t)(uint16_t)o[0] & 0xFFu;
  const uint32_t hi = b != b ? 0x7Fu : ((uint32_t)(uint16_t)o[0] >> 8) & 0xFFu;
  return lo | (hi << 8);
}

// FP32 -> E2M1 code (sign in bit 3): the nearest of the magnitudes {0, .5, 1,
// 1.5, 2, 3, 4, 6}, a tie going to the code with a zero low bit, magnitudes
// above 6 giving 6; NaN gives 0
__device__ __forceinline__ uint32_t f32_to_e2m1_rne_sat(float v) {
  if (v != v) return 0u;
  const float a = fabsf(v);
  const uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                   : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return c | ((__builtin_bit_cast(uint32_t, v) >> 28) & 8u);
}

}  // namespace mg
