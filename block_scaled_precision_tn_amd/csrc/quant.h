// quant.h -- FP32 -> narrow-format encoders for the in-kernel re-quantisation
// of the MoE's h (MXFP8 and NVFP4), nearest even, saturating.
#pragma once
#include "common.h"

namespace mg {

// FP32 -> E4M3-FN byte, nearest even, saturating at +-448 (NaN -> 0x7F)
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t au = u & 0x7FFFFFFFu;
  if (au > 0x7F800000u) return 0x7Fu;
  const float a = __builtin_bit_cast(float, au);
  if (!(a < 448.0f)) return sign | 0x7Eu;
  if (a < 0.015625f) {                   // below 2^-6: steps of 2^-9
    const uint32_t m = (uint32_t)__builtin_rintf(a * 512.0f);
    return sign | m;                      // m == 8 is the smallest normal, code 0x08
  }
  const uint32_t r = (au + 0x7FFFFu + ((au >> 20) & 1u)) >> 20;  // 8-bit exp | 3-bit mantissa
  return sign | (r - (120u << 3));
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
