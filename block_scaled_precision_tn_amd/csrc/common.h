// common.h -- device-side building blocks shared by the gfx950 GEMM kernels.
//
// MFMA fragment layouts used throughout (CDNA3/CDNA4 32x32 family, wave64):
//   operand (A or B) of v_mfma_f32_32x32x16_{bf16,fp8_fp8}: lane l holds row
//     (l % 32) of the 32-row slab, K-elements 8*(l/32) .. 8*(l/32)+7.
//   operand of v_mfma_scale_f32_32x32x64_f8f6f4 (8-bit formats): lane l holds
//     row (l % 32); its bytes 0..15 are K-elements 16*(l/32) .. +15 and its
//     bytes 16..31 are K-elements 32 + 16*(l/32) .. +15.  Scale block 0
//     (K 0..31) takes its E8M0 byte from lane (l % 32), block 1 (K 32..63)
//     from lane 32 + (l % 32).  (Measured on gfx950 with a one-byte probe.)
//   accumulator (16 floats): lane l holds column (l % 32); register r holds
//     row 8*(r/4) + 4*(l/32) + (r%4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x32 __attribute__((ext_vector_type(32)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace mg {

__device__ __forceinline__ f32x16 mfma_fp8(uint64_t a, uint64_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8((long)a, (long)b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// E8M0-scaled MFMA on E4M3 operands (format code 0 for both sides)
__device__ __forceinline__ f32x16 mfma_mx_fp8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// E2M1 -> E4M3 by bit operations (metrale_circuit hardware::exec module
// description): a code whose sign sits in bit 7 and magnitude in bits 6..4 of
// a byte becomes the E4M3 byte of value x 2^-6 by keeping the sign and moving
// the magnitude down two places.  `w` holds 8 packed NVFP4 codes (byte i: low
// nibble element 2i, high nibble element 2i+1).  Returns the 8 E4M3 bytes in
// lane-local order [e0 e2 e4 e6 | e1 e3 e5 e7]; the matching operand of the
// same MFMA must use the same order (a K-permutation inside one lane's slice
// leaves every dot product unchanged).
__device__ __forceinline__ uint64_t nvfp4x8_to_e4m3x8(uint32_t w) {
  uint32_t odd = (w & 0x80808080u) | ((w >> 2) & 0x1C1C1C1Cu);
  uint32_t even = ((w << 4) & 0x80808080u) | ((w << 2) & 0x1C1C1C1Cu);
  return (uint64_t)even | ((uint64_t)odd << 32);
}

// The same lane-local order applied to 8 E4M3 bytes already in natural order
// (activations of the W4A8 route): [b0 b2 b4 b6 | b1 b3 b5 b7].
__device__ __forceinline__ uint64_t e4m3x8_even_odd(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  uint32_t even = __builtin_amdgcn_perm(hi, lo, 0x06040200u);
  uint32_t odd = __builtin_amdgcn_perm(hi, lo, 0x07050301u);
  return (uint64_t)even | ((uint64_t)odd << 32);
}

// E4M3-FN byte -> BF16 bits of (its value x 64).  Exact: an E4M3 value has at
// most 4 significant bits.  NaN bytes give a NaN.
__device__ __forceinline__ uint32_t e4m3_x64_to_bf16(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const uint32_t normal = ((e + 126u) << 7) | (m << 4);                      // 2^(e-7) * 64
  const uint32_t sub = __builtin_bit_cast(uint32_t, (float)m * 0.125f) >> 16;  // m/8 * 2^-6 * 64
  uint32_t bits = e != 0u ? normal : sub;
  bits = (e == 15u && m == 7u) ? 0x7FC0u : bits;
  return ((b & 0x80u) << 8) | bits;
}

// E4M3-FN byte -> FP32 value (exact)
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float normal = __builtin_bit_cast(float, ((e + 120u) << 23) | (m << 20));
  const float sub = (float)m * 0.001953125f;  // m * 2^-9
  float v = e != 0u ? normal : sub;
  v = (e == 15u && m == 7u) ? __builtin_nanf("") : v;
  return (b & 0x80u) ? -v : v;
}

// E4M3-FN byte -> FP32 value x 64, in three integer/float operations: the
// byte's exponent and mantissa fields placed in an FP32 pattern give
// 2^(e-127)(1+m/8) for e >= 1 and, as an FP32 subnormal, m * 2^-129 for
// e == 0; one multiply by 2^126 rescales both cases to 64 * value exactly.
// (NaN bytes are not special-cased.)
__device__ __forceinline__ float e4m3_x64_to_f32(uint32_t b) {
  const float f = __builtin_bit_cast(float, ((b & 0x7Fu) << 20) | ((b & 0x80u) << 24));
  return f * 8.5070591730234616e+37f;  // 2^126
}

// The same with the E4M3 NaN bytes (0x7F, 0xFF) mapped to a NaN.
__device__ __forceinline__ float e4m3_x64_to_f32_nan(uint32_t b) {
  const float v = e4m3_x64_to_f32(b);
  return (b & 0x7Fu) == 0x7Fu ? __builtin_nanf("") : v;
}

// FP32 -> BF16 bits, round to nearest even (NaN stays NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u | ((u >> 16) & 0x8000u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Tile of a 1-D launch of T = tiles_m * tiles_n workgroups, chosen for L2 reuse
// on a chip whose XCDs (each with its own L2) receive workgroups round-robin
// (workgroup id i runs on XCD i % 8): each XCD gets one contiguous run of the
// tile order, and that order walks groups of 8 tile rows column by column, so
// the workgroups running together on an XCD share A row panels and W column
// panels.
__device__ __forceinline__ void xcd_tile(int id, int tiles_m, int tiles_n, int &tm, int &tn) {
  constexpr int XCDS = 8, GROUP = 8;
  const int T = tiles_m * tiles_n, q = T / XCDS, r = T % XCDS;
  const int x = id % XCDS, j = id / XCDS;
  const int t = x < r ? x * (q + 1) + j : r * (q + 1) + (x - r) * q + j;
  const int per_group = GROUP * tiles_n, first = (t / per_group) * GROUP;
  const int gsz = tiles_m - first < GROUP ? tiles_m - first : GROUP;
  tm = first + (t % per_group) % gsz;
  tn = (t % per_group) / gsz;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) at maximum).
// A workgroup barrier written as __syncthreads() carries a memory fence that
// waits for every outstanding global load; kernels that keep loads in flight
// across a barrier use these waits with __builtin_amdgcn_s_barrier() instead.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) only
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(63 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Direct-to-LDS loads (global_load_lds): lane i's bytes land at
// lds + size * i (sizes below 4 fill one dword per lane, zero-extended).
// Written as inline assembly so the compiler does not track them: for the
// builtin form it cannot always tell which LDS buffer a load fills and then
// makes every LDS read wait for all loads in flight.  Kernels wait for these
// loads with explicit vmcnt counts (loads complete in issue order).
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ uint32_t lds_addr(const void *lds) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const lds_void *)lds);
}
__device__ __forceinline__ void dma16(const void *g, const void *lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(lds_addr(lds))
               : "memory", "m0");
}
// the same load addressed as a uniform 64-bit base plus a 32-bit per-lane
// byte offset: the offsets of a tile's rows stay fixed from stage to stage
// (only the base moves along K), so they cost one register each
// (lds: the LDS byte address, uniform)
__device__ __forceinline__ void dma16_s(uint32_t off, const void *base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off),
               "s"(base), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma2(const void *g, const void *lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_ushort %0, off" ::"v"(g),
               "s"(lds_addr(lds))
               : "memory", "m0");
}

// row held by accumulator register r of lane l (see the layout note above)
__device__ __forceinline__ int acc_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

}  // namespace mg
