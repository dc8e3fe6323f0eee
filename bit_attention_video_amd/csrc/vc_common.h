// Device helpers shared by the VC-Attention kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define VC_D 128
#define VC_BLK 128

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v6i __attribute__((ext_vector_type(6)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// Streaming loads for data a kernel reads once (the bf16 K and V rows of the preprocessing passes):
// nontemporal, so the lines are not kept in the caches for reuse that never comes.  On MI355X a
// read-only stream of this form sustains about 6 TB/s against about 5.4 TB/s for plain loads.
__device__ __forceinline__ uint2 ld_stream2(const void* p) {
  typedef unsigned int v2u __attribute__((ext_vector_type(2)));
  const v2u v = __builtin_nontemporal_load((const v2u*)p);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld_stream4(const void* p) {
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load((const v4u*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 bit pattern -> float32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// E4M3 (OCP E4M3FN) codes of two float32 values, round to nearest even, saturating to
// +-448: the hardware conversion rounds to nearest even and has no saturation, so the
// operands are clamped first (|x| <= 448 keeps every finite input in range).
// Returns the two codes in bits [0,16) of the result (x0 in byte 0).
__device__ __forceinline__ uint32_t e4m3x2(float x0, float x1) {
  x0 = fminf(fmaxf(x0, -448.0f), 448.0f);
  x1 = fminf(fmaxf(x1, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false) & 0xFFFFu;
}

// Four E4M3 codes packed little-endian (x0 in byte 0).
__device__ __forceinline__ uint32_t e4m3x4(float x0, float x1, float x2, float x3) {
  x0 = fminf(fmaxf(x0, -448.0f), 448.0f);
  x1 = fminf(fmaxf(x1, -448.0f), 448.0f);
  x2 = fminf(fmaxf(x2, -448.0f), 448.0f);
  x3 = fminf(fmaxf(x3, -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}

// ExpCast rounding and clip (Eq. 7): byte `sel` of `old` <- clamp(RNE(t), 0, 255).
// v_cvt_pk_u8_f32 rounds to nearest even and saturates to [0, 255] (NaN -> 0); the
// callers guarantee t <= 120.5 or clip the integer to 120 themselves.
__device__ __forceinline__ uint32_t expcast_byte(float t, uint32_t sel, uint32_t old) {
  return __builtin_amdgcn_cvt_pk_u8_f32(t, sel, old);
}

// Exponent E of the smallest power of two 2^E with amax <= 448 * 2^E (0 when amax == 0,
// never below -100 so 2^E and 2^-E stay normal floats): with amax = m 2^e, m in [0.5, 1),
// 448 * 2^(e-8) always fits and 448 * 2^(e-10) never does.  The Q/K block scales are these
// powers of two, i.e. E8M0 values the FP8 matrix instructions apply themselves.
__device__ __forceinline__ int pow2_block_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  (void)__builtin_frexpf(amax, &e);
  int E = e - 8;
  if (amax <= __builtin_ldexpf(448.0f, E - 1)) E -= 1;
  return E < -100 ? -100 : E;
}

// E2M1 (OCP MX FP4) codes of x0 and x1, which the caller has already divided by their power-
// of-two group scale (|x| <= 6), written into byte SEL of `old` with x0 in the low nibble: the
// hardware round-to-nearest-even conversion, applied with unit scale.
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2(uint32_t old, float x0, float x1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, x0, x1, 1.0f, SEL);
}

// Exponent E of an MX (E8M0) group scale: the smallest power of two 2^E with amax <= 6 * 2^E,
// 6 being E2M1's largest magnitude (0 when amax == 0, never below -100).  With
// amax = m 2^e, m in [0.5, 1): 6 * 2^(e-3) = 0.75 * 2^e fits iff m <= 0.75, and
// 6 * 2^(e-4) < 2^(e-1) <= amax never does.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  const float m = __builtin_frexpf(amax, &e);
  const int E = m <= 0.75f ? e - 3 : e - 2;
  return E < -100 ? -100 : E;
}

// E2M3 (OCP MX FP6) codes of the 32 values x[0..31], which the caller has already divided by
// their power-of-two group scale (|x| <= 7.5): the hardware round-to-nearest-even conversion
// with unit scale into six dwords, value k in bits 6k .. 6k + 5 of the 192 bits.  The
// instruction interleaves its two 16-value operands (field 2i from the first, 2i + 1 from the
// second; a layout probe on the device showed it), so the even values go in the first.
__device__ __forceinline__ v6i fp6x32(const float* x) {
  v16f lo, hi;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    lo[k] = x[2 * k];
    hi[k] = x[2 * k + 1];
  }
  return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, 1.0f);
}

// Exponent E of an MX group scale for E2M3 elements: the smallest power of two 2^E with
// amax <= 7.5 * 2^E (0 when amax == 0, never below -100).  With amax = m 2^e, m in [0.5, 1):
// 7.5 * 2^(e-3) = 0.9375 * 2^e fits iff m <= 0.9375, and 7.5 * 2^(e-4) < 2^(e-1) never does.
__device__ __forceinline__ int mx6_exponent(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  const float m = __builtin_frexpf(amax, &e);
  const int E = m <= 0.9375f ? e - 3 : e - 2;
  return E < -100 ? -100 : E;
}

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Block -> logical work item, XCD-aware: the hardware hands workgroup b to XCD b % 8, so
// XCD x receives every 8th workgroup.  Remap so XCD x walks one contiguous range of the
// logical order instead, so the CUs sharing one L2 work on neighbouring items at once.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t G) {
  const uint32_t X = 8;
  uint32_t x = b % X, i = b / X;
  uint32_t q = G / X, r = G % X;
  uint32_t start = x * q + (x < r ? x : r);
  return start + i;
}
