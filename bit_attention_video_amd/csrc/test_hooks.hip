// Single-stage kernels exposed for testing: the ExpCast code (Sec. 3.3, Eq. 7), the E4M3
// quantiser, the E2M1 conversion of the 4-bit path and the E2M3 conversion of the 6-bit path, each with the exact instruction
// sequence the production kernels use; and a dense FP8 matrix-instruction loop that measures
// the attainable FP8 rate of the device the attention kernel is compared against.
#include "vc_common.h"
#include "vc_internal.h"

// c(u) = clip(RNE(fma(8, u, C)), 0, 120), C = float32(120 + beta) = float32(119.65).
// 8u is exact, so the FMA rounds once, as the Eq. 7 contract requires.  The byte comes from
// the same saturating round-to-nearest-even conversion vc_attn_fwd uses; the integer is
// clipped to 120 for u > 0 (outside the method's domain u <= 0, where t <= 119.65).
__global__ void k_test_expcast(const float* __restrict__ u, uint8_t* __restrict__ codes, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    float t = __builtin_fmaf(8.0f, u[i], 119.65f);
    uint32_t c = expcast_byte(t, 0, 0u) & 0xFFu;
    codes[i] = (uint8_t)(c > 120u ? 120u : c);
  }
}

__global__ void k_test_e4m3(const float* __restrict__ x, uint8_t* __restrict__ codes, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) codes[i] = (uint8_t)(e4m3x2(x[i], 0.0f) & 0xFFu);
}

// Words 6i .. 6i+5 = the E2M3 codes of x[32i .. 32i+31] packed as the 6-bit paths pack them,
// converted with the group's scale operand (scale[i], 1 when scale is null): the instruction
// divides by it, as the 6-bit attention's P conversion relies on.
__global__ void k_test_fp6(const float* __restrict__ x, const float* __restrict__ scale,
                           uint32_t* __restrict__ words, size_t ngroups) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < ngroups; i += stride) {
    v16f lo, hi;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      lo[k] = x[32 * i + 2 * k];
      hi[k] = x[32 * i + 2 * k + 1];
    }
    const float sc = scale ? scale[i] : 1.0f;
    const v6i w = scale ? __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, sc) : fp6x32(&x[32 * i]);
#pragma unroll
    for (int k = 0; k < 6; ++k) words[6 * i + k] = (uint32_t)w[k];
  }
}

// Byte i = E2M1 codes of the pair (x[2i], x[2i+1]) as the 4-bit quantisers pack them.
__global__ void k_test_fp4(const float* __restrict__ x, uint8_t* __restrict__ codes, size_t npair) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < npair; i += stride) codes[i] = (uint8_t)(fp4x2<0>(0u, x[2 * i], x[2 * i + 1]) & 0xFFu);
}

// Each wave issues iters x 4 independent 32x32x64 FP8 products (E8M0 scales 1), each on its
// own pseudo-random operand pair: E4M3 bytes hashed from (thread, register, product) and masked
// with 0xF7 (bit 3 cleared, so never the NaN code; magnitudes up to 240).  Data that toggles the
// multipliers like real operands do matters: constant operands draw less power and let the
// clock run higher.  One float per thread keeps the results live; 4 x 131072 FLOP per wave and
// iteration.  With clock_mhz, wave 0 of each workgroup also reads the shader-cycle counter
// (s_memtime) and the constant-rate counter (s_memrealtime, wall_mhz ticks per microsecond)
// around its loop and writes the shader clock they imply.
__global__ __launch_bounds__(512) void k_test_mfma_fp8_rate(float* __restrict__ out, int iters,
                                                            float* __restrict__ clock_mhz, float wall_mhz) {
  const uint32_t t = threadIdx.x + 512u * blockIdx.x;
  v8i a0, a1, a2, a3, b0, b1, b2, b3;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    auto h = [&](uint32_t i) { return (int)(((t * 2654435761u) ^ (k * 40503u + 1u) * 2246822519u ^ i * 3266489917u) & 0xF7F7F7F7u); };
    a0[k] = h(1); a1[k] = h(2); a2[k] = h(3); a3[k] = h(4);
    b0[k] = h(5); b1[k] = h(6); b2[k] = h(7); b3[k] = h(8);
  }
  uint64_t c_beg = 0, w_beg = 0;
  if (clock_mhz) {
    w_beg = wall_clock64();
    c_beg = clock64();
  }
  // the operands reach the loop only through this fence, so no product starts before the stamps
  asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3));
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a2, b2, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a3, b3, c3, 0, 0, 0, 127, 0, 127);
  }
  float r = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  if (clock_mhz) {
    asm volatile("" ::"v"(r));   // every product has completed before the end stamps
    const uint64_t c_end = clock64(), w_end = wall_clock64();
    if (threadIdx.x == 0)
      clock_mhz[blockIdx.x] =
          w_end > w_beg ? (float)((double)(c_end - c_beg) / (double)(w_end - w_beg) * (double)wall_mhz) : 0.0f;
  }
  out[t] = r;
}

static unsigned grid_for(size_t n) {
  size_t g = (n + 255) / 256;
  return (unsigned)(g > 65536 ? 65536 : g);
}

hipError_t vc_launch_test_expcast(const float* u, uint8_t* codes, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_test_expcast, dim3(grid_for(n)), dim3(256), 0, s, u, codes, n);
  return hipGetLastError();
}

hipError_t vc_launch_test_e4m3(const float* x, uint8_t* codes, size_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_test_e4m3, dim3(grid_for(n)), dim3(256), 0, s, x, codes, n);
  return hipGetLastError();
}

hipError_t vc_launch_test_fp6(const float* x, const float* scale, uint32_t* words, size_t ngroups, hipStream_t s) {
  hipLaunchKernelGGL(k_test_fp6, dim3(grid_for(ngroups)), dim3(256), 0, s, x, scale, words, ngroups);
  return hipGetLastError();
}

hipError_t vc_launch_test_fp4(const float* x, uint8_t* codes, size_t npair, hipStream_t s) {
  hipLaunchKernelGGL(k_test_fp4, dim3(grid_for(npair)), dim3(256), 0, s, x, codes, npair);
  return hipGetLastError();
}

hipError_t vc_launch_test_mfma_fp8_rate(float* out, int workgroups, int iters, float* clock_mhz,
                                        hipStream_t s) {
  float wall_mhz = 0.0f;
  if (clock_mhz) {   // the constant-rate counter's frequency (kHz)
    int dev = 0, khz = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e != hipSuccess) return e;
    if (khz <= 0) return hipErrorInvalidValue;
    wall_mhz = (float)khz * 1e-3f;
  }
  hipLaunchKernelGGL(k_test_mfma_fp8_rate, dim3(workgroups), dim3(512), 0, s, out, iters, clock_mhz, wall_mhz);
  return hipGetLastError();
}
