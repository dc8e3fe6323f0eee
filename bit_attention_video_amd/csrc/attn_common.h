// Device helpers shared by the attention kernels (gfx950 only): lane-pair exchange, direct
// global -> LDS copies, phase barriers, the bf16 matrix instruction and the query-row rotation.
#pragma once

#include "vc_common.h"

namespace vc_attn {

// Maximum of lanes q and q+32 (v_permlane32_swap returns both in every lane).
__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Direct global -> LDS copies (global_load_lds: lane i of the wave writes bytes
// [base + size*i, base + size*(i+1)) of LDS, base taken from M0).  They are issued as inline
// assembly on purpose: the compiler cannot tell the tile being filled from the tiles being
// read, and would otherwise wait for every prefetch before the next LDS read.  Completion
// is awaited explicitly (vmcnt) before the barrier that publishes a tile.
// M0 is written inside the same asm block by s_mov_b32 from a scalar operand, so it is always a
// scalar write, which needs one wait state before the copy reads M0 (the s_nop 0), whatever
// code produced the operand.  (M0 is not in the clobber lists: the compiler treats it as a
// reserved register and keeps no value in it across these kernels, whose only M0 uses are these
// copies.)
// The global address is a scalar base plus a per-lane 32-bit offset, so a copy costs no vector
// instruction.  The base is first moved by s_mov_b64 into a scalar pair of the asm block's own,
// so the copy reads an SGPR pair written by a scalar instruction, which needs no wait states; a
// base written by a vector instruction (v_readfirstlane) would need five before a memory
// instruction reads it, and the compiler does not insert them in front of inline assembly.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds_base) {
  uint64_t base;
  asm volatile("s_mov_b64 %0, %2\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %0"
               : "=&s"(base)
               : "v"(voff), "s"(gbase), "s"(lds_base)
               : "memory");
}
__device__ __forceinline__ void dma4(const void* gbase, uint32_t voff, uint32_t lds_base) {
  uint64_t base;
  asm volatile("s_mov_b64 %0, %2\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %0"
               : "=&s"(base)
               : "v"(voff), "s"(gbase), "s"(lds_base)
               : "memory");
}
// Workgroup barrier between two phases.  No LDS read needs to be complete here: every tile
// buffer is rewritten only after the instructions that consume its reads, and the compiler
// waits for a read before its consumer.  The copies in flight keep going.  The scheduling
// fences keep the compiler from moving any instruction across the barrier, which would mix
// the two phases.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// Wait until at most NOUT of this wave's copies into LDS are in flight (they complete in
// issue order), then the barrier that publishes the completed ones.
template <int NOUT>
__device__ __forceinline__ void wait_dma_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NOUT) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// Pins a phase's results before the barrier that ends it: the compiler may not sink the
// instructions that produce them into the next phase (no instruction is emitted).
template <typename T>
__device__ __forceinline__ void keep(T& x) {
  asm volatile("" : "+v"(x));
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

// Maxima of sixteen elements folded into two running maxima a (even pairs) and b (odd pairs):
// the two chains alternate, so no instruction reads the result of the one just before it (a
// dependent vector instruction waits ~9 cycles, an independent one issues every ~5.5).  With
// INIT the chains start from the first pairs instead of reading a and b.
template <bool INIT>
__device__ __forceinline__ void max16_2chains(float& a, float& b, const v16f& x) {
  if constexpr (INIT)
    asm("v_max_f32 %0, %2, %3\n\t"
        "v_max_f32 %1, %4, %5\n\t"
        "v_max3_f32 %0, %0, %6, %7\n\t"
        "v_max3_f32 %1, %1, %8, %9\n\t"
        "v_max3_f32 %0, %0, %10, %11\n\t"
        "v_max3_f32 %1, %1, %12, %13\n\t"
        "v_max3_f32 %0, %0, %14, %15\n\t"
        "v_max3_f32 %1, %1, %16, %17"
        : "=&v"(a), "=&v"(b)
        : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]),
          "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]));
  else
    asm("v_max3_f32 %0, %0, %2, %3\n\t"
        "v_max3_f32 %1, %1, %4, %5\n\t"
        "v_max3_f32 %0, %0, %6, %7\n\t"
        "v_max3_f32 %1, %1, %8, %9\n\t"
        "v_max3_f32 %0, %0, %10, %11\n\t"
        "v_max3_f32 %1, %1, %12, %13\n\t"
        "v_max3_f32 %0, %0, %14, %15\n\t"
        "v_max3_f32 %1, %1, %16, %17"
        : "+v"(a), "+v"(b)
        : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]),
          "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]));
}

__device__ __forceinline__ v16f mfma_bf16(v8s a, v8s b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                 0, 0, 0);
}

// Rotation of one query row by the Sylvester Hadamard matrix H (entries +-1, App. B's Q pass).
// Lane (q, hl) holds channels 64 c + 32 hl + 8 m + j of row q as x[32 c + 8 m + j]: local index
// bits 0-4 are channel bits 0-4, local bit 5 is channel bit 6, and channel bit 5 is the lane
// half.  The butterflies run in float64, where the signed sum of the 128 float32 terms is exact
// whatever the order, and each result is rounded to float32 once.
__device__ __forceinline__ void hadamard_q_row(float* x, int hl) {
  double y[64];
#pragma unroll
  for (int k = 0; k < 64; ++k) y[k] = (double)x[k];
#pragma unroll
  for (int b = 1; b < 64; b <<= 1)
#pragma unroll
    for (int k = 0; k < 64; ++k)
      if (!(k & b)) {
        const double u = y[k], v = y[k | b];
        y[k] = u + v;
        y[k | b] = u - v;
      }
#pragma unroll
  for (int k = 0; k < 64; ++k) {
    const double o = __shfl_xor(y[k], 32, 64);
    x[k] = (float)(hl ? o - y[k] : y[k] + o);
  }
}

// Query prologue of the 8-bit attention (App. B's Q pass): lane (q, hl) of a wave owns query
// row q and holds its channels 64 c + 32 hl + 8 m + j as x[32 c + 8 m + j] (c, hl in {0,1},
// m < 4, j < 8), multiplied by L = float32(8 log2(e) softmax_scale), then rotated by H when HAD.
template <bool HAD>
__device__ __forceinline__ void q_row_scaled(const uint16_t* __restrict__ qrow, int hl, float L, float* x) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 raw = *(const uint4*)(qrow + 64 * c + 32 * hl + 8 * m);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[32 * c + 8 * m + 2 * e] = bf16_to_f32(wd[e] & 0xFFFFu) * L;
        x[32 * c + 8 * m + 2 * e + 1] = bf16_to_f32(wd[e] >> 16) * L;
      }
    }
  if constexpr (HAD) hadamard_q_row(x, hl);
}
__device__ __forceinline__ float q_row_absmax(const float* x) {
  float a = 0.0f;
#pragma unroll
  for (int k = 0; k < 64; ++k) a = fmaxf(a, fabsf(x[k]));
  return a;
}
// E4M3 codes of x / 2^EQ (qinv = 2^-EQ, exact): word d4 of qf[c] holds the codes of channels
// 64 c + 32 hl + 4 d4 .. 64 c + 32 hl + 4 d4 + 3, the A/B operand bytes of the QK product.
__device__ __forceinline__ void q_row_codes(const float* x, float qinv, v8i* qf) {
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int d4 = 0; d4 < 8; ++d4) {
      const float* y = &x[32 * c + 4 * d4];
      qf[c][d4] = (int)e4m3x4(y[0] * qinv, y[1] * qinv, y[2] * qinv, y[3] * qinv);
    }
}

// Shader-clock stamp: the shader-cycle counter (s_memtime) and the constant-rate counter
// (s_memrealtime) written by lane 0 of the calling wave to out[0], out[1].  A workgroup writes one stamp
// at its start and one at its end; nothing stays live in registers in between.
__device__ __forceinline__ void clock_stamp(uint64_t* out) {
  if (out) {
    const uint64_t w = wall_clock64(), c = clock64();
    if (__lane_id() == 0) {
      out[0] = c;
      out[1] = w;
    }
  }
}

}  // namespace vc_attn
