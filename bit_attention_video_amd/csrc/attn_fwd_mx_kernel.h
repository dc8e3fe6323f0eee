// The 4-bit and 6-bit VC-Attention forward kernel on gfx950 (a header: the rotated no-mean
// 6-bit instantiation is built in a translation unit of its own, attn_fwd_mx6_rn.hip).
// At 4 bits the operands are MX E2M1 under per-32 E8M0 scales for Q, K, P
// and the value residual (VC-Attention Sec. 3.2 Eq. 4 and Eq. 6 with the 4-bit value quantiser;
// Sec. 4.1 "Implementation"; App. A "Scope of ExpCast-FP8"; App. B).
//
// The schedule is the 8-bit kernel's (attn_fwd.hip): one workgroup = two groups of four waves
// in ping-pong, group g owning the 128-query block 2 wb + g and each wave 32 queries; K and R
// tiles copied three steps ahead into four-deep LDS rings by direct global->LDS copies; both
// products computed transposed (S^T = K Q^T, O^T += R^T P^T) so that one lane owns one query
// row; row sums and Eq. 6's mean term on the matrix unit.  What changes at 4 bits:
//  * a tile is 128 x 64 bytes of E2M1 codes (two per byte, even index in the low nibble) plus
//    128 x 4 scale bytes, one per 32-element group of a row;
//  * the FP4 matrix instruction takes a scale per lane: lane (q, h) of the 32x32x64 product
//    holds 32 K-elements of one row or column, exactly one scale group, and the instruction's
//    byte select picks that group's byte from a 32-bit register.  K and R scales come from
//    LDS (a row's four group bytes in one dword; step s of lane half h needs group 2 s + h,
//    i.e. bytes 0 and 2 of the dword shifted right by 8 h), Q scales from the prologue, P
//    scales from the vector phase (byte s for step s);
//  * P = 2^(S L4 - m) with L4 = log2(e) softmax_scale, by v_exp_f32: E2M1 has no affine
//    log-domain code map, so ExpCast does not apply (App. A).  A lane's 32 values of one PV
//    step form one 32-key group, so its scale and codes need no other lane;
//  * the running maximum lives in the accumulator input b = -m, so the score instruction
//    returns t = S L4 - m directly; alpha = 2^(-delta);
//  * means are stored unscaled (App. B: the microscales act inside the instruction) and
//    O = bf16(A / l).
// The same kernel runs the 6-bit path (BITS = 6, MX E2M3 elements): a row of a tile is then
// 128 bytes holding four groups of 24 code bytes (the first 16 bytes of each group in chunks 0-3,
// the last 8 of groups 0 and 2 in chunk 4, of groups 1 and 3 in chunk 5, then 32 zero bytes),
// swizzled like the 8-bit kernel's rows; a lane's fragment is the 24 code bytes of its group (six
// registers), and the conversions are the E2M3 ones (scale rule: amax <= 7.5 2^E).
#pragma once

#include "vc_common.h"
#include "vc_internal.h"
#include "vc_attn.h"
#include "attn_common.h"

#include <type_traits>

namespace {

using namespace vc_attn;

typedef int v4i __attribute__((ext_vector_type(4)));

typedef int v6i_ __attribute__((ext_vector_type(6)));

// Element formats: bytes per tile row, the matrix instructions' format code, 16-byte copies per
// lane and wave for one tile, the register type of a lane's 32 elements.
template <int BITS> struct MxFmt;
template <> struct MxFmt<4> {
  static constexpr int ROWB = 64, CODE = 4, NCOPY = 1;
  typedef v4i frag_t;
};
template <> struct MxFmt<6> {
  static constexpr int ROWB = 128, CODE = 2, NCOPY = 2;
  typedef v6i_ frag_t;
};
constexpr int STILE = 128 * 4;      // scale bytes of a tile
constexpr int NWAVE = 8;
constexpr int MRING = 32;
constexpr int NBUF = 4;

// Byte offset of 16-byte chunk c (0..3) of row `row` in a 128 x 64-byte LDS tile.  The chunk
// index is XORed with (row / 4) % 4: a 256-byte bank period holds four rows, and rows
// r .. r+15 then hit 16 different 16-byte bank groups.
__device__ __forceinline__ int swz4_phys(int row, int c) { return c ^ ((row >> 2) & 3); }
__device__ __forceinline__ int swz4(int row, int c) { return row * 64 + (swz4_phys(row, c) << 4); }

// Source offset of the chunk lane `lane` of wave w copies: the wave's one 16-byte copy per lane
// fills LDS chunks 64 w + lane of the swizzled tile.
__device__ __forceinline__ int stage4_src(int w, int lane) {
  const int P = 64 * w + lane;
  const int row = P >> 2;
  return row * 64 + (swz4_phys(row, P & 3) << 4);
}

__device__ __forceinline__ v4i lds_frag16(const uint8_t* tile, int row, int c) {
  const uint4 v = *(const uint4*)(tile + swz4(row, c));
  return v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
}

// 6-bit tiles: 128-byte rows, 16-byte chunk c16 (0..7) of row `row` XOR-swizzled by
// (row % 8) ^ (row / 8 % 2) as in the 8-bit kernel; group g is chunks 2 g and 2 g + 1.
__device__ __forceinline__ int swz6(int row, int c16) {
  return row * 128 + ((c16 ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}
// Source offset of the chunk lane `lane` of wave w copies with instruction i: the instruction
// fills LDS chunks (2 w + i) * 64 + lane of the swizzled tile.
__device__ __forceinline__ int stage6_src(int w, int i, int lane) {
  const int P = (2 * w + i) * 64 + lane;
  const int row = P >> 3;
  return row * 128 + (((P & 7) ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}
// The fragments of groups hl and 2 + hl of row `row` (a lane's two groups).  In a 6-bit row, chunk g
// holds the first 16 code bytes of group g and chunk 4 + hl the last 8 of groups hl and 2 + hl, so
// three 16-byte reads give both fragments; every read is a whole chunk, which the swizzle keeps
// free of bank conflicts (an 8-byte read of half a chunk by 32 lanes could reach only half of the
// banks).
template <int BITS>
__device__ __forceinline__ void lds_frag_pair(const uint8_t* tile, int row, int hl,
                                              typename MxFmt<BITS>::frag_t& fa,
                                              typename MxFmt<BITS>::frag_t& fb) {
  if constexpr (BITS == 4) {
    fa = lds_frag16(tile, row, hl);
    fb = lds_frag16(tile, row, 2 + hl);
  } else {
    const uint4 la = *(const uint4*)(tile + swz6(row, hl));
    const uint4 lb = *(const uint4*)(tile + swz6(row, 2 + hl));
    const uint4 hi = *(const uint4*)(tile + swz6(row, 4 + hl));
    fa = v6i_{(int)la.x, (int)la.y, (int)la.z, (int)la.w, (int)hi.x, (int)hi.y};
    fb = v6i_{(int)lb.x, (int)lb.y, (int)lb.z, (int)lb.w, (int)hi.z, (int)hi.w};
  }
}
template <int BITS>
__device__ __forceinline__ int stage_src_mx(int w, int i, int lane) {
  if constexpr (BITS == 4) return stage4_src(w, lane);
  else return stage6_src(w, i, lane);
}

// The instructions take eight registers; only the first four (E2M1) or six (E2M3) are read.
__device__ __forceinline__ v8i wide(v4i a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3); }
__device__ __forceinline__ v8i wide(v6i_ a) { return __builtin_shufflevector(a, a, 0, 1, 2, 3, 4, 5, 0, 1); }

// E2M1 x E2M1 -> float32; byte OA of sa and byte OB of sb are the E8M0 scales of this lane's
// A and B groups.
template <int BITS, int OA, int OB, typename F>
__device__ __forceinline__ v16f mfma_mx(F a, F b, v16f c, int sa, int sb) {
  constexpr int C = MxFmt<BITS>::CODE;
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wide(a), wide(b), c, C, C, OA, sa, OB, sb);
}
template <int BITS, int OB, typename F>
__device__ __forceinline__ v4f mfma_mx_16(F a, F b, v4f c, int sb) {
  constexpr int C = MxFmt<BITS>::CODE;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wide(a), wide(b), c, C, C, 0, 127, OB, sb);
}

// Constant A operand of the row-sum product (16x16x128, E2M1): the same 0/1 pattern as the
// 8-bit kernel's (lane l holds row/column l%16 and k-block l/16; rows 0 and 8 are ones on
// k-blocks 0 and 2, rows 4 and 12 on k-blocks 1 and 3), with E2M1 1.0 = nibble 0x2.  With the
// P codes as B and each lane's P scale as the B scale, lane l reads in result register 0 the
// sum of its own query's dequantised P over the 64 keys of one PV step.
__device__ __forceinline__ int rowsum_ones4_word(int lane) {
  const int i = lane & 15, G = lane >> 4;
  const bool one = (G & 1) ? (i == 4 || i == 12) : (i == 0 || i == 8);
  return one ? 0x22222222 : 0;   // eight E2M1 1.0
}
// Built once and kept in registers for the whole key loop (opaque, so it is not rebuilt per tile).
__device__ __forceinline__ v4i rowsum_ones4(int lane) {
  const int word = rowsum_ones4_word(lane);
  v4i r = v4i{word, word, word, word};
  asm volatile("" : "+v"(r));
  return r;
}

// E2M1 codes of 32 values x divided by their power-of-two group scale `scale`: nibble k = value
// k.  The conversion instruction divides by its scale operand itself (bit for bit the codes of
// x / scale, checked on the device for power-of-two scales), so no separate multiply runs.
__device__ __forceinline__ v4i pack_fp4_32(const float* x, float scale) {
  v4i r;
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * wd + 0], x[8 * wd + 1], scale, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * wd + 2], x[8 * wd + 3], scale, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * wd + 4], x[8 * wd + 5], scale, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[8 * wd + 6], x[8 * wd + 7], scale, 3);
    r[wd] = (int)w;
  }
  return r;
}
// E2M3 codes of 32 values divided by their group scale (the conversion divides by its scale
// operand; checked on the device for power-of-two scales), value k in bits 6k .. 6k + 5: the
// conversion interleaves its two operands, so the even values go in the first (as fp6x32).
__device__ __forceinline__ v6i_ pack_fp6_32(const float* x, float scale) {
  v16f lo, hi;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    lo[k] = x[2 * k];
    hi[k] = x[2 * k + 1];
  }
  return __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(lo, hi, scale);
}
// The row-sum operand in E2M3: 1.0 (code 0b001000) in all 32 fields of the lanes that
// rowsum_ones4_word marks, zero elsewhere.  It is rebuilt in each matrix phase from a per-lane
// 0/1 flag made opaque there (six selects), not kept resident: at 6 bits the 256-register
// budget has no room for it beside the residual and key fragments.
__device__ __forceinline__ v6i_ rowsum_ones6(uint32_t flag) {
  asm volatile("" : "+v"(flag));
  const int m = -(int)flag;
  return v6i_{m & 0x08208208, m & (int)0x82082082u, m & 0x20820820, m & 0x08208208, m & (int)0x82082082u,
              m & 0x20820820};
}

template <int BITS>
__device__ __forceinline__ typename MxFmt<BITS>::frag_t pack_mx(const float* x, float scale) {
  if constexpr (BITS == 4) return pack_fp4_32(x, scale);
  else return pack_fp6_32(x, scale);
}
template <int BITS>
__device__ __forceinline__ int mx_exp(float amax) {
  if constexpr (BITS == 4) return mx_exponent(amax);
  else return mx6_exponent(amax);
}

template <int BITS, bool NO_MEAN, bool HAD>
__global__ __launch_bounds__(512) void k_attn_fwd_mx4(const uint16_t* __restrict__ Q,
                                                      const uint8_t* __restrict__ Kq4,
                                                      const uint8_t* __restrict__ sK4,
                                                      const uint8_t* __restrict__ Rq4,
                                                      const uint8_t* __restrict__ sR4,
                                                      const uint16_t* __restrict__ mu, int N, int nqb,
                                                      int nwb, uint32_t G, float L4,
                                                      uint16_t* __restrict__ O) {
  using FM = MxFmt<BITS>;
  typedef typename FM::frag_t frag_t;
  constexpr int TILE4 = 128 * FM::ROWB;    // code bytes of a 128 x 128 tile
  __shared__ __attribute__((aligned(1024))) uint8_t kt[NBUF][TILE4];
  __shared__ __attribute__((aligned(1024))) uint8_t rt[NBUF][TILE4];
  __shared__ __attribute__((aligned(256))) uint8_t kst[NBUF][STILE];
  __shared__ __attribute__((aligned(256))) uint8_t rst[NBUF][STILE];
  __shared__ __attribute__((aligned(256))) uint16_t mring[MRING][128];
  __shared__ __attribute__((aligned(16))) float rsnap[NWAVE * 32][12];

  const int t = threadIdx.x, lane = t & 63, q = lane & 31, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = w >> 2;
  const uint32_t item = xcd_remap(blockIdx.x, G);
  const int bh = (int)(item / (uint32_t)nwb), qb = 2 * (int)(item % (uint32_t)nwb) + grp;
  const bool valid = qb < nqb;
  const int T = N / 128;
  const size_t headN = (size_t)bh * N;
  const int qi = (valid ? qb : nqb - 1) * 128 + (w & 3) * 32 + q;
  const uint8_t* Kh = Kq4 + headN * FM::ROWB;
  const uint8_t* sKh = sK4 + headN * 4;
  const uint8_t* Rh = Rq4 + (size_t)bh * T * TILE4;
  const uint8_t* sRh = sR4 + (size_t)bh * T * STILE;
  const uint16_t* muh = mu + (size_t)bh * T * VC_D;

  // copies per wave and step: NCOPY 16-byte chunks per lane of the K and of the R code tile;
  // waves 0-1 copy the K scale tile, waves 2-3 the R scale tile (4 bytes per lane), wave 4 the
  // mean row
  constexpr int NC = FM::NCOPY;
  const uint32_t so = stage_src_mx<BITS>(w, 0, lane), so1 = stage_src_mx<BITS>(w, NC - 1, lane);
  const uint32_t kt0 = lds_addr(&kt[0][0]) + NC * w * 1024, rt0 = lds_addr(&rt[0][0]) + NC * w * 1024;
  const uint32_t ks0 = lds_addr(&kst[0][0]), rs0 = lds_addr(&rst[0][0]);
  const uint32_t mr0 = lds_addr(&mring[0][0]);
  constexpr int D = NBUF - 1;
  auto clampT = [&](int i) { return i < T ? i : T - 1; };
  auto lane4 = [&]() { return (uint32_t)(4 * lane); };   // the 4-byte copies' lane offset
  auto k_tile = [&](int i, int slot) {
    dma16(Kh + (size_t)i * TILE4, so, kt0 + slot * TILE4);
    if constexpr (NC == 2) dma16(Kh + (size_t)i * TILE4, so1, kt0 + slot * TILE4 + 1024);
    if (w < 2) dma4(sKh + (size_t)i * STILE + 256 * w, lane4(), ks0 + slot * STILE + 256 * w);
  };
  auto r_tile = [&](int i, int slot) {
    dma16(Rh + (size_t)i * TILE4, so, rt0 + slot * TILE4);
    if constexpr (NC == 2) dma16(Rh + (size_t)i * TILE4, so1, rt0 + slot * TILE4 + 1024);
    if (w == 2 || w == 3) dma4(sRh + (size_t)i * STILE + 256 * (w - 2), lane4(), rs0 + slot * STILE + 256 * (w - 2));
    if (!NO_MEAN && w == 4) dma4(muh + (size_t)i * VC_D, lane4(), mr0 + (i % MRING) * 256);
  };
  auto issue = [&](int j) {
    k_tile(clampT(j + D), (j + D) % NBUF);
    r_tile(clampT(j + D - 1), (j + D - 1) % NBUF);
  };
  const bool extra = w < 4 || (!NO_MEAN && w == 4);   // this wave issues a third copy per step
  auto wait_step = [&]() {
    if (extra) wait_dma_barrier<(D - 2) * (2 * NC + 1)>();
    else wait_dma_barrier<(D - 2) * 2 * NC>();
  };

  if (!NO_MEAN)
    for (int i = t; i < MRING * 128 / 2; i += NWAVE * 64) ((uint32_t*)&mring[0][0])[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < D; ++i) k_tile(clampT(i), i);
#pragma unroll
  for (int i = 0; i < D - 1; ++i) r_tile(clampT(i), i);

  // ---- prologue: Q L4 (rotated by H when HAD), E2M1 per 32-channel group of the row.  Lane
  // (q, h) holds channels 64 c + 32 h + k as qs[32 c + k]: group 2 c + h, which is also the
  // lane's B-operand block of the score product's step c. ----
  const uint16_t* qrow = Q + (headN + qi) * VC_D;
  float qs[64];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 raw = *(const uint4*)(qrow + 64 * c + 32 * hl + 8 * m);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qs[32 * c + 8 * m + 2 * e] = bf16_to_f32(wd[e] & 0xFFFFu) * L4;
        qs[32 * c + 8 * m + 2 * e + 1] = bf16_to_f32(wd[e] >> 16) * L4;
      }
    }
  if constexpr (HAD) hadamard_q_row(qs, hl);
  frag_t qf[2];
  int qsc = 0;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    float a = 0.0f;
#pragma unroll
    for (int k = 0; k < 32; ++k) a = fmaxf(a, fabsf(qs[32 * c + k]));
    const int E = mx_exp<BITS>(a);
    qf[c] = pack_mx<BITS>(&qs[32 * c], __builtin_ldexpf(1.0f, E));
    qsc |= (E + 127) << (8 * c);
  }
  wait_dma_barrier<0>();

  const v4i ones4 = rowsum_ones4(lane);   // resident at 4 bits
  const uint32_t ones_flag = rowsum_ones4_word(lane) ? 1u : 0u;
  auto ones = [&]() {
    if constexpr (BITS == 4) return ones4;
    else return rowsum_ones6(ones_flag);
  };
  float b = 0.0f, l_run = 0.0f;   // b = -m
  // b in every element: the QK accumulator input, kept in registers and rebuilt only when b
  // changes (a running-maximum update)
  v16f bsplat = {};
  float rA[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rA[k] = 0.0f;
  bool snapped = false;
  float* my_snap = &rsnap[w * 32 + q][0];
  auto push_r = [&](float r, int e) {   // r of tile e (see attn_fwd.hip)
#pragma unroll
    for (int k = 0; k < 7; ++k) rA[k] = rA[k + 1];
    rA[7] = r;
    if ((e & 15) == 7) {
      *(float4*)my_snap = make_float4(rA[0], rA[1], rA[2], rA[3]);
      *(float4*)(my_snap + 4) = make_float4(rA[4], rA[5], rA[6], rA[7]);
#pragma unroll
      for (int k = 0; k < 8; ++k) rA[k] = 0.0f;
      my_snap[8] = b;
      snapped = true;
    }
  };
  v16f acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = v16f{};
  v16f s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) s[kb] = v16f{};
  frag_t pw[2] = {};
  int psc = 0x7F7F;               // P scales of the two PV steps (bytes 0 and 1)
  frag_t rf[8];                   // residual fragments of the next PV product
#pragma unroll
  for (int i = 0; i < 8; ++i) rf[i] = frag_t{};
  // their scale dwords shifted right by 8 h: bytes 0 and 2 are then the groups h and 2 + h of
  // this lane half's 32-slot blocks in the two PV steps
  int rsw[4] = {0, 0, 0, 0};
  v4f rs = {};

  // Eq. 6's mean term of the 16-tile group that ends with tile e: A += mu~^T rho
  auto mean_group = [&](int e) {
    float rB[8];
    if (snapped) {
      const float4 s0 = *(const float4*)my_snap, s1 = *(const float4*)(my_snap + 4);
      const float f = __builtin_amdgcn_exp2f(b - my_snap[8]);
      rB[0] = s0.x * f; rB[1] = s0.y * f; rB[2] = s0.z * f; rB[3] = s0.w * f;
      rB[4] = s1.x * f; rB[5] = s1.y * f; rB[6] = s1.z * f; rB[7] = s1.w * f;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) rB[k] = 0.0f;
    }
    snapped = false;
    // rho = bf16 hi + bf16 lo, two values per hardware conversion (round to nearest even)
    typedef float v2f_ __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf_ __attribute__((ext_vector_type(2)));
    v8s bhi, blo;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const v2f_ x = {hl ? rA[k] : rB[k], hl ? rA[k + 1] : rB[k + 1]};
      const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf_));
      const v2f_ rest = {x[0] - __uint_as_float(hw << 16), x[1] - __uint_as_float(hw & 0xFFFF0000u)};
      const uint32_t lw = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, v2bf_));
      bhi[k] = (short)(hw & 0xFFFFu); bhi[k + 1] = (short)(hw >> 16);
      blo[k] = (short)(lw & 0xFFFFu); blo[k + 1] = (short)(lw >> 16);
      rA[k] = 0.0f; rA[k + 1] = 0.0f;
    }
    const int t0 = hl ? e - 7 : (e & ~15);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      v8s am;
#pragma unroll
      for (int k = 0; k < 8; ++k) am[k] = (short)mring[(t0 + k) & (MRING - 1)][32 * db + q];
      acc[db] = mfma_bf16(am, bhi, acc[db]);
      acc[db] = mfma_bf16(am, blo, acc[db]);
    }
  };

  // M(j): A += P R and the row sum of tile j-1, then S^T of tile j (t = S L4 + b).
  auto mphase = [&](int j, auto qk, auto pv) {
    constexpr bool QK = decltype(qk)::value, PV = decltype(pv)::value;
    frag_t kf[8];
    int ksw[4];
    auto load_k = [&]() {
      const uint8_t* kb_ = kt[j % NBUF];
      const uint8_t* ksb = kst[j % NBUF];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        lds_frag_pair<BITS>(kb_, 32 * kb + q, hl, kf[2 * kb], kf[2 * kb + 1]);
        ksw[kb] = (int)(*(const uint32_t*)(ksb + 4 * (32 * kb + q)) >> (8 * hl));
      }
    };
    // the key fragments are read first, their latency hidden behind the PV products.  (Reading
    // them after the PV products are issued, into the residual fragments' registers, frees
    // registers at 6 bits but gave wrong products on the device: nothing keeps the reads from
    // overwriting a source of a product still queued on the matrix unit.)
    if constexpr (QK) load_k();
    if constexpr (PV) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        acc[db] = mfma_mx<BITS, 0, 0>(rf[db], pw[0], acc[db], rsw[db], psc);
        acc[db] = mfma_mx<BITS, 2, 1>(rf[4 + db], pw[1], acc[db], rsw[db], psc);
      }
      const frag_t one = ones();
      rs = mfma_mx_16<BITS, 0>(one, pw[0], v4f{}, psc);
      rs = mfma_mx_16<BITS, 1>(one, pw[1], rs, psc);
    }
    if constexpr (QK) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = mfma_mx<BITS, 0, 0>(kf[2 * kb], qf[0], bsplat, ksw[kb], qsc);
        s[kb] = mfma_mx<BITS, 2, 1>(kf[2 * kb + 1], qf[1], s[kb], ksw[kb], qsc);
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) keep(s[kb]);
    }
    if constexpr (PV) keep(rs);
    if constexpr (PV)
      if (!NO_MEAN && j >= 2 && ((j - 2) & 15) == 15) mean_group(j - 2);
  };
  constexpr std::true_type Y{};
  constexpr std::false_type X{};

  // V(j): r of tile j-1 into l and rho, running maximum of tile j, P = 2^t and its E2M1 codes
  auto vphase = [&](int j) {
    {
      const float r = rs[0];
      l_run += r;
      if (!NO_MEAN) push_r(r, j - 1);
    }
    // the maxima of the two 32-value groups (PV step p: blocks 2p and 2p+1), then the row's
    float gA, gB, hA, hB;
    max16_2chains<true>(gA, gB, s[0]);
    max16_2chains<false>(gA, gB, s[1]);
    max16_2chains<true>(hA, hB, s[2]);
    max16_2chains<false>(hA, hB, s[3]);
    const float gmax[2] = {fmaxf(gA, gB), fmaxf(hA, hB)};
    const float tm = pair_max(fmaxf(gmax[0], gmax[1]));
    const bool first = j == 0;
    const float delta = first ? tm : fmaxf(tm, 0.0f);
    if (first || __ballot(delta > 0.0f) != 0ull) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] -= delta;
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        l_run *= alpha;
#pragma unroll
        for (int k = 0; k < 8; ++k) rA[k] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
      b -= delta;
      {   // eight 64-bit copies of the pair (b, b)
        typedef double v8d __attribute__((ext_vector_type(8)));
        double bb = __builtin_bit_cast(double, ((uint64_t)__float_as_uint(b) << 32) | __float_as_uint(b));
        asm("" : "+v"(bb));   // opaque, so the compiler does not turn it back into a float splat
        const v8d wv = {bb, bb, bb, bb, bb, bb, bb, bb};
        bsplat = __builtin_bit_cast(v16f, wv);
      }
      asm volatile("" : "+v"(bsplat));   // opaque: kept, not rebuilt from b where it is used
    }
    // value k of PV step p is element (kb = 2p + k/16, i = k%16) of S^T
    int sc = 0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float e[32];
#pragma unroll
      for (int k = 0; k < 32; ++k) e[k] = __builtin_amdgcn_exp2f(s[2 * p + (k >> 4)][k & 15]);
      // the group's largest P: its largest score shifted like every score (delta is 0 where the
      // maximum did not grow) is the very float32 its exponential came from, so one more
      // exp2 returns that element's value (exp2 is monotonic) instead of a 32-value max
      const float a = __builtin_amdgcn_exp2f(gmax[p] - delta);
      const int E = mx_exp<BITS>(a);
      pw[p] = pack_mx<BITS>(e, __builtin_ldexpf(1.0f, E));
      sc |= (E + 127) << (8 * p);
    }
    psc = sc;
    keep(pw[0]);
    keep(pw[1]);
    keep(psc);
    {   // the residual fragments of PV(j) and their scales, the first products of M(j+1)
      const uint8_t* rb = rt[j % NBUF];
      const uint8_t* rsb = rst[j % NBUF];
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        lds_frag_pair<BITS>(rb, 32 * db + q, hl, rf[db], rf[4 + db]);
        rsw[db] = (int)(*(const uint32_t*)(rsb + 4 * (32 * db + q)) >> (8 * hl));
      }
    }
  };

  if (!valid) {
    for (int j = 0; j < T; ++j) {
      issue(j);
      phase_barrier();
      wait_step();
    }
    phase_barrier();
    wait_dma_barrier<0>();
    return;
  }
  if (grp == 0) {
    mphase(0, Y, X);
    phase_barrier();
    issue(0);
    vphase(0);
    wait_step();
    for (int j = 1; j < T; ++j) {
      mphase(j, Y, Y);
      phase_barrier();
      issue(j);
      vphase(j);
      wait_step();
    }
    mphase(T, X, Y);
    phase_barrier();
    wait_dma_barrier<0>();
  } else {
    issue(0);
    phase_barrier();
    mphase(0, Y, X);
    wait_step();
    for (int j = 1; j < T; ++j) {
      issue(j);
      vphase(j - 1);
      phase_barrier();
      mphase(j, Y, Y);
      wait_step();
    }
    vphase(T - 1);
    phase_barrier();
    mphase(T, X, Y);
    wait_dma_barrier<0>();
  }

  // ---- epilogue: r of the last tile, the last mean group, O = A / l -> bf16 ----
  {
    const float r = rs[0];
    l_run += r;
    if (!NO_MEAN) {
      push_r(r, T - 1);
      mean_group(T - 1);
    }
  }
  const float inv_l = 1.0f / l_run;
  uint16_t* orow = O + (headN + qi) * VC_D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int d0 = 32 * db + 8 * ig + 4 * hl;
      const uint32_t o0 = f32_to_bf16_rne(acc[db][4 * ig + 0] * inv_l);
      const uint32_t o1 = f32_to_bf16_rne(acc[db][4 * ig + 1] * inv_l);
      const uint32_t o2 = f32_to_bf16_rne(acc[db][4 * ig + 2] * inv_l);
      const uint32_t o3 = f32_to_bf16_rne(acc[db][4 * ig + 3] * inv_l);
      *(uint2*)(orow + d0) = make_uint2(o0 | (o1 << 16), o2 | (o3 << 16));
    }
}

// One launch of the kernel: one workgroup per pair of 128-query blocks of a head.
template <int BITS, bool NO_MEAN, bool HAD>
hipError_t launch_attn_mx(const uint16_t* Q, const uint8_t* Kq, const uint8_t* sK, const uint8_t* Rq,
                          const uint8_t* sR, const uint16_t* mu, int BH, int N, float L4, uint16_t* O,
                          hipStream_t s) {
  const int nqb = N / 128, nwb = (nqb + 1) / 2;
  const uint32_t G = (uint32_t)BH * (uint32_t)nwb;
  hipLaunchKernelGGL((k_attn_fwd_mx4<BITS, NO_MEAN, HAD>), dim3(G), dim3(NWAVE * 64), 0, s, Q, Kq, sK, Rq, sR,
                     mu, N, nqb, nwb, G, L4, O);
  return hipGetLastError();
}

}  // namespace
