// FP8 VC-Attention forward on gfx950 (VC-Attention Sec. 3.1 Eq. 1, Sec. 3.2 Eq. 6,
// Sec. 3.3 Eq. 7, App. B).
//
// One workgroup = 4 waves = one 128-row query block of one (b, h); wave w owns queries
// 32w .. 32w+31.  Keys/values stream in tiles of 128 (= B_v, so each tile has one key
// scale sK_j and one mean mu_j), double-buffered in LDS and filled by direct global->LDS
// loads (no staging registers).
//
// Layouts.  Both products use the FP8 32x32x64 matrix instruction with the key index as the
// reduction dimension of PV, computed transposed so one lane owns one query row:
//   S^T (keys x queries) = Kq_j (keys x d) . Qq^T (d x queries)
//   O^T (d x queries)   += Rq_j^T (d x keys) . P^T (keys x queries)
// In the 32x32 result layout lane (q = lane%32, g = lane/32) holds column q and rows
// 8(i/4) + 4g + i%4 (i = 0..15), so every score, row statistic and output element of a
// lane belongs to query q; the lanes q and q+32 share a row and exchange one value.
// The P bytes a lane produces are exactly its B-operand bytes for PV once the residual
// tile is stored in the matching key order (vc_vsmooth_demean_quant's tile-transposed Rq).
//
// ExpCast inside the matrix unit.  The query block is quantised as E4M3(Q L / sQ) with
// L = float32(8 log2(e) softmax_scale), and sQ, sK_j are powers of two (E8M0), so the scaled
// FP8 instruction with block scales sK_j and sQ already returns a*s = 8 log2(e) S, the
// score in Eq. 7's units.  Its accumulator input is b = 119.65 - m (the row maximum folded
// into the constant, Fig. 2 caption), so it returns t = a*s + b and Eq. 7 is left with
// Round and clip: one v_cvt_pk_u8_f32 per element (RNE, saturating; t <= 119.65 + ulp, so
// the saturation at 0 is the clip and 120 is never exceeded).
//
// Running maximum (Eq. 1).  With t = a s + C - m, rowmax(t) - C = a*max(s) - m, so a row's
// maximum grows by delta = max(0, rowmax(t) - C); then t, b and m move by -delta, +delta
// and alpha = 2^(-delta/8) rescales A and l.  Rows that do not grow skip all of it: the
// branch is taken per wave only when some row of the wave grew.
//
// Per tile and row, the rest of Eq. 6: r = sum of decoded codes; l += r; A += P R (FP8 MFMA).
// The rank-one mean term r mu~_j^T also runs on the matrix unit: each row keeps the r of the
// last 16 tiles (rho, rescaled with A when the maximum grows), and once per 16 tiles
// A += mu~^T rho with the bf16 32x32x16 instruction (mu~ is exact bf16; rho is split into
// bf16 hi + lo, 16 significant bits).  So the accumulator A is only touched by vector
// instructions on the tiles where a row maximum grows.
// Epilogue: O = bf16(A * sV / l) (App. B: one multiply by sV serves both terms).
#include "vc_common.h"
#include "vc_internal.h"
#include "vc_attn.h"

namespace {

constexpr int TILE_BYTES = 128 * 128;
constexpr float EC_C = 119.65f;    // 120 + beta, beta = -0.35 (Eq. 7)

typedef __attribute__((address_space(3))) void lds_void;

// Byte offset of 16-byte chunk c16 (0..7) of row `row` in a 128 x 128-byte LDS tile.  The
// chunk index is XORed with (row % 8) ^ (row / 8 % 2): rows r..r+7 then hit 8 different
// 16-byte bank groups of a 128-byte bank period, and rows r..r+15 hit 16 different groups
// of a 256-byte period, so the lanes one LDS cycle serves never share a bank.
__device__ __forceinline__ int swz_phys(int row, int c16) { return c16 ^ (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int c16) { return row * 128 + (swz_phys(row, c16) << 4); }

// Values of lanes q and q+32 (v_permlane32_swap returns both in every lane).
__device__ __forceinline__ float pair_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Direct global -> LDS copy of one 16 KB tile into the swizzled layout: wave w, instruction i
// fills LDS chunks (4w + i) * 64 + lane, so each lane fetches the global chunk that belongs there.
__device__ __forceinline__ void stage_tile(const uint8_t* gtile, uint8_t* ltile, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int P = (4 * w + i) * 64 + lane;
    const int row = P >> 3, c16 = swz_phys(row, P & 7);   // the XOR is an involution
    __builtin_amdgcn_global_load_lds((const void*)(gtile + row * 128 + c16 * 16),
                                     (lds_void*)(ltile + (4 * w + i) * 1024), 16, 0, 0);
  }
}

__device__ __forceinline__ v8i lds_frag32(const uint8_t* tile, int row, int c16) {
  const uint4 lo = *(const uint4*)(tile + swz(row, c16));
  const uint4 hi = *(const uint4*)(tile + swz(row, c16 + 1));
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// E4M3 x E4M3 -> float32, operands scaled by 2^(sa-127) and 2^(sb-127) (E8M0 block scales).
__device__ __forceinline__ v16f mfma_fp8(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ v16f mfma_bf16(v8s a, v8s b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                 0, 0, 0);
}

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
constexpr v2bf BF16_ONES = {(__bf16)1.0f, (__bf16)1.0f};

constexpr int MRING = 32;   // LDS ring of mean rows: two 16-tile groups (one being summed, one filling)

}  // namespace

template <bool NO_MEAN>
__global__ __launch_bounds__(256) void k_attn_fwd(const uint16_t* __restrict__ Q,
                                                  const uint8_t* __restrict__ Kq,
                                                  const float* __restrict__ sK,
                                                  const uint8_t* __restrict__ Rq,
                                                  const uint16_t* __restrict__ mu,
                                                  const float* __restrict__ sV, int N, int nqb,
                                                  uint32_t G, float L, uint16_t* __restrict__ O) {
  __shared__ __attribute__((aligned(1024))) uint8_t kt[2][TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t rt[2][TILE_BYTES];
  __shared__ __attribute__((aligned(256))) uint16_t mring[MRING][128];
  __shared__ float red[4];

  const int t = threadIdx.x, w = t >> 6, lane = t & 63, q = lane & 31, g = lane >> 5;
  const uint32_t item = xcd_remap(blockIdx.x, G);
  const int bh = (int)(item / (uint32_t)nqb), qb = (int)(item % (uint32_t)nqb);
  const int T = N / 128;
  const size_t headN = (size_t)bh * N;
  const int qi = qb * 128 + w * 32 + q;
  const uint8_t* Kh = Kq + headN * VC_D;
  const uint8_t* Rh = Rq + (size_t)bh * T * TILE_BYTES;
  const uint16_t* muh = mu + (size_t)bh * T * VC_D;

  // stage tile 0 (and clear the mean ring)
  stage_tile(Kh, kt[0], w, lane);
  stage_tile(Rh, rt[0], w, lane);
  if (!NO_MEAN)
    for (int i = t; i < MRING * 128 / 2; i += 256) ((uint32_t*)&mring[0][0])[i] = 0u;

  // ---- prologue: Q L, its block scale sQ = 2^E (amax over the 128 x 128 block), E4M3 ----
  const uint16_t* qrow = Q + (headN + qi) * VC_D;
  float qs[64];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint4 raw = *(const uint4*)(qrow + 64 * c + 32 * g + 8 * m);
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_to_f32(wd[e] & 0xFFFFu) * L, hi = bf16_to_f32(wd[e] >> 16) * L;
        qs[32 * c + 8 * m + 2 * e] = lo;
        qs[32 * c + 8 * m + 2 * e + 1] = hi;
        amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
      }
    }
  amax = wave_max(amax);
  if (lane == 0) red[w] = amax;

  __syncthreads();   // red[] and the cleared ring
  if (!NO_MEAN && w == 0)
    __builtin_amdgcn_global_load_lds((const void*)(muh + 2 * lane), (lds_void*)&mring[0][0], 4, 0, 0);
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int EQ = pow2_block_exponent(amax);
  const int sb = 127 + EQ;                         // E8M0 of sQ
  const float qinv = __builtin_ldexpf(1.0f, -EQ);  // exact
  v8i qf[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int d4 = 0; d4 < 8; ++d4) {
      const float* x = &qs[32 * c + 4 * d4];
      qf[c][d4] = (int)e4m3x4(x[0] * qinv, x[1] * qinv, x[2] * qinv, x[3] * qinv);
    }
  __builtin_amdgcn_s_waitcnt(0);   // tile 0 and its mean row have landed in LDS
  __syncthreads();

  float b = 0.0f, l_run = 0.0f;   // b = 119.65 - m; set on the first tile
  v16f bsplat = {};
  float rho[8];                   // r of this group's tiles 8g .. 8g+7 (query q)
#pragma unroll
  for (int k = 0; k < 8; ++k) rho[k] = 0.0f;
  v16f acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = v16f{};

  for (int j = 0; j < T; ++j) {
    const int cur = j & 1;
    if (j + 1 < T) {   // prefetch tile j+1 into the idle buffer (freed by the last barrier)
      stage_tile(Kh + (size_t)(j + 1) * TILE_BYTES, kt[cur ^ 1], w, lane);
      stage_tile(Rh + (size_t)(j + 1) * TILE_BYTES, rt[cur ^ 1], w, lane);
      if (!NO_MEAN && w == 0)
        __builtin_amdgcn_global_load_lds((const void*)(muh + (size_t)(j + 1) * VC_D + 2 * lane),
                                         (lds_void*)&mring[(j + 1) % MRING][0], 4, 0, 0);
    }

    // t = a s + b from the matrix unit: S^T = Kq_j . Qq^T with block scales sK_j, sQ
    const int sa = (int)((__float_as_uint(sK[(size_t)bh * T + j]) >> 23) & 0xFFu);  // E8M0 of sK_j
    v16f s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = mfma_fp8(lds_frag32(kt[cur], 32 * kb + q, 2 * g), qf[0], bsplat, sa, sb);
      s[kb] = mfma_fp8(lds_frag32(kt[cur], 32 * kb + q, 4 + 2 * g), qf[1], s[kb], sa, sb);
    }

    // running maximum (Eq. 1) in t's units
    float tm = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tm = fmaxf(tm, s[kb][i]);
    tm = pair_max(tm);
    const bool first = j == 0;
    const float delta = first ? tm - EC_C : fmaxf(tm - EC_C, 0.0f);
    if (first || __ballot(delta > 0.0f) != 0ull) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] -= delta;
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(-0.125f * delta);
        l_run *= alpha;
#pragma unroll
        for (int k = 0; k < 8; ++k) rho[k] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
      b -= delta;
#pragma unroll
      for (int i = 0; i < 16; ++i) bsplat[i] = b;
    }

    // ExpCast Round + clip: one saturating RNE byte conversion per element, then the PV
    // product of that key half.  Byte jj of the PV B-operand for key half p is element
    // (kb = 2p + jj/16, i = jj%16) of S^T.
    v8i pw[2];
    float r = 0.0f;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int kb = 2 * p + (wd >> 2), i0 = 4 * (wd & 3);
        uint32_t word = 0;
        word = expcast_byte(s[kb][i0 + 0], 0, word);
        word = expcast_byte(s[kb][i0 + 1], 1, word);
        word = expcast_byte(s[kb][i0 + 2], 2, word);
        word = expcast_byte(s[kb][i0 + 3], 3, word);
        pw[p][wd] = (int)word;
      }
      // O^T += Rq_j^T . P^T for this key half
#pragma unroll
      for (int db = 0; db < 4; ++db)
        acc[db] = mfma_fp8(lds_frag32(rt[cur], 32 * db + q, 4 * p + 2 * g), pw[p], acc[db], 127, 127);
      // row sum of the decoded codes (the values the PV instruction consumes): E4M3 values
      // are exact in bf16, and a bf16 dot with (1, 1) adds a pair into the float32 sum
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pw[p][wd], 1.0f, false),
                                            BF16_ONES, r, false);
        r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(pw[p][wd], 1.0f, true),
                                            BF16_ONES, r, false);
      }
    }
    r = pair_sum(r);
    l_run += r;

    // Eq. 6: the rank-one mean term r mu~_j^T, collected per 16-tile group (see the header)
    if (!NO_MEAN) {
      const int jl = j & 15;
#pragma unroll
      for (int k = 0; k < 8; ++k) rho[k] = (g == (jl >> 3) && k == (jl & 7)) ? r : rho[k];
      if (jl == 15 || j == T - 1) {
        v8s bhi, blo;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const uint32_t hi = f32_to_bf16_rne(rho[k]);
          bhi[k] = (short)hi;
          blo[k] = (short)f32_to_bf16_rne(rho[k] - bf16_to_f32(hi));
          rho[k] = 0.0f;
        }
        const int t0 = (j & ~15) + 8 * g;   // first tile of this lane's K-slots
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          v8s am;
#pragma unroll
          for (int k = 0; k < 8; ++k) am[k] = (short)mring[(t0 + k) % MRING][32 * db + q];
          acc[db] = mfma_bf16(am, bhi, acc[db]);
          acc[db] = mfma_bf16(am, blo, acc[db]);
        }
      }
    }

    __builtin_amdgcn_s_waitcnt(0);   // the prefetched tile has landed before the barrier publishes it
    __syncthreads();
  }

  // ---- epilogue: O = A * sV / l -> bf16 ----
  const float inv_l = 1.0f / l_run;
  const float* sv = sV + (size_t)bh * VC_D;
  uint16_t* orow = O + (headN + qi) * VC_D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int d0 = 32 * db + 8 * ig + 4 * g;
      const float4 s4 = *(const float4*)(sv + d0);
      const uint32_t o0 = f32_to_bf16_rne(acc[db][4 * ig + 0] * s4.x * inv_l);
      const uint32_t o1 = f32_to_bf16_rne(acc[db][4 * ig + 1] * s4.y * inv_l);
      const uint32_t o2 = f32_to_bf16_rne(acc[db][4 * ig + 2] * s4.z * inv_l);
      const uint32_t o3 = f32_to_bf16_rne(acc[db][4 * ig + 3] * s4.w * inv_l);
      *(uint2*)(orow + d0) = make_uint2(o0 | (o1 << 16), o2 | (o3 << 16));
    }
}

hipError_t vc_launch_attn_fwd(const uint16_t* Q, const uint8_t* Kq, const float* sK,
                              const uint8_t* Rq, const uint16_t* mu, const float* sV,
                              int BH, int N, float L, unsigned flags, uint16_t* O,
                              hipStream_t s) {
  const int nqb = N / 128;
  const uint32_t G = (uint32_t)BH * (uint32_t)nqb;
  if (flags & VC_ATTN_NO_MEAN)
    hipLaunchKernelGGL(k_attn_fwd<true>, dim3(G), dim3(256), 0, s, Q, Kq, sK, Rq, mu, sV, N, nqb, G, L, O);
  else
    hipLaunchKernelGGL(k_attn_fwd<false>, dim3(G), dim3(256), 0, s, Q, Kq, sK, Rq, mu, sV, N, nqb, G, L, O);
  return hipGetLastError();
}
