// FP8 VC-Attention forward on gfx950 (VC-Attention Sec. 3.1 Eq. 1, Sec. 3.2 Eq. 6,
// Sec. 3.3 Eq. 7, App. B).
//
// One workgroup = 4 waves = one 128-row query block of one (b, h); wave w owns queries
// 32w .. 32w+31.  Keys/values stream in tiles of 128 (= B_v, so each tile has one key
// scale sK_j and one mean mu_j), double-buffered through LDS.
//
// Layouts.  Both products use the FP8 32x32x64 matrix instruction with the key index as the
// reduction dimension of PV, computed transposed so one lane owns one query row:
//   S^T (keys x queries) = Kq_j (keys x d) . Qq^T (d x queries)
//   O^T (d x queries)   += Rq_j^T (d x keys) . P^T (keys x queries)
// In the 32x32 result layout lane (q = lane%32, g = lane/32) holds column q and rows
// 8(i/4) + 4g + i%4 (i = 0..15), so every score, row statistic and output element of a
// lane belongs to query q; the two lanes q and q+32 share a row and exchange one value.
// The P bytes a lane produces are exactly its B-operand bytes for PV once the residual
// tile is stored in the matching key order (vc_vsmooth_demean_quant's tile-transposed Rq).
//
// Per tile, per query row (Eq. 1 with the Fig. 2 / Eq. 7 folding, in units of 8 log2(e) S):
//   a = float32(qa * sK_j), qa = float32(L * sQ), L = float32(8 log2(e) softmax_scale)
//   m' = max(m, a * rowmax s);  b = float32(119.65 - m');  alpha = 2^((m - m')/8)
//   code = clamp(RNE(fma(a, s, b)), 0, 255) by v_cvt_pk_u8_f32; fma(a,s,b) <= 119.65 + ulp,
//          so this is Eq. 7's clip to [0, 120]; the byte is the E4M3 P element
//   r = sum of decoded codes;  l = alpha l + r;  A = alpha A + r mu~_j (Eq. 6), then += P R
// Epilogue: O = bf16(A * sV / l) (App. B: one multiply by sV serves both terms).
#include "vc_common.h"
#include "vc_internal.h"
#include "vc_attn.h"

namespace {

constexpr int TILE_BYTES = 128 * 128;

// Byte offset of 16-byte chunk c16 (0..7) of row `row` in a 128 x 128-byte LDS tile; the
// chunk index is XORed with row%8 so the 8 lanes served together hit 8 different bank groups.
__device__ __forceinline__ int swz(int row, int c16) { return row * 128 + ((c16 ^ (row & 7)) << 4); }

__device__ __forceinline__ v8i lds_frag32(const uint8_t* tile, int row, int c16) {
  const uint4 lo = *(const uint4*)(tile + swz(row, c16));
  const uint4 hi = *(const uint4*)(tile + swz(row, c16 + 1));
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ v16f mfma_fp8(v8i a, v8i b, v16f c) {
  // cbsz = blgp = 0: both operands E4M3; E8M0 scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

}  // namespace

template <bool NO_MEAN>
__global__ __launch_bounds__(256) void k_attn_fwd(const uint16_t* __restrict__ Q,
                                                  const uint8_t* __restrict__ Kq,
                                                  const float* __restrict__ sK,
                                                  const uint8_t* __restrict__ Rq,
                                                  const uint16_t* __restrict__ mu,
                                                  const float* __restrict__ sV, int N, int nqb,
                                                  uint32_t G, float L, uint16_t* __restrict__ O) {
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t rt[2][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) float mus[2][128];
  __shared__ float red[4];

  const int t = threadIdx.x, w = t >> 6, lane = t & 63, q = lane & 31, g = lane >> 5;
  const uint32_t item = xcd_remap(blockIdx.x, G);
  const int bh = (int)(item / (uint32_t)nqb), qb = (int)(item % (uint32_t)nqb);
  const int T = N / 128;
  const size_t headN = (size_t)bh * N;
  const int qi = qb * 128 + w * 32 + q;

  // ---- prologue: Q block scale (amax over the 128 x 128 block) and E4M3 Q fragments ----
  const uint16_t* qrow = Q + (headN + qi) * VC_D;
  uint4 qraw[2][4];
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      qraw[c][m] = *(const uint4*)(qrow + 64 * c + 32 * g + 8 * m);
      const uint32_t wd[4] = {qraw[c][m].x, qraw[c][m].y, qraw[c][m].z, qraw[c][m].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        amax = fmaxf(amax, fabsf(bf16_to_f32(wd[e] & 0xFFFFu)));
        amax = fmaxf(amax, fabsf(bf16_to_f32(wd[e] >> 16)));
      }
    }
  amax = wave_max(amax);
  if (lane == 0) red[w] = amax;

  // stage tile 0
  {
    const uint4* ks = (const uint4*)(Kq + headN * VC_D);
    const uint4* rs = (const uint4*)(Rq + (size_t)bh * T * TILE_BYTES);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = t + 256 * i, row = u >> 3, c16 = u & 7;
      *(uint4*)(&kt[0][swz(row, c16)]) = ks[u];
      *(uint4*)(&rt[0][swz(row, c16)]) = rs[u];
    }
    if (!NO_MEAN && t < 64) {
      const uint32_t mr = *(const uint32_t*)(mu + (size_t)bh * T * VC_D + 2 * t);
      mus[0][2 * t] = bf16_to_f32(mr & 0xFFFFu);
      mus[0][2 * t + 1] = bf16_to_f32(mr >> 16);
    }
  }
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sQ = amax == 0.0f ? 1.0f : amax / 448.0f;
  v8i qf[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t wd[4] = {qraw[c][m].x, qraw[c][m].y, qraw[c][m].z, qraw[c][m].w};
      qf[c][2 * m] = (int)e4m3x4(bf16_to_f32(wd[0] & 0xFFFFu) / sQ, bf16_to_f32(wd[0] >> 16) / sQ,
                                 bf16_to_f32(wd[1] & 0xFFFFu) / sQ, bf16_to_f32(wd[1] >> 16) / sQ);
      qf[c][2 * m + 1] = (int)e4m3x4(bf16_to_f32(wd[2] & 0xFFFFu) / sQ, bf16_to_f32(wd[2] >> 16) / sQ,
                                     bf16_to_f32(wd[3] & 0xFFFFu) / sQ, bf16_to_f32(wd[3] >> 16) / sQ);
    }
  const float qa = L * sQ;

  float m_run = -__builtin_inff(), l_run = 0.0f;
  v16f acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = v16f{};

  for (int j = 0; j < T; ++j) {
    const int cur = j & 1;
    // prefetch tile j+1 into registers (the last iteration re-reads tile T-1 into the idle
    // buffer, which keeps the loop free of branches around the loads)
    const int jn = j + 1 < T ? j + 1 : j;
    uint4 kr[4], rr[4];
    uint32_t mr = 0;
    {
      const uint4* ks = (const uint4*)(Kq + (headN + (size_t)jn * 128) * VC_D);
      const uint4* rs = (const uint4*)(Rq + ((size_t)bh * T + jn) * TILE_BYTES);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kr[i] = ks[t + 256 * i];
        rr[i] = rs[t + 256 * i];
      }
      if (!NO_MEAN && t < 64) mr = *(const uint32_t*)(mu + ((size_t)bh * T + jn) * VC_D + 2 * t);
    }

    // S^T = Kq_j . Qq^T
    v16f s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = v16f{};
#pragma unroll
      for (int c = 0; c < 2; ++c) s[kb] = mfma_fp8(lds_frag32(kt[cur], 32 * kb + q, 4 * c + 2 * g), qf[c], s[kb]);
    }

    // running maximum and the FMA constants of Eq. 7
    const float a = qa * sK[(size_t)bh * T + j];
    float mx = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float xhat = a * mx;
    const float m_new = fmaxf(m_run, xhat);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * 0.125f);
    const float b = 119.65f - m_new;

    // ExpCast: one FMA and one saturating RNE byte conversion per element.  Byte jj of the
    // PV B-operand for key half p is element (kb = 2p + jj/16, i = jj%16) of S^T.
    v8i pw[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int kb = 2 * p + (wd >> 2), i0 = 4 * (wd & 3);
        uint32_t word = 0;
        word = expcast_byte(__builtin_fmaf(a, s[kb][i0 + 0], b), 0, word);
        word = expcast_byte(__builtin_fmaf(a, s[kb][i0 + 1], b), 1, word);
        word = expcast_byte(__builtin_fmaf(a, s[kb][i0 + 2], b), 2, word);
        word = expcast_byte(__builtin_fmaf(a, s[kb][i0 + 3], b), 3, word);
        pw[p][wd] = (int)word;
      }

    // row sum of the decoded codes (the values the PV instruction consumes)
    float r = 0.0f;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(pw[p][wd], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(pw[p][wd], true);
        r += (lo[0] + lo[1]) + (hi[0] + hi[1]);
      }
    r += __shfl_xor(r, 32, 64);
    l_run = alpha * l_run + r;

    // Eq. 6: rescale the numerator and add the rank-one mean term r mu~_j^T
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        if (NO_MEAN) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * ig + e] *= alpha;
        } else {
          const float4 m4 = *(const float4*)(&mus[cur][32 * db + 8 * ig + 4 * g]);
          acc[db][4 * ig + 0] = __builtin_fmaf(r, m4.x, acc[db][4 * ig + 0] * alpha);
          acc[db][4 * ig + 1] = __builtin_fmaf(r, m4.y, acc[db][4 * ig + 1] * alpha);
          acc[db][4 * ig + 2] = __builtin_fmaf(r, m4.z, acc[db][4 * ig + 2] * alpha);
          acc[db][4 * ig + 3] = __builtin_fmaf(r, m4.w, acc[db][4 * ig + 3] * alpha);
        }
      }

    // O^T += Rq_j^T . P^T
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int p = 0; p < 2; ++p) acc[db] = mfma_fp8(lds_frag32(rt[cur], 32 * db + q, 4 * p + 2 * g), pw[p], acc[db]);

    m_run = m_new;

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = t + 256 * i, row = u >> 3, c16 = u & 7;
      *(uint4*)(&kt[cur ^ 1][swz(row, c16)]) = kr[i];
      *(uint4*)(&rt[cur ^ 1][swz(row, c16)]) = rr[i];
    }
    if (!NO_MEAN && t < 64) {
      mus[cur ^ 1][2 * t] = bf16_to_f32(mr & 0xFFFFu);
      mus[cur ^ 1][2 * t + 1] = bf16_to_f32(mr >> 16);
    }
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
