// K smoothing and V block demeaning with E4M3 quantisation, in permuted order
// (VC-Attention Sec. 3.2 Eq. 3-4, "Block demeaning"; App. B, the K and V passes).
//
// Every statistic that feeds a code is reproducible bit for bit: sums of bf16 values are
// taken in float64 (exact for the data here, hence order-free) and rounded to float32 once;
// maxima are exact; x / s is one correctly rounded float32 division; E4M3 rounding is the
// hardware's round-to-nearest-even conversion of a value already inside +-448.
//
// Passes (all grids are (blocks, b*h); 256 or 512 threads = 32 channel quads x 8 or 16 row
// groups):
//   k_kstat_partial  float64 channel sums of K per 1024-row chunk (256 for small shapes)
//   k_kstat_final    kbar = float32(sum / N) in chunk order
//   k_kquant         per 128-row block of K[pi]: K' = K - kbar, sK = 2^E (smallest power of two
//                    with amax <= 448 sK, an E8M0 block scale), codes
//   k_kquant_had     the same with VC_DQ_HADAMARD: the rows K' H (Sylvester H, App. B) are
//                    quantised and sK = 2^(E-7)
//   k_vpass1         per block of V[pi]: mu_j (float64 sum / 128), the block's |R| maxima
//   k_vamax          per-channel maximum over each eighth of the blocks (no atomics)
//   k_vpass2         sV = (maximum of the eight) / 448; codes of R / sV into the tile-transposed
//                    PV operand order;
//                    mu~ = bf16(mu / sV)
//   k_kquant4, k_vquant4   the 4-bit path's K and V operands (MX E2M1, per-32 scales)
//   k_kquant6, k_vquant6   the 6-bit path's (MX E2M3, per-32 scales, 128-byte rows of four groups)
#include "vc_common.h"
#include "vc_internal.h"
#include "vc_attn.h"

// Token at permuted position pos.  An entry outside [0, N) (a caller error; vc_validate_perm
// detects it) is read as token 0, so no gather leaves the head's rows.
__device__ __forceinline__ int dq_token(const int32_t* perm, int bh, int N, int pos) {
  if (!perm) return pos;
  const int t = perm[(size_t)bh * N + pos];
  return (unsigned)t < (unsigned)N ? t : 0;
}

// Four bf16 channels of a row, read with a streaming load: every pass of this file reads each
// K or V row once (the two passes over a tensor are separate launches over all its rows).
__device__ __forceinline__ void load4(const uint16_t* p, float* v) {
  const uint2 raw = ld_stream2(p);
  v[0] = bf16_to_f32(raw.x & 0xFFFFu);
  v[1] = bf16_to_f32(raw.x >> 16);
  v[2] = bf16_to_f32(raw.y & 0xFFFFu);
  v[3] = bf16_to_f32(raw.y >> 16);
}

// Maximum over a 512-thread block (8 waves).
__device__ __forceinline__ float block_max_512(float v, float* red8) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red8[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(fmaxf(red8[0], red8[1]), fmaxf(red8[2], red8[3])),
               fmaxf(fmaxf(red8[4], red8[5]), fmaxf(red8[6], red8[7])));
}

__global__ __launch_bounds__(256) void k_kstat_partial(const uint16_t* __restrict__ K, int N, int nchunk,
                                                       int chunk, double* __restrict__ kpart) {
  __shared__ double part[8][VC_D];
  const int bh = blockIdx.y, ch = blockIdx.x, t = threadIdx.x;
  const int q4 = t & 31, rg = t >> 5;
  double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
  const int r0 = ch * chunk;
  // 64 rows per step, 8 loads in flight per thread; N is a multiple of 64, so a step that
  // starts inside the matrix ends inside it.
  for (int g = 0; g < chunk / 64; ++g) {
    const int rb = r0 + 64 * g + rg;
    if (rb >= N) break;
    float v[8][4];
#pragma unroll
    for (int m = 0; m < 8; ++m) load4(K + ((size_t)bh * N + rb + 8 * m) * VC_D + 4 * q4, v[m]);
#pragma unroll
    for (int m = 0; m < 8; ++m) { a0 += v[m][0]; a1 += v[m][1]; a2 += v[m][2]; a3 += v[m][3]; }
  }
  part[rg][4 * q4 + 0] = a0;
  part[rg][4 * q4 + 1] = a1;
  part[rg][4 * q4 + 2] = a2;
  part[rg][4 * q4 + 3] = a3;
  __syncthreads();
  if (t < VC_D) {
    double s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += part[i][t];
    kpart[((size_t)bh * nchunk + ch) * VC_D + t] = s;
  }
}

__global__ __launch_bounds__(128) void k_kstat_final(const double* __restrict__ kpart, int N, int nchunk,
                                                     float* __restrict__ kbar) {
  const int bh = blockIdx.x, t = threadIdx.x;
  const double* p = kpart + (size_t)bh * nchunk * VC_D + t;
  // eight independent partial sums, so the loads are in flight together (exact either way)
  double a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int c = 0;
  for (; c + 8 <= nchunk; c += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) a[u] += p[(size_t)(c + u) * VC_D];
  for (; c < nchunk; ++c) a[0] += p[(size_t)c * VC_D];
  const double s = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
  kbar[(size_t)bh * VC_D + t] = (float)(s / (double)N);
}

// Rotation of one centred key row by the Sylvester Hadamard matrix H (entries +-1; App. B's K
// pass).  The 32 lanes of a half-wave hold the row, lane q4 the channels 4 q4 .. 4 q4 + 3: channel
// bits 0-1 are local, bits 2-6 are the bits of q4.  The butterflies run in float64, where the
// signed sum of the 128 float32 terms is exact whatever the order, and round to float32 once.
__device__ __forceinline__ void hadamard_k_row(float* x, int q4) {
  double a0 = x[0], a1 = x[1], a2 = x[2], a3 = x[3];
  const double b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
  a0 = b0 + b2;
  a2 = b0 - b2;
  a1 = b1 + b3;
  a3 = b1 - b3;
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) {
    const bool upper = q4 & m;   // this lane holds the partner with channel bit set
    const double o0 = __shfl_xor(a0, m, 64), o1 = __shfl_xor(a1, m, 64);
    const double o2 = __shfl_xor(a2, m, 64), o3 = __shfl_xor(a3, m, 64);
    a0 = upper ? o0 - a0 : a0 + o0;
    a1 = upper ? o1 - a1 : a1 + o1;
    a2 = upper ? o2 - a2 : a2 + o2;
    a3 = upper ? o3 - a3 : a3 + o3;
  }
  x[0] = (float)a0;
  x[1] = (float)a1;
  x[2] = (float)a2;
  x[3] = (float)a3;
}

// 512 threads per 128-row block: thread (q4, rg) takes channels 4 q4 .. 4 q4 + 3 of rows
// rg + 16 i, i < 8 (few registers per thread, so many blocks stream at once).
__global__ __launch_bounds__(512) void k_kquant(const uint16_t* __restrict__ K, const int32_t* __restrict__ perm,
                                                const float* __restrict__ kbar, int N,
                                                uint8_t* __restrict__ Kq, float* __restrict__ sK) {
  __shared__ float red8[8];
  const int bh = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int q4 = t & 31, rg = t >> 5;
  const float4 kb = *(const float4*)(kbar + (size_t)bh * VC_D + 4 * q4);
  float x[8][4];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tok = dq_token(perm, bh, N, j * VC_BLK + rg + 16 * i);
    float v[4];
    load4(K + ((size_t)bh * N + tok) * VC_D + 4 * q4, v);
    x[i][0] = v[0] - kb.x;
    x[i][1] = v[1] - kb.y;
    x[i][2] = v[2] - kb.z;
    x[i][3] = v[3] - kb.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) amax = fmaxf(amax, fabsf(x[i][e]));
  }
  amax = block_max_512(amax, red8);
  const int E = pow2_block_exponent(amax);
  const float inv = __builtin_ldexpf(1.0f, -E);   // exact: the scale is a power of two
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = j * VC_BLK + rg + 16 * i;
    const uint32_t w = e4m3x4(x[i][0] * inv, x[i][1] * inv, x[i][2] * inv, x[i][3] * inv);
    *(uint32_t*)(Kq + ((size_t)bh * N + r) * VC_D + 4 * q4) = w;
  }
  if (t == 0) sK[(size_t)bh * (N / VC_BLK) + j] = __builtin_ldexpf(1.0f, E);
}

// The rotated K pass (VC_DQ_HADAMARD): 4 lanes per row, lane (row, c4) holding channels
// 32 c4 .. 32 c4 + 31 as y[i] (channel bits 0-4 local, bits 5-6 the lane's bits 0-1).  Five
// butterfly stages run in registers and two across the lanes of a quad (DPP quad permutes, no
// LDS traffic).  float64 throughout: the signed sum of the 128 float32 terms is exact whatever
// the order, so each rotated value is float32(exact K' H) and the codes match the oracle bit for
// bit.  The stored scale is 2^(E-7), carrying the 1/128 of H / 128.
__device__ __forceinline__ double dpp_quad_xor(double v, int m) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  int rlo, rhi;
  if (m == 1) {   // quad_perm [1,0,3,2]
    rlo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false);
    rhi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false);
  } else {        // quad_perm [2,3,0,1]
    rlo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false);
    rhi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false);
  }
  return __builtin_bit_cast(double, ((uint64_t)(uint32_t)rhi << 32) | (uint32_t)rlo);
}

// One quarter of a permuted row, channels 32 c4 .. 32 c4 + 31, centred: z = float32(K - kbar).
// With HAD, the quad's four lanes then rotate their row by H (float64 butterflies, as above)
// and z is float32 of the exact rotated value.
template <bool HAD>
__device__ __forceinline__ void centred_quarter_row(const uint16_t* __restrict__ krow, const float* __restrict__ kb,
                                                    int c4, float* z) {
  const uint4* src = (const uint4*)(krow + 32 * c4);
  if constexpr (!HAD) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 raw = src[v];
      const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
      const float4 k0 = *(const float4*)(kb + 8 * v), k1 = *(const float4*)(kb + 8 * v + 4);
      const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[8 * v + 2 * e] = bf16_to_f32(wd[e] & 0xFFFFu) - kk[2 * e];
        z[8 * v + 2 * e + 1] = bf16_to_f32(wd[e] >> 16) - kk[2 * e + 1];
      }
    }
    return;
  }
  double y[32];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint4 raw = src[v];
    const uint32_t wd[4] = {raw.x, raw.y, raw.z, raw.w};
    const float4 k0 = *(const float4*)(kb + 8 * v), k1 = *(const float4*)(kb + 8 * v + 4);
    const float kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[8 * v + 2 * e] = (double)(bf16_to_f32(wd[e] & 0xFFFFu) - kk[2 * e]);       // float32 K' = K - kbar
      y[8 * v + 2 * e + 1] = (double)(bf16_to_f32(wd[e] >> 16) - kk[2 * e + 1]);
    }
  }
#pragma unroll
  for (int b = 1; b < 32; b <<= 1)
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (!(k & b)) {
        const double u = y[k], v = y[k | b];
        y[k] = u + v;
        y[k | b] = u - v;
      }
#pragma unroll
  for (int m = 1; m <= 2; m <<= 1) {
    const bool upper = c4 & m;   // this lane holds the partner with channel bit set
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const double o = dpp_quad_xor(y[k], m);
      y[k] = upper ? o - y[k] : y[k] + o;
    }
  }
#pragma unroll
  for (int k = 0; k < 32; ++k) z[k] = (float)y[k];
}

__global__ __launch_bounds__(512) void k_kquant_had(const uint16_t* __restrict__ K, const int32_t* __restrict__ perm,
                                                    const float* __restrict__ kbar, int N,
                                                    uint8_t* __restrict__ Kq, float* __restrict__ sK) {
  __shared__ float red8[8];
  const int bh = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int row = t >> 2, c4 = t & 3;
  const int tok = dq_token(perm, bh, N, j * VC_BLK + row);
  float z[32];
  centred_quarter_row<true>(K + ((size_t)bh * N + tok) * VC_D, kbar + (size_t)bh * VC_D + 32 * c4, c4, z);
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(z[k]));
  amax = block_max_512(amax, red8);
  const int E = pow2_block_exponent(amax);
  const float inv = __builtin_ldexpf(1.0f, -E);   // exact: the scale is a power of two
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = e4m3x4(z[4 * i] * inv, z[4 * i + 1] * inv, z[4 * i + 2] * inv, z[4 * i + 3] * inv);
  uint4* dst = (uint4*)(Kq + ((size_t)bh * N + j * VC_BLK + row) * VC_D + 32 * c4);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  if (t == 0) sK[(size_t)bh * (N / VC_BLK) + j] = __builtin_ldexpf(1.0f, E - 7);
}

// amax[bh][g][c] = max over tiles j in slice g (of 8) of amaxp[bh][j][c]; 128 threads per
// (slice, b*h), four maxima in flight per thread.
__global__ __launch_bounds__(128) void k_vamax(const float* __restrict__ amaxp, int T, float* __restrict__ amax) {
  const int g = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int j0 = (int)((long long)T * g / 8), j1 = (int)((long long)T * (g + 1) / 8);
  const float* p = amaxp + (size_t)bh * T * VC_D + t;
  float a[4] = {0, 0, 0, 0};
  int j = j0;
  for (; j + 4 <= j1; j += 4)
#pragma unroll
    for (int u = 0; u < 4; ++u) a[u] = fmaxf(a[u], p[(size_t)(j + u) * VC_D]);
  for (; j < j1; ++j) a[0] = fmaxf(a[0], p[(size_t)j * VC_D]);
  amax[((size_t)bh * 8 + g) * VC_D + t] = fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3]));
}

// 512 threads per block: thread (q4, rg) takes channels 4 q4 .. 4 q4 + 3 of rows rg + 16 i.
__global__ __launch_bounds__(512) void k_vpass1(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                int N, int demean, float* __restrict__ mu,
                                                float* __restrict__ amaxp) {
  __shared__ double part[16][VC_D];
  __shared__ float mus[VC_D];
  __shared__ float mx[16][VC_D];
  const int bh = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int q4 = t & 31, rg = t >> 5;
  float x[8][4];
  double a0 = 0, a1 = 0, a2 = 0, a3 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int tok = dq_token(perm, bh, N, j * VC_BLK + rg + 16 * i);
    load4(V + ((size_t)bh * N + tok) * VC_D + 4 * q4, x[i]);
    a0 += x[i][0]; a1 += x[i][1]; a2 += x[i][2]; a3 += x[i][3];
  }
  part[rg][4 * q4 + 0] = a0;
  part[rg][4 * q4 + 1] = a1;
  part[rg][4 * q4 + 2] = a2;
  part[rg][4 * q4 + 3] = a3;
  __syncthreads();
  if (t < VC_D) {
    double s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += part[i][t];
    const float m = demean ? (float)(s / 128.0) : 0.0f;
    mus[t] = m;
    mu[((size_t)bh * (N / VC_BLK) + j) * VC_D + t] = m;
  }
  __syncthreads();
  float m[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) m[e] = 0.0f;
  const float4 mv = *(const float4*)(mus + 4 * q4);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m[0] = fmaxf(m[0], fabsf(x[i][0] - mv.x));
    m[1] = fmaxf(m[1], fabsf(x[i][1] - mv.y));
    m[2] = fmaxf(m[2], fabsf(x[i][2] - mv.z));
    m[3] = fmaxf(m[3], fabsf(x[i][3] - mv.w));
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) mx[rg][4 * q4 + e] = m[e];
  __syncthreads();
  if (t < VC_D) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, mx[i][t]);
    amaxp[((size_t)bh * (N / VC_BLK) + j) * VC_D + t] = a;
  }
}

// Position of permuted row r (0..127) of a tile in the PV operand order of vc_attn_fwd:
// slot s = 64 p + 32 g + i holds key(s) = 64 p + 32 (i/16) + 8 ((i%16)/4) + 4 g + (i%4).
__device__ __forceinline__ int pv_slot_of_key(int r) {
  const int p = r >> 6, ih = (r >> 5) & 1, b8 = (r >> 3) & 3, g = (r >> 2) & 1, i4 = r & 3;
  return 64 * p + 32 * g + 16 * ih + 4 * b8 + i4;
}

constexpr int TILE_ROW = 132;   // LDS bytes per channel row of the transposed tile (128 + pad)

__global__ __launch_bounds__(256) void k_vpass2(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                int N, const float* __restrict__ mu,
                                                const float* __restrict__ amax,
                                                uint8_t* __restrict__ Rq, uint16_t* __restrict__ mu_out,
                                                float* __restrict__ sV) {
  __shared__ float sc[VC_D];
  __shared__ float mus[VC_D];
  __shared__ __attribute__((aligned(16))) uint8_t tile[VC_D * TILE_ROW];
  const int bh = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int q4 = t & 31, rg = t >> 5;
  const int nt = N / VC_BLK;
  if (t < VC_D) {
    float a = 0.0f;
#pragma unroll
    for (int g = 0; g < 8; ++g) a = fmaxf(a, amax[((size_t)bh * 8 + g) * VC_D + t]);
    const float s = a == 0.0f ? 1.0f : a / 448.0f;
    const float m = mu[((size_t)bh * nt + j) * VC_D + t];
    sc[t] = s;
    mus[t] = m;
    mu_out[((size_t)bh * nt + j) * VC_D + t] = (uint16_t)f32_to_bf16_rne(m / s);
    if (j == 0) sV[(size_t)bh * VC_D + t] = s;
  }
  __syncthreads();
  const float4 s4 = *(const float4*)(sc + 4 * q4);
  const float4 m4 = *(const float4*)(mus + 4 * q4);
  // R / sV correctly rounded, as the float32 division the definition uses, from the channel's
  // reciprocal y = RN(1 / sV) (one true division per channel instead of one per element):
  // q1 = RN(x y) corrected once, q1 + RN(x - sV q1) y, is within one ulp of x / sV, and a second
  // correction from an exact FMA residual then gives RN(x / sV) (Markstein's theorem: y within
  // half an ulp of 1 / sV, q1 within one ulp of x / sV, no underflow or overflow; the quotients
  // here lie in [-448, 448] and the residuals are far from the subnormal range).
  const float4 y4 = make_float4(1.0f / s4.x, 1.0f / s4.y, 1.0f / s4.z, 1.0f / s4.w);
  auto qdiv = [](float x, float sv, float y) {
    float q = x * y;
    q = fmaf(fmaf(-q, sv, x), y, q);
    return fmaf(fmaf(-q, sv, x), y, q);
  };
  // Thread (q4, rg) takes the 4-row groups rg, rg+8, rg+16, rg+24 of the tile and channels
  // 4 q4 .. 4 q4 + 3.  The rows 4 G .. 4 G + 3 of a group land in 4 consecutive PV slots, so
  // each channel's four codes form one 32-bit word of the transposed tile.
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r0 = 4 * (rg + 8 * k);
    uint32_t wc[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int tok = dq_token(perm, bh, N, j * VC_BLK + r0 + i4);
      float v[4];
      load4(V + ((size_t)bh * N + tok) * VC_D + 4 * q4, v);
      const uint32_t w = e4m3x4(qdiv(v[0] - m4.x, s4.x, y4.x), qdiv(v[1] - m4.y, s4.y, y4.y),
                                qdiv(v[2] - m4.z, s4.z, y4.z), qdiv(v[3] - m4.w, s4.w, y4.w));
#pragma unroll
      for (int e = 0; e < 4; ++e) wc[e] |= ((w >> (8 * e)) & 0xFFu) << (8 * i4);
    }
    const int slot0 = pv_slot_of_key(r0);   // a multiple of 4
#pragma unroll
    for (int e = 0; e < 4; ++e) *(uint32_t*)(tile + (4 * q4 + e) * TILE_ROW + slot0) = wc[e];
  }
  __syncthreads();
  // copy the 128 x 128 bytes out, one 32-bit word per lane (consecutive lanes, consecutive words)
  uint32_t* dst = (uint32_t*)(Rq + ((size_t)bh * nt + j) * (VC_D * VC_BLK));
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int wi = t + 256 * i, c = wi >> 5, x = wi & 31;
    dst[wi] = *(const uint32_t*)(tile + c * TILE_ROW + 4 * x);
  }
}

// ---- 4-bit path (MX E2M1 with per-32 E8M0 scales; the analogue of the pages' NVFP4 value
// quantiser, Sec. 3.2 after Eq. 4, App. B) ----

// K: per permuted row and 32-channel group, E = mx_exponent(amax), codes E2M1(x / 2^E) packed
// two per byte (even channel in the low nibble), scale byte E + 127 (E - 7 + 127 with the
// rotation, whose H / 128 rides on the scale).  Thread (q4, rg) takes channels 4 q4 .. 4 q4 + 3
// of rows rg + 8 i; the eight lanes q4 = 8 G .. 8 G + 7 hold group G of a row.
// One row's group scale and codes (see k_kquant4).
template <bool HAD>
__device__ __forceinline__ void kquant4_row(const float* x, int q4, size_t row, uint8_t* __restrict__ Kq4,
                                            uint8_t* __restrict__ sK4) {
  float a = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
  a = fmaxf(a, __shfl_xor(a, 1, 64));
  a = fmaxf(a, __shfl_xor(a, 2, 64));
  a = fmaxf(a, __shfl_xor(a, 4, 64));
  const int E = mx_exponent(a);
  const float inv = __builtin_ldexpf(1.0f, -E);   // exact
  uint32_t w = fp4x2<0>(0u, x[0] * inv, x[1] * inv);
  w = fp4x2<1>(w, x[2] * inv, x[3] * inv);
  *(uint16_t*)(Kq4 + row * (VC_D / 2) + 2 * q4) = (uint16_t)w;
  if ((q4 & 7) == 0) sK4[row * 4 + (q4 >> 3)] = (uint8_t)(E - (HAD ? 7 : 0) + 127);
}

template <bool HAD>
__global__ __launch_bounds__(256) void k_kquant4(const uint16_t* __restrict__ K, const int32_t* __restrict__ perm,
                                                 const float* __restrict__ kbar, int N,
                                                 uint8_t* __restrict__ Kq4, uint8_t* __restrict__ sK4) {
  const int bh = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int q4 = t & 31, rg = t >> 5;
  const float4 kb = *(const float4*)(kbar + (size_t)bh * VC_D + 4 * q4);
  float x[16][4];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tok = dq_token(perm, bh, N, j * VC_BLK + rg + 8 * i);
    float v[4];
    load4(K + ((size_t)bh * N + tok) * VC_D + 4 * q4, v);
    x[i][0] = v[0] - kb.x;
    x[i][1] = v[1] - kb.y;
    x[i][2] = v[2] - kb.z;
    x[i][3] = v[3] - kb.w;
  }
  const size_t row0 = (size_t)bh * N + j * VC_BLK + rg;
#pragma unroll
  for (int i = 0; i < 16; i += 2) {
    if constexpr (HAD) {   // two rows per scheduling region (32 lanes per row)
      hadamard_k_row(x[i], q4);
      hadamard_k_row(x[i + 1], q4);
    }
    kquant4_row<HAD>(x[i], q4, row0 + 8 * i, Kq4, sK4);
    kquant4_row<HAD>(x[i + 1], q4, row0 + 8 * (i + 1), Kq4, sK4);
    if constexpr (HAD) __builtin_amdgcn_sched_barrier(0);
  }
}

constexpr int TILE4_ROW = 72;   // LDS bytes per channel row of a 4-bit transposed tile (64 + pad)

// V: per tile j and channel, the residual R = V'[pi] - mu_j in MX E2M1 over each 32-key group
// (keys of one 64-key half with equal index bit 2, i.e. the slots 32 g .. 32 g + 31 of the PV
// operand order), tile-transposed [channel][slot] two slots per byte; scale bytes
// [channel][group]; mu_out = bf16(mu_j) unscaled (App. B: at 4 bits the microscales act
// inside the matrix instruction).  Thread (q4, sub, g) takes channels 4 q4 .. 4 q4 + 3 and the
// 16 rows 64 (g/2) + 8 a + 4 (g%2) + i4, a = 4 sub .. 4 sub + 3: slots 32 g + 16 sub + 4 (a - 4 sub)
// + i4.  Its partner for the group maximum is lane ^ 32 (same wave, other sub).
__global__ __launch_bounds__(256) void k_vquant4(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                 int N, const float* __restrict__ mu,
                                                 uint8_t* __restrict__ Rq4, uint8_t* __restrict__ sR4,
                                                 uint16_t* __restrict__ mu_out) {
  __shared__ float mus[VC_D];
  __shared__ __attribute__((aligned(16))) uint8_t tile[VC_D * TILE4_ROW];
  __shared__ __attribute__((aligned(16))) uint8_t stile[VC_D * 4];
  const int bh = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int q4 = t & 31, sub = (t >> 5) & 1, g = t >> 6;
  const int nt = N / VC_BLK;
  if (t < VC_D) {
    const float m = mu[((size_t)bh * nt + j) * VC_D + t];
    mus[t] = m;
    mu_out[((size_t)bh * nt + j) * VC_D + t] = (uint16_t)f32_to_bf16_rne(m);
  }
  __syncthreads();
  const float4 m4 = *(const float4*)(mus + 4 * q4);
  float x[16][4];
#pragma unroll
  for (int aa = 0; aa < 4; ++aa)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int r = 64 * (g >> 1) + 8 * (4 * sub + aa) + 4 * (g & 1) + i4;
      const int tok = dq_token(perm, bh, N, j * VC_BLK + r);
      float v[4];
      load4(V + ((size_t)bh * N + tok) * VC_D + 4 * q4, v);
      float* xi = x[4 * aa + i4];
      xi[0] = v[0] - m4.x;
      xi[1] = v[1] - m4.y;
      xi[2] = v[2] - m4.z;
      xi[3] = v[3] - m4.w;
    }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(x[i][e]));
    a = fmaxf(a, __shfl_xor(a, 32, 64));
    const int E = mx_exponent(a);
    const float inv = __builtin_ldexpf(1.0f, -E);
    uint32_t w0 = 0u, w1 = 0u;
    w0 = fp4x2<0>(w0, x[0][e] * inv, x[1][e] * inv);
    w0 = fp4x2<1>(w0, x[2][e] * inv, x[3][e] * inv);
    w0 = fp4x2<2>(w0, x[4][e] * inv, x[5][e] * inv);
    w0 = fp4x2<3>(w0, x[6][e] * inv, x[7][e] * inv);
    w1 = fp4x2<0>(w1, x[8][e] * inv, x[9][e] * inv);
    w1 = fp4x2<1>(w1, x[10][e] * inv, x[11][e] * inv);
    w1 = fp4x2<2>(w1, x[12][e] * inv, x[13][e] * inv);
    w1 = fp4x2<3>(w1, x[14][e] * inv, x[15][e] * inv);
    *(uint2*)(tile + (4 * q4 + e) * TILE4_ROW + 16 * g + 8 * sub) = make_uint2(w0, w1);
    if (sub == 0) stile[(4 * q4 + e) * 4 + g] = (uint8_t)(E + 127);
  }
  __syncthreads();
  uint8_t* dst = Rq4 + ((size_t)bh * nt + j) * (VC_D * VC_BLK / 2);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int c = t + 256 * k, ch = c >> 2, part = c & 3;
    const uint2 lo = *(const uint2*)(tile + ch * TILE4_ROW + 16 * part);
    const uint2 hi = *(const uint2*)(tile + ch * TILE4_ROW + 16 * part + 8);
    *(uint4*)(dst + 16 * c) = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  if (t < VC_D) ((uint32_t*)(sR4 + ((size_t)bh * nt + j) * (VC_D * 4)))[t] = ((const uint32_t*)stile)[t];
}

// Group g (0..3) of a 6-bit row of 128 bytes: its first 16 code bytes at 16 g, its last 8 at
// 64 + 16 (g % 2) + 8 (g / 2) (groups 0 and 2 share chunk 4, groups 1 and 3 chunk 5, so an
// attention lane reads the tails of both its groups in one 16-byte read), and 8 of the row's 32
// trailing zero bytes at 96 + 8 g.
__device__ __forceinline__ void fp6_row_store(uint8_t* row, int g, const v6i& w) {
  *(uint4*)(row + 16 * g) = make_uint4((uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]);
  *(uint2*)(row + 64 + 16 * (g & 1) + 8 * (g >> 1)) = make_uint2((uint32_t)w[4], (uint32_t)w[5]);
  *(uint2*)(row + 96 + 8 * g) = make_uint2(0u, 0u);
}

// 6-bit K (MX E2M3): four lanes per permuted row, lane (row, c4) quantising channels
// 32 c4 .. 32 c4 + 31, one scale group: its own maximum, E = mx6_exponent, codes of z / 2^E
// (exact division) packed into 24 bytes and stored as group c4 of the row (fp6_row_store, the
// layout the 6-bit attention's fragments read).  With HAD the row is rotated first and the
// stored exponent lowered by 7 (the 1/128 of H / 128).
template <bool HAD>
__global__ __launch_bounds__(512) void k_kquant6(const uint16_t* __restrict__ K, const int32_t* __restrict__ perm,
                                                 const float* __restrict__ kbar, int N,
                                                 uint8_t* __restrict__ Kq6, uint8_t* __restrict__ sK6) {
  const int bh = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int row = t >> 2, c4 = t & 3;
  const int tok = dq_token(perm, bh, N, j * VC_BLK + row);
  float z[32];
  centred_quarter_row<HAD>(K + ((size_t)bh * N + tok) * VC_D, kbar + (size_t)bh * VC_D + 32 * c4, c4, z);
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(z[k]));
  const int E = mx6_exponent(amax);
  const float inv = __builtin_ldexpf(1.0f, -E);   // exact
#pragma unroll
  for (int k = 0; k < 32; ++k) z[k] *= inv;
  const v6i w = fp6x32(z);
  const size_t r = (size_t)bh * N + j * VC_BLK + row;
  fp6_row_store(Kq6 + r * VC_D, c4, w);
  sK6[r * 4 + c4] = (uint8_t)(E - (HAD ? 7 : 0) + 127);
}

// Slot of permuted row r (0..127) of a tile in the PV operand order: row 64 p + 32 hi + 8 mid
// + 4 g + lo sits in slot 64 p + 32 g + 16 hi + 4 mid + lo.
__device__ __forceinline__ int pv_slot(int r) {
  return (r & 64) + 32 * ((r >> 2) & 1) + 16 * ((r >> 5) & 1) + 4 * ((r >> 3) & 3) + (r & 3);
}

// 6-bit V residual (MX E2M3), per tile j: the gathered rows V'[pi] staged in LDS as bf16 in
// slot order [slot][channel] (a thread copies four channels of one row); then thread
// (channel pair, group) takes the 32 slots of its group for both channels, R = V' - mu_j in
// float32, each channel's maximum and scale, and writes its two 24-code-byte groups into the
// channels' 128-byte rows of the tile-transposed operand (fp6_row_store); scale bytes [channel][group];
// mu_out = bf16(mu_j), unscaled.
constexpr int V6_OROW = 144;   // LDS bytes per channel row of the 6-bit output tile (128 + pad)

__global__ __launch_bounds__(256) void k_vquant6(const uint16_t* __restrict__ V, const int32_t* __restrict__ perm,
                                                 int N, const float* __restrict__ mu,
                                                 uint8_t* __restrict__ Rq6, uint8_t* __restrict__ sR6,
                                                 uint16_t* __restrict__ mu_out) {
  __shared__ float mus[VC_D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[VC_BLK * VC_D];
  const int bh = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  const int q4 = t & 31, rg = t >> 5;
  const int nt = N / VC_BLK;
  const size_t tile = (size_t)bh * nt + j;
  if (t < VC_D) {
    const float m = mu[tile * VC_D + t];
    mus[t] = m;
    mu_out[tile * VC_D + t] = (uint16_t)f32_to_bf16_rne(m);
  }
  uint2 raw[16];   // all sixteen gathered loads in flight before any LDS write
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int tok = dq_token(perm, bh, N, j * VC_BLK + rg + 8 * i);
    raw[i] = ld_stream2(V + ((size_t)bh * N + tok) * VC_D + 4 * q4);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) *(uint2*)(vs + pv_slot(rg + 8 * i) * VC_D + 4 * q4) = raw[i];
  __syncthreads();
  const int c2 = t & 63, g = t >> 6;
  const float m0 = mus[2 * c2], m1 = mus[2 * c2 + 1];
  float x0[32], x1[32];
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t w = *(const uint32_t*)(vs + (32 * g + i) * VC_D + 2 * c2);
    x0[i] = bf16_to_f32(w & 0xFFFFu) - m0;
    x1[i] = bf16_to_f32(w >> 16) - m1;
    a0 = fmaxf(a0, fabsf(x0[i]));
    a1 = fmaxf(a1, fabsf(x1[i]));
  }
  const int E0 = mx6_exponent(a0), E1 = mx6_exponent(a1);
  const float i0 = __builtin_ldexpf(1.0f, -E0), i1 = __builtin_ldexpf(1.0f, -E1);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    x0[i] *= i0;
    x1[i] *= i1;
  }
  const v6i w0 = fp6x32(x0), w1 = fp6x32(x1);
  // the codes go through LDS (rows padded to 144 bytes) so the tile leaves as one contiguous
  // 16 KB copy rather than 32-byte pieces of 128 rows
  __syncthreads();   // every read of vs is done
  uint8_t* ot = (uint8_t*)vs;
  fp6_row_store(ot + (2 * c2) * V6_OROW, g, w0);
  fp6_row_store(ot + (2 * c2 + 1) * V6_OROW, g, w1);
  uint8_t* sc = (uint8_t*)(ot + VC_D * V6_OROW);
  sc[(2 * c2) * 4 + g] = (uint8_t)(E0 + 127);
  sc[(2 * c2 + 1) * 4 + g] = (uint8_t)(E1 + 127);
  __syncthreads();
  uint8_t* dst = Rq6 + tile * VC_D * VC_BLK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = t + 256 * i, row = c >> 3, part = c & 7;   // 16-byte chunk c of the 16 KB tile
    *(uint4*)(dst + 16 * c) = *(const uint4*)(ot + row * V6_OROW + 16 * part);
  }
  if (t < VC_D) ((uint32_t*)(sR6 + tile * VC_D * 4))[t] = ((const uint32_t*)sc)[t];
}

hipError_t vc_launch_demean_quant_mx6(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                      int BH, int N, unsigned flags, uint8_t* Kq6, uint8_t* sK6,
                                      uint8_t* Rq6, uint8_t* sR6, uint16_t* mu_out, char* ws,
                                      const vc_dq_ws& L, hipStream_t s) {
  const int chunk = vc_kstat_chunk(BH, N);
  const int nchunk = (N + chunk - 1) / chunk;
  const int nt = N / VC_BLK;
  double* kpart = (double*)(ws + L.kpart);
  float* kbar = (float*)(ws + L.kbar);
  float* mu = (float*)(ws + L.mu);
  float* amaxp = (float*)(ws + L.amaxp);
  hipLaunchKernelGGL(k_kstat_partial, dim3(nchunk, BH), dim3(256), 0, s, K, N, nchunk, chunk, kpart);
  hipLaunchKernelGGL(k_kstat_final, dim3(BH), dim3(128), 0, s, (const double*)kpart, N, nchunk, kbar);
  if (flags & VC_DQ_HADAMARD)
    hipLaunchKernelGGL(k_kquant6<true>, dim3(nt, BH), dim3(512), 0, s, K, perm, (const float*)kbar, N, Kq6, sK6);
  else
    hipLaunchKernelGGL(k_kquant6<false>, dim3(nt, BH), dim3(512), 0, s, K, perm, (const float*)kbar, N, Kq6, sK6);
  hipLaunchKernelGGL(k_vpass1, dim3(nt, BH), dim3(512), 0, s, V, perm, N,
                     (flags & VC_DQ_NO_DEMEAN) ? 0 : 1, mu, amaxp);
  hipLaunchKernelGGL(k_vquant6, dim3(nt, BH), dim3(256), 0, s, V, perm, N, (const float*)mu, Rq6, sR6, mu_out);
  return hipGetLastError();
}

hipError_t vc_launch_demean_quant_mx4(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                      int BH, int N, unsigned flags, uint8_t* Kq4, uint8_t* sK4,
                                      uint8_t* Rq4, uint8_t* sR4, uint16_t* mu_out, char* ws,
                                      const vc_dq_ws& L, hipStream_t s) {
  const int chunk = vc_kstat_chunk(BH, N);
  const int nchunk = (N + chunk - 1) / chunk;
  const int nt = N / VC_BLK;
  double* kpart = (double*)(ws + L.kpart);
  float* kbar = (float*)(ws + L.kbar);
  float* mu = (float*)(ws + L.mu);
  float* amaxp = (float*)(ws + L.amaxp);
  hipLaunchKernelGGL(k_kstat_partial, dim3(nchunk, BH), dim3(256), 0, s, K, N, nchunk, chunk, kpart);
  hipLaunchKernelGGL(k_kstat_final, dim3(BH), dim3(128), 0, s, (const double*)kpart, N, nchunk, kbar);
  if (flags & VC_DQ_HADAMARD)
    hipLaunchKernelGGL(k_kquant4<true>, dim3(nt, BH), dim3(256), 0, s, K, perm, (const float*)kbar, N, Kq4, sK4);
  else
    hipLaunchKernelGGL(k_kquant4<false>, dim3(nt, BH), dim3(256), 0, s, K, perm, (const float*)kbar, N, Kq4, sK4);
  // the block means (the per-tile maxima it also writes are not used at 4 bits)
  hipLaunchKernelGGL(k_vpass1, dim3(nt, BH), dim3(512), 0, s, V, perm, N,
                     (flags & VC_DQ_NO_DEMEAN) ? 0 : 1, mu, amaxp);
  hipLaunchKernelGGL(k_vquant4, dim3(nt, BH), dim3(256), 0, s, V, perm, N, (const float*)mu, Rq4, sR4, mu_out);
  return hipGetLastError();
}

hipError_t vc_launch_demean_quant(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                  int BH, int N, unsigned flags, uint8_t* Kq, float* sK,
                                  uint8_t* Rq, uint16_t* mu_out, float* sV, char* ws,
                                  const vc_dq_ws& L, hipStream_t s) {
  const int chunk = vc_kstat_chunk(BH, N);
  const int nchunk = (N + chunk - 1) / chunk;
  const int nt = N / VC_BLK;
  double* kpart = (double*)(ws + L.kpart);
  float* kbar = (float*)(ws + L.kbar);
  float* mu = (float*)(ws + L.mu);
  float* amaxp = (float*)(ws + L.amaxp);
  hipLaunchKernelGGL(k_kstat_partial, dim3(nchunk, BH), dim3(256), 0, s, K, N, nchunk, chunk, kpart);
  hipLaunchKernelGGL(k_kstat_final, dim3(BH), dim3(128), 0, s, (const double*)kpart, N, nchunk, kbar);
  if (flags & VC_DQ_HADAMARD)
    hipLaunchKernelGGL(k_kquant_had, dim3(nt, BH), dim3(512), 0, s, K, perm, (const float*)kbar, N, Kq, sK);
  else
    hipLaunchKernelGGL(k_kquant, dim3(nt, BH), dim3(512), 0, s, K, perm, (const float*)kbar, N, Kq, sK);
  float* amax = (float*)(ws + L.amax);
  hipLaunchKernelGGL(k_vpass1, dim3(nt, BH), dim3(512), 0, s, V, perm, N,
                     (flags & VC_DQ_NO_DEMEAN) ? 0 : 1, mu, amaxp);
  hipLaunchKernelGGL(k_vamax, dim3(8, BH), dim3(128), 0, s, (const float*)amaxp, nt, amax);
  hipLaunchKernelGGL(k_vpass2, dim3(nt, BH), dim3(256), 0, s, V, perm, N, (const float*)mu,
                     (const float*)amax, Rq, mu_out, sV);
  return hipGetLastError();
}
