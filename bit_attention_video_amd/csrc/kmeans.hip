// k-means grouping of value tokens (VC-Attention Sec. 3.2, "Value-guided permutation").
//
// Batch Lloyd per (b, h):
//   init      c_c = V[floor((c + 1/2) N / k)] (float32)
//   assign    z_t = argmin_c ||v_t - c_c||^2, ties to the lowest c, taken as the argmax of
//             v.c - ||c||^2 / 2 (the same order: ||v - c||^2 = ||v||^2 - 2 (v.c - ||c||^2/2)).
//             The products run on the bf16 matrix cores: v is exactly bf16, c is split into
//             bf16 hi + lo parts (16 significant bits), the accumulator starts from
//             -||c||^2 / 2 and the MFMAs add v.c in float32; each lane keeps the best of its 16
//             centroids per block, one cross-lane exchange finishes.  The split centroids and
//             -||c||^2 / 2 are computed once per (b, h) and round (by a prep kernel for the first
//             round, by the previous round's update afterwards); every assign workgroup copies
//             them into LDS and also counts its labels for the label sort (a workgroup's tokens,
//             1024 or for small shapes 256, are one sort tile).  Two centroid blocks are
//             processed together so that consecutive products belong to independent chains, and
//             each block's best candidate comes from a depth-4 comparison tree.
//   update    c_c = float32(sum of its rows / count), the sum in float64 in a fixed order over
//             the rows of cluster c in sorted order (perm, offsets from the label sort); an
//             empty cluster keeps its centroid.
//   objective J = sum_t ||v_t - c_{z_t}||^2 with the final labels and centroids, taken in the
//             last update from its own sums: per cluster, sum ||v||^2 - 2 c.S + n ||c||^2 with
//             S the exact float64 row sum and c the stored float32 centroid (no extra pass over
//             V), then summed over the clusters in index order.
#include "vc_common.h"
#include "vc_internal.h"
#include "vc_attn.h"

#include <atomic>

constexpr int KM_THREADS = 512;  // assign workgroup size
constexpr int KM_ROW = 136;      // LDS row stride in bf16: 128 + 8 pad = 272 bytes

__global__ __launch_bounds__(128) void k_kmeans_init(const uint16_t* __restrict__ V, int N, int k,
                                                     float* __restrict__ C) {
  const int c = blockIdx.x, bh = blockIdx.y, e = threadIdx.x;
  const long long row = ((2LL * c + 1) * N) / (2LL * k);
  C[((size_t)bh * k + c) * VC_D + e] = bf16_to_f32(V[((size_t)bh * N + row) * VC_D + e]);
}

// Centroids as bf16 hi + lo rows [kpad][128] and -||c||^2 / 2 (float32, the squares summed over
// the channels in order; padding rows get -inf so they never win).
__global__ __launch_bounds__(128) void k_kmeans_prep(const float* __restrict__ C, int k, int kpad,
                                                     uint16_t* __restrict__ chi, uint16_t* __restrict__ clo,
                                                     float* __restrict__ cn) {
  const int c = blockIdx.x, bh = blockIdx.y, e = threadIdx.x;
  const size_t o = ((size_t)bh * kpad + c) * VC_D + e;
  if (c >= k) {   // padding row (uniform per block)
    chi[o] = 0;
    clo[o] = 0;
    if (e == 0) cn[(size_t)bh * kpad + c] = -__builtin_inff();
    return;
  }
  const float* crow = C + ((size_t)bh * k + c) * VC_D;
  const float x = crow[e];
  const uint32_t hi = f32_to_bf16_rne(x);
  const uint32_t lo = f32_to_bf16_rne(x - bf16_to_f32(hi));
  chi[o] = (uint16_t)hi;
  clo[o] = (uint16_t)lo;
  if (e == 0) {
    float s = 0.0f;
    for (int i = 0; i < VC_D; ++i) s = fmaf(crow[i], crow[i], s);
    cn[(size_t)bh * kpad + c] = -0.5f * s;
  }
}

// TOK tokens per workgroup (8 waves x TOK/(256 NSET) groups x NSET sets of 32): one label-sort tile.
// The 1024-token tile takes two sets per wave without prefetch: each centroid fragment read from
// LDS then feeds two products, and the kernel keeps four waves per SIMD (126 registers).  One set
// with the next group prefetched reads twice the LDS bytes per token; two sets with prefetch need
// 194 registers (two waves per SIMD), and four sets 220; at the video and long sizes the chosen
// form is 2-4 % faster over the whole grouping than either, with the same labels.
template <int TOK, int NSET, bool PF>
__global__ __launch_bounds__(512) void k_kmeans_assign(const uint16_t* __restrict__ V,
                                                       const uint16_t* __restrict__ phi,
                                                       const uint16_t* __restrict__ plo,
                                                       const float* __restrict__ pcn, int N, int kpad,
                                                       int32_t* __restrict__ labels,
                                                       float* __restrict__ mindist,
                                                       int32_t* __restrict__ hist) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int hcount[256];   // this tile's label histogram (the label sort's first pass)
  uint16_t* chi = (uint16_t*)smem;                     // [kpad][KM_ROW]
  uint16_t* clo = chi + (size_t)kpad * KM_ROW;         // [kpad][KM_ROW]
  float* cn = (float*)(clo + (size_t)kpad * KM_ROW);   // [kpad]
  const int bh = blockIdx.y, t = threadIdx.x;

  // copy the prepared centroids into the padded LDS rows (16-byte chunks)
  const uint4* ghi = (const uint4*)(phi + (size_t)bh * kpad * VC_D);
  const uint4* glo = (const uint4*)(plo + (size_t)bh * kpad * VC_D);
  for (int i = t; i < kpad * (VC_D / 8); i += KM_THREADS) {
    const int c = i >> 4, ch = i & 15;
    *(uint4*)(chi + c * KM_ROW + 8 * ch) = ghi[i];
    *(uint4*)(clo + c * KM_ROW + 8 * ch) = glo[i];
  }
  for (int c = t; c < kpad; c += KM_THREADS) cn[c] = pcn[(size_t)bh * kpad + c];
  if (t < 256) hcount[t] = 0;
  __syncthreads();

  // Each wave takes NSET sets of 32 tokens per group (lane (q, g): token q of every set, channel
  // half g of every 16-channel chunk); with PF the rows of the next group are loaded while the
  // current one is computed.  Token indices past N are clamped (their labels are not written).
  constexpr int SET = KM_THREADS / 2, NG = TOK / (SET * NSET);
  const int w = t >> 6, lane = t & 63, q = lane & 31, g = lane >> 5;
  const int nblk = kpad >> 5;
  const uint16_t* Vb = V + (size_t)bh * N * VC_D + 8 * g;
  auto tok_of = [&](int grp, int u) { return blockIdx.x * TOK + (grp * NSET + u) * SET + w * 32 + q; };
  auto load_rows = [&](int grp, v8s (&vb)[NSET][8]) {
#pragma unroll
    for (int u = 0; u < NSET; ++u) {
      const int tok = tok_of(grp, u);
      const uint16_t* vrow = Vb + (size_t)(tok < N ? tok : N - 1) * VC_D;
#pragma unroll
      for (int c = 0; c < 8; ++c) vb[u][c] = __builtin_bit_cast(v8s, *(const uint4*)(vrow + 16 * c));
    }
  };
  // Block cb's accumulator starts from -||c||^2 / 2 of this lane's 16 candidates,
  // ci = 32 cb + 8 m + 4 g + r in element 4 m + r.
  auto init = [&](int cb) {
    v16f a;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float4 n4 = *(const float4*)(cn + cb * 32 + 8 * m + 4 * g);
      a[4 * m + 0] = n4.x; a[4 * m + 1] = n4.y; a[4 * m + 2] = n4.z; a[4 * m + 3] = n4.w;
    }
    return a;
  };
  auto frag = [&](const uint16_t* tab, int cb, int c) {
    return __builtin_bit_cast(v8bf, *(const v8s*)(tab + (cb * 32 + q) * KM_ROW + 8 * g + 16 * c));
  };
  // The best of a block's 16 candidates by a depth-4 tree in which the higher-index side wins
  // only when strictly larger: the maximum, and among equal maxima the lowest candidate, as a
  // scan in index order finds (for finite distances).  Then merged into the running best,
  // the blocks taken in index order.
  auto block_best = [&](const v16f& a, int cb, float& best, int& bi) {
    float v[8];
    int e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool gt = a[2 * i + 1] > a[2 * i];
      v[i] = gt ? a[2 * i + 1] : a[2 * i];
      e[i] = gt ? 2 * i + 1 : 2 * i;
    }
#pragma unroll
    for (int n = 4; n >= 1; n >>= 1)
#pragma unroll
      for (int i = 0; i < n; ++i) {
        const bool gt = v[2 * i + 1] > v[2 * i];
        v[i] = gt ? v[2 * i + 1] : v[2 * i];
        e[i] = gt ? e[2 * i + 1] : e[2 * i];
      }
    if (v[0] > best) {
      best = v[0];
      bi = cb * 32 + 4 * g + e[0] + 4 * (e[0] >> 2);   // element 4 m + r -> 8 m + 4 g + r
    }
  };
  v8s vcur[NSET][8], vnext[PF ? NSET : 1][8];
  load_rows(0, vcur);
#pragma unroll
  for (int grp = 0; grp < NG; ++grp) {
    if constexpr (PF)
      if (grp + 1 < NG) load_rows(grp + 1, vnext);
    float best[NSET];   // max of v.c - ||c||^2 / 2
    int bi[NSET];
#pragma unroll
    for (int u = 0; u < NSET; ++u) { best[u] = -__builtin_inff(); bi[u] = 0; }
    // Each block's own sum runs in the same order (-||c||^2/2, then hi and lo of chunk 0, hi and
    // lo of chunk 1, ...).  With one set, two blocks at a time: their product chains are
    // independent, so the matrix unit never waits for the previous product of the same chain;
    // with two sets, the sets' chains are the independent pair and each centroid fragment read
    // from LDS feeds both.
    if constexpr (NSET == 1) {
      int cb = 0;
      for (; cb + 1 < nblk; cb += 2) {
        v16f a0 = init(cb), a1 = init(cb + 1);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const v8bf b = __builtin_bit_cast(v8bf, vcur[0][c]);
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(chi, cb, c), b, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(chi, cb + 1, c), b, a1, 0, 0, 0);
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(clo, cb, c), b, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(clo, cb + 1, c), b, a1, 0, 0, 0);
        }
        block_best(a0, cb, best[0], bi[0]);
        block_best(a1, cb + 1, best[0], bi[0]);
      }
      if (cb < nblk) {   // an odd last block (uniform)
        v16f a0 = init(cb);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const v8bf b = __builtin_bit_cast(v8bf, vcur[0][c]);
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(chi, cb, c), b, a0, 0, 0, 0);
          a0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag(clo, cb, c), b, a0, 0, 0, 0);
        }
        block_best(a0, cb, best[0], bi[0]);
      }
    } else {
      for (int cb = 0; cb < nblk; ++cb) {
        v16f a[NSET];
        a[0] = init(cb);
#pragma unroll
        for (int u = 1; u < NSET; ++u) a[u] = a[0];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const v8bf fh = frag(chi, cb, c), fl = frag(clo, cb, c);
#pragma unroll
          for (int u = 0; u < NSET; ++u)
            a[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fh, __builtin_bit_cast(v8bf, vcur[u][c]), a[u], 0, 0, 0);
#pragma unroll
          for (int u = 0; u < NSET; ++u)
            a[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fl, __builtin_bit_cast(v8bf, vcur[u][c]), a[u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < NSET; ++u) block_best(a[u], cb, best[u], bi[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < NSET; ++u) {
      float bu = best[u];
      int iu = bi[u];
      const float ob = __shfl_xor(bu, 32, 64);
      const int oi = __shfl_xor(iu, 32, 64);
      if (ob > bu || (ob == bu && oi < iu)) { bu = ob; iu = oi; }
      const int tok = tok_of(grp, u);
      if (tok < N && g == 0) {
        labels[(size_t)bh * N + tok] = iu;
        if (hist) atomicAdd(&hcount[iu & 255], 1);   // integer counts: order-free
      }
      if (mindist) {   // ||v||^2 - 2 (v.c - ||c||^2 / 2) of the winner (test output only)
        float vn = 0.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = bf16_to_f32((uint16_t)vcur[u][c][e]);
            vn = fmaf(x, x, vn);
          }
        vn += __shfl_xor(vn, 32, 64);
        if (tok < N && g == 0) mindist[(size_t)bh * N + tok] = fmaf(-2.0f, bu, vn);
      }
    }
    if (grp + 1 < NG) {
      if constexpr (PF) {
#pragma unroll
        for (int u = 0; u < NSET; ++u)
#pragma unroll
          for (int c = 0; c < 8; ++c) vcur[u][c] = vnext[u][c];
      } else {
        load_rows(grp + 1, vcur);
      }
    }
  }
  if (hist) {   // a workgroup's TOK tokens are one tile of the label sort
    __syncthreads();
    if (t < 256) hist[((size_t)bh * gridDim.x + blockIdx.x) * 256 + t] = hcount[t];
  }
}

// Centroid update: one workgroup per (cluster, b*h); 32 row streams x 16 lanes of 8 channels.
// The sums are float64 sums of bf16 values (exact unless a cluster's values span more than
// about 45 binary orders of magnitude), reduced in a fixed order.  With OBJ the workgroup also
// sums the squares of its rows and writes the cluster's objective term
//   J_c = sum_{t in c} ||v_t||^2 - 2 c.S + n ||c||^2 = sum_{t in c} ||v_t - c||^2
// with S the exact row sum and c the float32 centroid just stored (float64 arithmetic).
// With chi non-null the workgroup also writes what the next assign needs of its centroid (the
// prep kernel's bf16 hi + lo split and -||c||^2 / 2, the same operations in the same order).
// With NT the rows are read with nontemporal loads (chosen when V is larger than the chip's last-level
// cache, which then cannot hold V from one pass to the next anyway).
template <bool OBJ, bool NT>
__global__ __launch_bounds__(512) void k_kmeans_update(const uint16_t* __restrict__ V,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ offsets,
                                                       int N, int k, float* __restrict__ C,
                                                       double* __restrict__ jc, int kpad,
                                                       uint16_t* __restrict__ chi, uint16_t* __restrict__ clo,
                                                       float* __restrict__ cnorm) {
  __shared__ double part[32][VC_D];
  __shared__ double red[512];
  __shared__ float crow[VC_D];
  const int c = blockIdx.x, bh = blockIdx.y, t = threadIdx.x;
  const int l8 = t & 15, st = t >> 4;
  const int beg = offsets[(size_t)bh * (k + 1) + c], end = offsets[(size_t)bh * (k + 1) + c + 1];
  if (end <= beg) {  // empty cluster keeps its centroid and adds nothing to J (uniform branch)
    if (OBJ && t == 0) jc[(size_t)bh * k + c] = 0.0;
    return;
  }
  const int32_t* pb = perm + (size_t)bh * N;
  const uint16_t* Vb = V + (size_t)bh * N * VC_D + 8 * l8;
  double a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  double sq = 0.0;
  // stream st takes the rows beg+st, beg+st+32, ...; its 16 lanes fetch the next 16 row
  // indices at once and share them, so 16 row loads are in flight per stream
  for (int p0 = beg + st; p0 < end; p0 += 32 * 16) {
    const int pl = p0 + 32 * l8;
    const int mytok = pl < end ? pb[pl] : 0;
    const int n = (end - p0 + 31) / 32 < 16 ? (end - p0 + 31) / 32 : 16;   // rows of this batch
    uint4 raw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int tok = __shfl(mytok, (t & 48) + i, 64);   // lane i of this 16-lane stream
      const uint16_t* row = Vb + (size_t)tok * VC_D;
      raw[i] = i < n ? (NT ? ld_stream4(row) : *(const uint4*)row) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double x0 = (double)bf16_to_f32(wd[e] & 0xFFFFu), x1 = (double)bf16_to_f32(wd[e] >> 16);
        a[2 * e] += x0;
        a[2 * e + 1] += x1;
        if constexpr (OBJ) sq = fma(x1, x1, fma(x0, x0, sq));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[st][8 * l8 + i] = a[i];
  if constexpr (OBJ) red[t] = sq;
  __syncthreads();
  if (t < VC_D) {
    double s = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += part[i][t];
    const double n = (double)(end - beg);
    const float cf = (float)(s / n);
    C[((size_t)bh * k + c) * VC_D + t] = cf;
    if (chi) {
      const size_t o = ((size_t)bh * kpad + c) * VC_D + t;
      const uint32_t hi = f32_to_bf16_rne(cf);
      chi[o] = (uint16_t)hi;
      clo[o] = (uint16_t)f32_to_bf16_rne(cf - bf16_to_f32(hi));
      crow[t] = cf;
    }
    if constexpr (OBJ) {
      const double cd = (double)cf;
      red[t] += cd * (n * cd - 2.0 * s);   // this channel's -2 c S + n c^2
    }
  }
  if (chi) {
    __syncthreads();
    if (t == 0) {
      float sq2 = 0.0f;
      for (int i = 0; i < VC_D; ++i) sq2 = fmaf(crow[i], crow[i], sq2);
      cnorm[(size_t)bh * kpad + c] = -0.5f * sq2;
    }
  }
  if constexpr (OBJ) {
    __syncthreads();
    for (int off = 256; off > 0; off >>= 1) {   // fixed-order tree over the 512 terms
      if (t < off) red[t] += red[t + off];
      __syncthreads();
    }
    if (t == 0) jc[(size_t)bh * k + c] = red[0];
  }
}

// J per (b, h): the clusters' terms summed in index order.
__global__ void k_kmeans_objective_final(const double* __restrict__ jc, int k, double* __restrict__ J) {
  const int bh = blockIdx.x;
  if (threadIdx.x == 0) {
    double s = 0;
    for (int i = 0; i < k; ++i) s += jc[(size_t)bh * k + i];
    J[bh] = s;
  }
}

hipError_t vc_launch_kmeans_init(const uint16_t* V, int BH, int N, int k, float* C, hipStream_t s) {
  hipLaunchKernelGGL(k_kmeans_init, dim3(k, BH), dim3(128), 0, s, V, N, k, C);
  return hipGetLastError();
}

// The assign kernel's dynamic-LDS limit, raised once per device to what the largest k needs.
// A function attribute is host-side state: setting it on every launch would also run inside a
// caller's graph capture, where only the launches belong.
static hipError_t assign_lds_limit() {
  static std::atomic<unsigned long long> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const unsigned long long bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const size_t lds_max = (size_t)2 * VC_MAX_K * KM_ROW * sizeof(uint16_t) + (size_t)VC_MAX_K * sizeof(float);
  e = hipFuncSetAttribute((const void*)k_kmeans_assign<VC_SORT_TILE, 2, false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)lds_max);
  if (e == hipSuccess)
    e = hipFuncSetAttribute((const void*)k_kmeans_assign<VC_SORT_TILE_SMALL, 1, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_max);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

hipError_t vc_launch_kmeans_assign(const uint16_t* V, const float* C, int BH, int N, int k,
                                   int32_t* labels, float* mindist, uint16_t* chi, uint16_t* clo,
                                   float* cn, bool prep, int32_t* hist, hipStream_t s) {
  const int kpad = (k + 31) & ~31;
  if (prep) hipLaunchKernelGGL(k_kmeans_prep, dim3(kpad, BH), dim3(128), 0, s, C, k, kpad, chi, clo, cn);
  const size_t lds = (size_t)2 * kpad * KM_ROW * sizeof(uint16_t) + (size_t)kpad * sizeof(float);
  hipError_t e = assign_lds_limit();
  if (e != hipSuccess) return e;
  const int tile = vc_group_tile(BH, N);   // the label sort's tile, whose histograms hist holds
  const int nblk = (N + tile - 1) / tile;
  if (tile == VC_SORT_TILE)
    hipLaunchKernelGGL((k_kmeans_assign<VC_SORT_TILE, 2, false>), dim3(nblk, BH), dim3(KM_THREADS), lds, s, V,
                       (const uint16_t*)chi, (const uint16_t*)clo, (const float*)cn, N, kpad, labels, mindist, hist);
  else
    hipLaunchKernelGGL((k_kmeans_assign<VC_SORT_TILE_SMALL, 1, true>), dim3(nblk, BH), dim3(KM_THREADS), lds, s, V,
                       (const uint16_t*)chi, (const uint16_t*)clo, (const float*)cn, N, kpad, labels, mindist, hist);
  return hipGetLastError();
}

hipError_t vc_launch_kmeans_update(const uint16_t* V, const int32_t* perm, const int32_t* offsets,
                                   int BH, int N, int k, float* C, double* jc, double* J,
                                   uint16_t* chi, uint16_t* clo, float* cn, hipStream_t s) {
  const int kpad = (k + 31) & ~31;
  // MI355X's last-level cache (Infinity Cache) holds 256 MB.  A V that fits is still partly there
  // when the update reads it after the assign, and plain loads keep it there for the next round;
  // a larger V streams from HBM either way, and nontemporal loads do that faster (measured: video
  // and long shapes 5-7 % faster per grouping call with them, the 201 MB reuse shape 9 % slower).
  const bool nt = (size_t)BH * N * VC_D * sizeof(uint16_t) > ((size_t)256 << 20);
  auto launch = [&](auto kern, double* jcp) {
    hipLaunchKernelGGL(kern, dim3(k, BH), dim3(512), 0, s, V, perm, offsets, N, k, C, jcp, kpad, chi, clo, cn);
  };
  if (J) {
    if (nt) launch(k_kmeans_update<true, true>, jc);
    else launch(k_kmeans_update<true, false>, jc);
    hipLaunchKernelGGL(k_kmeans_objective_final, dim3(BH), dim3(64), 0, s, (const double*)jc, k, J);
  } else {
    if (nt) launch(k_kmeans_update<false, true>, (double*)nullptr);
    else launch(k_kmeans_update<false, false>, (double*)nullptr);
  }
  return hipGetLastError();
}
