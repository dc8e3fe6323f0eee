// Stable counting sort of cluster labels (VC-Attention Sec. 3.2, Eq. 3: pi = argsort(z)).
//
// k <= 256, so one 8-bit digit suffices.  Three deterministic passes per (b, h):
//   1. per tile of 1024 (or, for small shapes, 256) tokens, a label histogram (integer LDS
//      atomics: order-free);
//   2. per (b, h), an exclusive scan in (label, tile) order -> the first sorted position of
//      each label inside each tile, and the cluster offsets;
//   3. per tile, each token's rank among equal labels before it (wave ballots for the
//      in-wave rank, an LDS prefix over the tile's waves) -> perm[pos] = token.
// Ties keep token order, so the result is the stable argsort.  Labels are masked to 8 bits,
// so any input keeps every write inside perm.
#include "vc_common.h"
#include "vc_internal.h"

template <int TILE>
__global__ __launch_bounds__(256) void k_sort_hist(const int32_t* __restrict__ labels, int N, int nblk,
                                                   int32_t* __restrict__ hist) {
  __shared__ int h[256];
  const int bh = blockIdx.y, blk = blockIdx.x, t = threadIdx.x;
  h[t] = 0;
  __syncthreads();
  const int32_t* lab = labels + (size_t)bh * N;
#pragma unroll
  for (int r = 0; r < TILE / 256; ++r) {
    int tok = blk * TILE + r * 256 + t;
    if (tok < N) atomicAdd(&h[lab[tok] & 255], 1);
  }
  __syncthreads();
  hist[((size_t)bh * nblk + blk) * 256 + t] = h[t];
}

// One workgroup per (b,h); thread c owns label c.
__global__ __launch_bounds__(256) void k_sort_scan(int N, int nblk, int k, int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ offsets) {
  __shared__ int s[256];
  const int bh = blockIdx.x, c = threadIdx.x;
  int32_t* hb = hist + (size_t)bh * nblk * 256;
  int total = 0;
  // both passes unrolled so each thread has 16 independent loads in flight (the loop is
  // otherwise one global-memory round trip per tile)
#pragma unroll 16
  for (int b = 0; b < nblk; ++b) total += hb[b * 256 + c];
  s[c] = total;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 labels
  for (int off = 1; off < 256; off <<= 1) {
    int v = c >= off ? s[c - off] : 0;
    __syncthreads();
    s[c] += v;
    __syncthreads();
  }
  int start = s[c] - total;  // exclusive
  int run = start;
#pragma unroll 16
  for (int b = 0; b < nblk; ++b) {
    int v = hb[b * 256 + c];
    hb[b * 256 + c] = run;
    run += v;
  }
  if (c <= k) offsets[(size_t)bh * (k + 1) + c] = start;
  if (k == 256 && c == 255) offsets[(size_t)bh * (k + 1) + 256] = s[255];
  (void)N;
}

// One thread per token of a TILE-token tile.
template <int TILE>
__global__ __launch_bounds__(TILE) void k_sort_scatter(const int32_t* __restrict__ labels, int N, int nblk,
                                                       const int32_t* __restrict__ base,
                                                       int32_t* __restrict__ perm) {
  constexpr int NW = TILE / 64;
  __shared__ int cnt[NW][256];
  const int bh = blockIdx.y, blk = blockIdx.x, t = threadIdx.x;
  const int w = t >> 6, lane = t & 63;
  for (int i = t; i < NW * 256; i += TILE) (&cnt[0][0])[i] = 0;
  const int tok = blk * TILE + t;
  const bool valid = tok < N;
  const int lab = valid ? (labels[(size_t)bh * N + tok] & 255) : 0;
  // lanes of this wave holding the same label
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    uint64_t b = __ballot(valid && ((lab >> bit) & 1));
    m &= ((lab >> bit) & 1) ? b : ~b;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(m & below);
  __syncthreads();
  if (valid && rank == 0) cnt[w][lab] = __popcll(m);
  __syncthreads();
  if (t < 256) {
    int run = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      int v = cnt[ww][t];
      cnt[ww][t] = run;
      run += v;
    }
  }
  __syncthreads();
  if (valid) {
    int pos = base[((size_t)bh * nblk + blk) * 256 + lab] + cnt[w][lab] + rank;
    perm[(size_t)bh * N + pos] = tok;
  }
}

hipError_t vc_launch_label_sort(const int32_t* labels, int BH, int N, int k, int32_t* hist,
                                int32_t* perm, int32_t* offsets, bool hist_ready, hipStream_t s) {
  const int tile = vc_group_tile(BH, N);
  const int nblk = (N + tile - 1) / tile;
  if (!hist_ready) {
    if (tile == VC_SORT_TILE)
      hipLaunchKernelGGL(k_sort_hist<VC_SORT_TILE>, dim3(nblk, BH), dim3(256), 0, s, labels, N, nblk, hist);
    else
      hipLaunchKernelGGL(k_sort_hist<VC_SORT_TILE_SMALL>, dim3(nblk, BH), dim3(256), 0, s, labels, N, nblk, hist);
  }
  hipLaunchKernelGGL(k_sort_scan, dim3(BH), dim3(256), 0, s, N, nblk, k, hist, offsets);
  if (tile == VC_SORT_TILE)
    hipLaunchKernelGGL(k_sort_scatter<VC_SORT_TILE>, dim3(nblk, BH), dim3(VC_SORT_TILE), 0, s, labels, N, nblk,
                       (const int32_t*)hist, perm);
  else
    hipLaunchKernelGGL(k_sort_scatter<VC_SORT_TILE_SMALL>, dim3(nblk, BH), dim3(VC_SORT_TILE_SMALL), 0, s, labels,
                       N, nblk, (const int32_t*)hist, perm);
  return hipGetLastError();
}
