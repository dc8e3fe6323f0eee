// Host-side launchers of the VC-Attention kernels (internal; the public ABI is vc_attn.h).
// Each launcher enqueues its kernels on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Workspace layout of the grouping call (byte offsets from ws, each 256-byte aligned).
struct vc_group_ws {
  size_t hist;      // int32 [BH][nblk][256] per-block label histograms, then scatter bases
  size_t jclust;    // float64 [BH][k] per-cluster objective terms
  size_t chi, clo;  // bf16 [BH][kpad][128] centroids split into hi + lo parts (kpad = k to 32)
  size_t cnorm;     // float32 [BH][kpad] -||c||^2 / 2 per centroid (the assign accumulator start)
  size_t total;
};
vc_group_ws vc_group_ws_layout(int BH, int N, int k);

// Workspace layout of the demean/quantise call.
struct vc_dq_ws {
  size_t kpart;     // float64 [BH][nchunk][128] key channel partial sums
  size_t kbar;      // float32 [BH][128] key channel means
  size_t mu;        // float32 [BH][N/128][128] block means
  size_t amaxp;     // float32 [BH][N/128][128] per-tile residual |R| maxima
  size_t amax;      // float32 [BH][8][128] residual |R| maxima over eight slices of the tiles
  size_t total;
};
vc_dq_ws vc_dq_ws_layout(int BH, int N);

// Tokens per label-sort tile, which is also one k-means assign workgroup's share: 1024, or 256
// when 1024-token tiles would give fewer than two workgroups per CU of the 256-CU chip (small
// B*H*N), so that small shapes still spread over the chip.  A pure function of the shape, so
// the workspace size and the launches agree.
constexpr int VC_SORT_TILE = 1024;
constexpr int VC_SORT_TILE_SMALL = 256;
constexpr long long VC_SMALL_GRID = 512;
inline int vc_group_tile(int BH, int N) {
  const long long wg = (long long)BH * ((N + VC_SORT_TILE - 1) / VC_SORT_TILE);
  return wg < VC_SMALL_GRID ? VC_SORT_TILE_SMALL : VC_SORT_TILE;
}
// VC_OK for hipSuccess, else VC_ERR_HIP with the error kept for vc_last_hip_error().
int vc_hip_status(hipError_t e);
// Rows per key-mean partial: 1024, or 256 for small shapes (the same rule).  The partials are
// exact float64 sums of bf16 values, so the chunking does not change the mean.
constexpr int VC_KSTAT_CHUNK = 1024;
constexpr int VC_KSTAT_CHUNK_SMALL = 256;
inline int vc_kstat_chunk(int BH, int N) {
  const long long wg = (long long)BH * ((N + VC_KSTAT_CHUNK - 1) / VC_KSTAT_CHUNK);
  return wg < VC_SMALL_GRID ? VC_KSTAT_CHUNK_SMALL : VC_KSTAT_CHUNK;
}

hipError_t vc_launch_test_expcast(const float* u, uint8_t* codes, size_t n, hipStream_t s);
hipError_t vc_launch_test_e4m3(const float* x, uint8_t* codes, size_t n, hipStream_t s);
hipError_t vc_launch_test_fp4(const float* x, uint8_t* codes, size_t npair, hipStream_t s);
hipError_t vc_launch_test_fp6(const float* x, const float* scale, uint32_t* words, size_t ngroups, hipStream_t s);
hipError_t vc_launch_test_mfma_fp8_rate(float* out, int workgroups, int iters, float* clock_mhz,
                                        hipStream_t s);

hipError_t vc_launch_kmeans_init(const uint16_t* V, int BH, int N, int k, float* C, hipStream_t s);
// Assignment with the centroids' split rows chi/clo and norms cn; with prep they are first
// computed from C (else they are the previous update's); with hist non-null the assign
// workgroups also write the label sort's per-tile histograms into it.
hipError_t vc_launch_kmeans_assign(const uint16_t* V, const float* C, int BH, int N, int k,
                                   int32_t* labels, float* mindist, uint16_t* chi, uint16_t* clo,
                                   float* cn, bool prep, int32_t* hist, hipStream_t s);
// Update of the centroids from the sorted rows; with J non-null (the last round) also the
// objective per (b,h) into J, via the per-cluster terms in jc; with chi non-null also the split
// rows and norms the next assign reads.
hipError_t vc_launch_kmeans_update(const uint16_t* V, const int32_t* perm, const int32_t* offsets,
                                   int BH, int N, int k, float* C, double* jc, double* J,
                                   uint16_t* chi, uint16_t* clo, float* cn, hipStream_t s);
// hist_ready: the per-tile histograms are already in hist (written by the assign kernel).
hipError_t vc_launch_label_sort(const int32_t* labels, int BH, int N, int k, int32_t* hist,
                                int32_t* perm, int32_t* offsets, bool hist_ready, hipStream_t s);

hipError_t vc_launch_demean_quant(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                  int BH, int N, unsigned flags, uint8_t* Kq, float* sK,
                                  uint8_t* Rq, uint16_t* mu_out, float* sV, char* ws,
                                  const vc_dq_ws& L, hipStream_t s);

hipError_t vc_launch_demean_quant_mx6(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                      int BH, int N, unsigned flags, uint8_t* Kq6, uint8_t* sK6,
                                      uint8_t* Rq6, uint8_t* sR6, uint16_t* mu_out, char* ws,
                                      const vc_dq_ws& L, hipStream_t s);

hipError_t vc_launch_demean_quant_mx4(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                      int BH, int N, unsigned flags, uint8_t* Kq4, uint8_t* sK4,
                                      uint8_t* Rq4, uint8_t* sR4, uint16_t* mu_out, char* ws,
                                      const vc_dq_ws& L, hipStream_t s);

// bits = 4 (E2M1 operands, 64-byte rows) or 6 (E2M3 operands, 128-byte rows of 32-byte groups)
hipError_t vc_launch_attn_fwd_mx4(const uint16_t* Q, const uint8_t* Kq4, const uint8_t* sK4,
                                  const uint8_t* Rq4, const uint8_t* sR4, const uint16_t* mu,
                                  int BH, int N, float L4, unsigned flags, uint16_t* O,
                                  int bits, hipStream_t s);  // L4 = float32(log2(e) softmax_scale)
// The 6-bit kernel with VC_ATTN_NO_MEAN | VC_ATTN_HADAMARD (built at -O2, attn_fwd_mx6_rn.hip).
hipError_t vc_launch_attn_fwd_mx6_rn(const uint16_t* Q, const uint8_t* Kq6, const uint8_t* sK6,
                                     const uint8_t* Rq6, const uint8_t* sR6, const uint16_t* mu, int BH, int N, float L4,
                                     uint16_t* O, hipStream_t s);

// clk: NULL, or 4 x vc_attn_fwd_workgroups(BH, N) uint64 that receive each workgroup's start
// and end stamps (shader cycles, constant-rate ticks) for the clock probe.
hipError_t vc_launch_attn_fwd(const uint16_t* Q, const uint8_t* Kq, const float* sK,
                              const uint8_t* Rq, const uint16_t* mu, const float* sV,
                              int BH, int N, float L, unsigned flags, uint16_t* O,
                              uint64_t* clk, hipStream_t s);  // L = float32(8 log2(e) softmax_scale)
uint32_t vc_attn_fwd_workgroups(int BH, int N);
hipError_t vc_launch_test_qquant(const uint16_t* Q, int BH, int N, float L, bool hadamard, uint8_t* Qq, float* sQ,
                                 hipStream_t s);
// Per (b,h): count of entries of perm [BH][N] outside [0, N) or repeated, into bad [BH]; bits is
// a scratch bitmap of BH * ceil(N/32) words.
hipError_t vc_launch_validate_perm(const int32_t* perm, int BH, int N, uint32_t* bits, int32_t* bad, hipStream_t s);
