// C ABI of the VC-Attention library: argument validation (host only, before any HIP call),
// workspace carving and kernel dispatch.  Contracts are documented in include/vc_attn.h.
#include "vc_attn.h"
#include "vc_internal.h"

#include <hip/hip_runtime.h>
#include <math.h>

namespace {

thread_local int g_last_hip_error = 0;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return VC_OK;
  g_last_hip_error = (int)e;
  return VC_ERR_HIP;
}

// Common shape checks. Returns VC_OK, an error, or 1 for an empty problem.
int check_shape(int B, int H, int N, int d) {
  if (B < 0 || H < 0 || N < 0) return VC_ERR_SHAPE;
  if (d != VC_HEAD_DIM) return VC_ERR_SHAPE;
  if (N % VC_BLOCK != 0) return VC_ERR_SHAPE;
  if (B == 0 || H == 0 || N == 0) return 1;
  long long total = (long long)B * H * (long long)N * d;
  if (total >= (1LL << 31)) return VC_ERR_OVERFLOW;
  return VC_OK;
}

}  // namespace

int vc_hip_status(hipError_t e) { return hip_status(e); }

vc_group_ws vc_group_ws_layout(int BH, int N, int k) {
  vc_group_ws L;
  const int tile = vc_group_tile(BH, N);
  size_t nblk = (size_t)(N + tile - 1) / tile;
  size_t kpad = (size_t)((k + 31) & ~31);
  size_t off = 0;
  L.hist = off;  off = align256(off + (size_t)BH * nblk * 256 * sizeof(int32_t));
  L.jclust = off; off = align256(off + (size_t)BH * (size_t)k * sizeof(double));
  L.chi = off;   off = align256(off + (size_t)BH * kpad * VC_HEAD_DIM * sizeof(uint16_t));
  L.clo = off;   off = align256(off + (size_t)BH * kpad * VC_HEAD_DIM * sizeof(uint16_t));
  L.cnorm = off; off = align256(off + (size_t)BH * kpad * sizeof(float));
  L.total = off;
  return L;
}

vc_dq_ws vc_dq_ws_layout(int BH, int N) {
  vc_dq_ws L;
  const int chunk = vc_kstat_chunk(BH, N);
  size_t nchunk = (size_t)(N + chunk - 1) / chunk;
  size_t off = 0;
  L.kpart = off; off = align256(off + (size_t)BH * nchunk * 128 * sizeof(double));
  L.kbar = off;  off = align256(off + (size_t)BH * 128 * sizeof(float));
  L.mu = off;    off = align256(off + (size_t)BH * (size_t)(N / 128) * 128 * sizeof(float));
  L.amaxp = off; off = align256(off + (size_t)BH * (size_t)(N / 128) * 128 * sizeof(float));
  L.amax = off;  off = align256(off + (size_t)BH * 8 * 128 * sizeof(float));
  L.total = off;
  return L;
}

extern "C" {

const char* vc_strerror(int status) {
  switch (status) {
    case VC_OK: return "ok";
    case VC_ERR_NULL: return "required pointer is NULL";
    case VC_ERR_SHAPE: return "bad shape (need d == 128, N % 128 == 0, sizes >= 0)";
    case VC_ERR_K: return "k must be in [1, min(256, N)]";
    case VC_ERR_ITERS: return "iters must be >= 1";
    case VC_ERR_WORKSPACE: return "workspace too small";
    case VC_ERR_OVERFLOW: return "B*H*N*d must be below 2^31";
    case VC_ERR_FLAGS: return "unknown flag bits";
    case VC_ERR_HIP: return "HIP call failed (see vc_last_hip_error)";
    default: return "unknown status";
  }
}

int vc_last_hip_error(void) { return g_last_hip_error; }

size_t vc_group_workspace_size(int B, int H, int N, int k) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  if (k < 1 || k > VC_MAX_K) k = VC_MAX_K;   // an invalid k is rejected by the call itself
  return vc_group_ws_layout(B * H, N, k).total;
}

size_t vc_demean_quant_workspace_size(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return vc_dq_ws_layout(B * H, N).total;
}

int vc_vsmooth_group(const uint16_t* V, int B, int H, int N, int d, int k, int iters,
                     const float* C_init, float* C_out, int32_t* labels, int32_t* perm,
                     int32_t* offsets, double* objective, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!V || !C_out || !labels || !perm || !offsets || !ws) return VC_ERR_NULL;
  if (k < 1 || k > VC_MAX_K || k > N) return VC_ERR_K;
  if (iters < 1) return VC_ERR_ITERS;
  int BH = B * H;
  vc_group_ws L = vc_group_ws_layout(BH, N, k);
  if (ws_bytes < L.total) return VC_ERR_WORKSPACE;
  char* w = (char*)ws;
  int32_t* hist = (int32_t*)(w + L.hist);
  double* jclust = (double*)(w + L.jclust);
  uint16_t* chi = (uint16_t*)(w + L.chi);
  uint16_t* clo = (uint16_t*)(w + L.clo);
  float* cnorm = (float*)(w + L.cnorm);
  hipError_t e = hipSuccess;
  if (C_init) {
    if (C_init != C_out)
      e = hipMemcpyAsync(C_out, C_init, (size_t)BH * k * VC_HEAD_DIM * sizeof(float),
                         hipMemcpyDeviceToDevice, stream);
  } else {
    e = vc_launch_kmeans_init(V, BH, N, k, C_out, stream);
  }
  if (e != hipSuccess) return hip_status(e);
  // Per round: assign (which also counts the label sort's per-tile histograms), the rest of the
  // sort, update (which also prepares the next assign's split centroids; the first round's come
  // from the prep kernel, the last update's are not needed).
  for (int it = 0; it < iters; ++it) {
    if ((e = vc_launch_kmeans_assign(V, C_out, BH, N, k, labels, nullptr, chi, clo, cnorm, it == 0, hist,
                                     stream)) != hipSuccess)
      return hip_status(e);
    if ((e = vc_launch_label_sort(labels, BH, N, k, hist, perm, offsets, true, stream)) != hipSuccess)
      return hip_status(e);
    const bool last = it == iters - 1;
    double* J = last ? objective : nullptr;   // J with the final labels and means
    if ((e = vc_launch_kmeans_update(V, perm, offsets, BH, N, k, C_out, jclust, J, last ? nullptr : chi, clo,
                                     cnorm, stream)) != hipSuccess)
      return hip_status(e);
  }
  return VC_OK;
}

int vc_vsmooth_demean_quant(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                            int B, int H, int N, int d, unsigned flags,
                            uint8_t* Kq, float* sK, uint8_t* Rq, uint16_t* mu_out, float* sV,
                            void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!K || !V || !Kq || !sK || !Rq || !mu_out || !sV || !ws) return VC_ERR_NULL;
  if (flags & ~(VC_DQ_NO_DEMEAN | VC_DQ_HADAMARD)) return VC_ERR_FLAGS;
  int BH = B * H;
  vc_dq_ws L = vc_dq_ws_layout(BH, N);
  if (ws_bytes < L.total) return VC_ERR_WORKSPACE;
  return hip_status(vc_launch_demean_quant(K, V, perm, BH, N, flags, Kq, sK, Rq, mu_out, sV,
                                           (char*)ws, L, stream));
}

int vc_attn_fwd(const uint16_t* Q, const uint8_t* Kq, const float* sK, const uint8_t* Rq,
                const uint16_t* mu, const float* sV, int B, int H, int N, int d,
                float softmax_scale, unsigned flags, uint16_t* O, hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!Q || !Kq || !sK || !Rq || !sV || !O) return VC_ERR_NULL;
  if (!mu && !(flags & VC_ATTN_NO_MEAN)) return VC_ERR_NULL;
  if (flags & ~(VC_ATTN_NO_MEAN | VC_ATTN_EXP_THEN_CAST | VC_ATTN_HADAMARD)) return VC_ERR_FLAGS;
  if (!(softmax_scale >= 0.0f) || isinf(softmax_scale)) return VC_ERR_SHAPE;
  // L = float32(8 log2(e) * scale), the scale taken in double (1/sqrt(d) when 0 is passed)
  const double scale = softmax_scale == 0.0f ? 1.0 / sqrt((double)d) : (double)softmax_scale;
  const float L = (float)(8.0 * 1.4426950408889634 * scale);
  return hip_status(vc_launch_attn_fwd(Q, Kq, sK, Rq, mu, sV, B * H, N, L, flags, O, nullptr, stream));
}

size_t vc_workspace_size(int op, int B, int H, int N, int d, int k) {
  if (d != VC_HEAD_DIM) return 0;
  switch (op) {
    case VC_OP_GROUP: return vc_group_workspace_size(B, H, N, k);
    case VC_OP_DEMEAN_QUANT:
    case VC_OP_DEMEAN_QUANT_MX4:
    case VC_OP_DEMEAN_QUANT_MX6: return vc_demean_quant_workspace_size(B, H, N);
    case VC_OP_VALIDATE_PERM:
      if (B <= 0 || H <= 0 || N <= 0) return 0;
      return align256((size_t)B * H * (size_t)((N + 31) / 32) * sizeof(uint32_t));
    case VC_OP_ATTN_FWD:
    case VC_OP_ATTN_FWD_MX4:
    case VC_OP_ATTN_FWD_MX6: return 0;
    default: return 0;
  }
}

int vc_validate_perm(const int32_t* perm, int B, int H, int N, int32_t* bad, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  if (B < 0 || H < 0 || N < 0) return VC_ERR_SHAPE;
  if (B == 0 || H == 0 || N == 0) return VC_OK;
  if ((long long)B * H * (long long)N >= (1LL << 31)) return VC_ERR_OVERFLOW;
  if (!perm || !bad || !ws) return VC_ERR_NULL;
  if (ws_bytes < vc_workspace_size(VC_OP_VALIDATE_PERM, B, H, N, VC_HEAD_DIM, 1)) return VC_ERR_WORKSPACE;
  return hip_status(vc_launch_validate_perm(perm, B * H, N, (uint32_t*)ws, bad, stream));
}

int vc_test_quantize_q(const uint16_t* Q, int B, int H, int N, int d, float softmax_scale, unsigned flags,
                       uint8_t* Qq, float* sQ, hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!Q || !Qq || !sQ) return VC_ERR_NULL;
  if (flags & ~VC_ATTN_HADAMARD) return VC_ERR_FLAGS;
  if (!(softmax_scale >= 0.0f) || isinf(softmax_scale)) return VC_ERR_SHAPE;
  const double scale = softmax_scale == 0.0f ? 1.0 / sqrt((double)d) : (double)softmax_scale;
  const float L = (float)(8.0 * 1.4426950408889634 * scale);
  return hip_status(vc_launch_test_qquant(Q, B * H, N, L, (flags & VC_ATTN_HADAMARD) != 0, Qq, sQ, stream));
}

int vc_test_wall_clock_khz(int* khz) {
  if (!khz) return VC_ERR_NULL;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(khz, hipDeviceAttributeWallClockRate, dev);
  return hip_status(e);
}

size_t vc_test_attn_clock_slots(int B, int H, int N) {
  if (B <= 0 || H <= 0 || N <= 0 || N % VC_BLOCK) return 0;
  return 4 * (size_t)vc_attn_fwd_workgroups(B * H, N);
}

int vc_test_attn_fwd_clock(const uint16_t* Q, const uint8_t* Kq, const float* sK, const uint8_t* Rq,
                           const uint16_t* mu, const float* sV, int B, int H, int N, int d,
                           float softmax_scale, unsigned flags, uint16_t* O, uint64_t* clk, hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!Q || !Kq || !sK || !Rq || !sV || !O || !clk) return VC_ERR_NULL;
  if (!mu && !(flags & VC_ATTN_NO_MEAN)) return VC_ERR_NULL;
  if (flags & ~(VC_ATTN_NO_MEAN | VC_ATTN_EXP_THEN_CAST | VC_ATTN_HADAMARD)) return VC_ERR_FLAGS;
  if (!(softmax_scale >= 0.0f) || isinf(softmax_scale)) return VC_ERR_SHAPE;
  const double scale = softmax_scale == 0.0f ? 1.0 / sqrt((double)d) : (double)softmax_scale;
  const float L = (float)(8.0 * 1.4426950408889634 * scale);
  return hip_status(vc_launch_attn_fwd(Q, Kq, sK, Rq, mu, sV, B * H, N, L, flags, O, clk, stream));
}

int vc_vsmooth_demean_quant_mx4(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                int B, int H, int N, int d, unsigned flags,
                                uint8_t* Kq4, uint8_t* sK4, uint8_t* Rq4, uint8_t* sR4,
                                uint16_t* mu_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!K || !V || !Kq4 || !sK4 || !Rq4 || !sR4 || !mu_out || !ws) return VC_ERR_NULL;
  if (flags & ~(VC_DQ_NO_DEMEAN | VC_DQ_HADAMARD)) return VC_ERR_FLAGS;
  int BH = B * H;
  vc_dq_ws L = vc_dq_ws_layout(BH, N);
  if (ws_bytes < L.total) return VC_ERR_WORKSPACE;
  return hip_status(vc_launch_demean_quant_mx4(K, V, perm, BH, N, flags, Kq4, sK4, Rq4, sR4, mu_out,
                                               (char*)ws, L, stream));
}

int vc_attn_fwd_mx4(const uint16_t* Q, const uint8_t* Kq4, const uint8_t* sK4, const uint8_t* Rq4,
                    const uint8_t* sR4, const uint16_t* mu, int B, int H, int N, int d,
                    float softmax_scale, unsigned flags, uint16_t* O, hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!Q || !Kq4 || !sK4 || !Rq4 || !sR4 || !O) return VC_ERR_NULL;
  if (!mu && !(flags & VC_ATTN_NO_MEAN)) return VC_ERR_NULL;
  if (flags & ~(VC_ATTN_NO_MEAN | VC_ATTN_HADAMARD)) return VC_ERR_FLAGS;
  if (!(softmax_scale >= 0.0f) || isinf(softmax_scale)) return VC_ERR_SHAPE;
  // L4 = float32(log2(e) * scale), the scale taken in double (1/sqrt(d) when 0 is passed)
  const double scale = softmax_scale == 0.0f ? 1.0 / sqrt((double)d) : (double)softmax_scale;
  const float L4 = (float)(1.4426950408889634 * scale);
  return hip_status(vc_launch_attn_fwd_mx4(Q, Kq4, sK4, Rq4, sR4, mu, B * H, N, L4, flags, O, 4, stream));
}

int vc_vsmooth_demean_quant_mx6(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                int B, int H, int N, int d, unsigned flags,
                                uint8_t* Kq6, uint8_t* sK6, uint8_t* Rq6, uint8_t* sR6,
                                uint16_t* mu_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!K || !V || !Kq6 || !sK6 || !Rq6 || !sR6 || !mu_out || !ws) return VC_ERR_NULL;
  if (flags & ~(VC_DQ_NO_DEMEAN | VC_DQ_HADAMARD)) return VC_ERR_FLAGS;
  int BH = B * H;
  vc_dq_ws L = vc_dq_ws_layout(BH, N);
  if (ws_bytes < L.total) return VC_ERR_WORKSPACE;
  return hip_status(vc_launch_demean_quant_mx6(K, V, perm, BH, N, flags, Kq6, sK6, Rq6, sR6, mu_out,
                                               (char*)ws, L, stream));
}

int vc_attn_fwd_mx6(const uint16_t* Q, const uint8_t* Kq6, const uint8_t* sK6, const uint8_t* Rq6,
                    const uint8_t* sR6, const uint16_t* mu, int B, int H, int N, int d,
                    float softmax_scale, unsigned flags, uint16_t* O, hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!Q || !Kq6 || !sK6 || !Rq6 || !sR6 || !O) return VC_ERR_NULL;
  if (!mu && !(flags & VC_ATTN_NO_MEAN)) return VC_ERR_NULL;
  if (flags & ~(VC_ATTN_NO_MEAN | VC_ATTN_HADAMARD)) return VC_ERR_FLAGS;
  if (!(softmax_scale >= 0.0f) || isinf(softmax_scale)) return VC_ERR_SHAPE;
  const double scale = softmax_scale == 0.0f ? 1.0 / sqrt((double)d) : (double)softmax_scale;
  const float L4 = (float)(1.4426950408889634 * scale);
  return hip_status(vc_launch_attn_fwd_mx4(Q, Kq6, sK6, Rq6, sR6, mu, B * H, N, L4, flags, O, 6, stream));
}

int vc_test_fp6_encode(const float* x, const float* scale, uint32_t* words, size_t ngroups, hipStream_t stream) {
  if (ngroups == 0) return VC_OK;
  if (!x || !words) return VC_ERR_NULL;
  if (ngroups >= (size_t(1) << 35)) return VC_ERR_OVERFLOW;
  return hip_status(vc_launch_test_fp6(x, scale, words, ngroups, stream));
}

int vc_test_fp4_encode(const float* x, uint8_t* codes, size_t n, hipStream_t stream) {
  if (n == 0) return VC_OK;
  if (!x || !codes) return VC_ERR_NULL;
  if (n & 1) return VC_ERR_SHAPE;
  if (n >= (size_t(1) << 40)) return VC_ERR_OVERFLOW;
  return hip_status(vc_launch_test_fp4(x, codes, n / 2, stream));
}

int vc_test_mfma_fp8_rate(float* out, int workgroups, int iters, float* clock_mhz, hipStream_t stream) {
  if (!out) return VC_ERR_NULL;
  if (workgroups < 1 || iters < 1) return VC_ERR_SHAPE;
  if ((double)workgroups * (double)iters * 4194304.0 > 4.611686018427388e18) return VC_ERR_SHAPE;
  return hip_status(vc_launch_test_mfma_fp8_rate(out, workgroups, iters, clock_mhz, stream));
}

int vc_test_expcast(const float* u, uint8_t* codes, size_t n, hipStream_t stream) {
  if (n == 0) return VC_OK;
  if (!u || !codes) return VC_ERR_NULL;
  if (n >= (size_t(1) << 40)) return VC_ERR_OVERFLOW;
  return hip_status(vc_launch_test_expcast(u, codes, n, stream));
}

int vc_test_e4m3_encode(const float* x, uint8_t* codes, size_t n, hipStream_t stream) {
  if (n == 0) return VC_OK;
  if (!x || !codes) return VC_ERR_NULL;
  if (n >= (size_t(1) << 40)) return VC_ERR_OVERFLOW;
  return hip_status(vc_launch_test_e4m3(x, codes, n, stream));
}

int vc_test_kmeans_assign(const uint16_t* V, const float* C, int B, int H, int N, int d, int k,
                          int32_t* labels, float* mindist, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!V || !C || !labels || !ws) return VC_ERR_NULL;
  if (k < 1 || k > VC_MAX_K || k > N) return VC_ERR_K;
  vc_group_ws L = vc_group_ws_layout(B * H, N, k);
  if (ws_bytes < L.total) return VC_ERR_WORKSPACE;
  char* w = (char*)ws;
  return hip_status(vc_launch_kmeans_assign(V, C, B * H, N, k, labels, mindist, (uint16_t*)(w + L.chi),
                                            (uint16_t*)(w + L.clo), (float*)(w + L.cnorm), true, nullptr,
                                            stream));
}

int vc_test_label_sort(const int32_t* labels, int B, int H, int N, int k, int32_t* perm,
                       int32_t* offsets, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(B, H, N, VC_HEAD_DIM);
  if (st < 0) return st;
  if (st == 1) return VC_OK;
  if (!labels || !perm || !offsets || !ws) return VC_ERR_NULL;
  if (k < 1 || k > VC_MAX_K || k > N) return VC_ERR_K;
  vc_group_ws L = vc_group_ws_layout(B * H, N, k);
  if (ws_bytes < L.total) return VC_ERR_WORKSPACE;
  return hip_status(vc_launch_label_sort(labels, B * H, N, k, (int32_t*)((char*)ws + L.hist),
                                         perm, offsets, false, stream));
}

}  // extern "C"
