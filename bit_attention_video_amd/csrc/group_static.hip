// Grouping with library-held scratch: vc_vsmooth_group for callers that cannot allocate device
// memory (code under graph capture, serving loops, harnesses that forbid hipMalloc).  The scratch
// lives in a file-scope device array of fixed size; each GPU holds its own copy until the process
// ends.  Its device address is resolved once per device with hipGetSymbolAddress (in host code
// the array's name is only a host-side stand-in) and kept; kernels receive that address.
#include "vc_attn.h"
#include "vc_internal.h"

#include <hip/hip_runtime.h>
#include <mutex>

static __device__ __align__(256) uint8_t scratch[VC_GROUP_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, resolved on the first use per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int vc_vsmooth_group_static(const uint16_t* V, int B, int H, int N, int d, int k, int iters,
                                       const float* C_init, float* C_out, int32_t* labels, int32_t* perm,
                                       int32_t* offsets, double* objective, hipStream_t stream) {
  // the argument checks of vc_vsmooth_group, on the host before any HIP call, plus the size limit
  if (B < 0 || H < 0 || N < 0 || d != VC_HEAD_DIM || N % VC_BLOCK != 0) return VC_ERR_SHAPE;
  if (B == 0 || H == 0 || N == 0) return VC_OK;
  if ((long long)B * H * (long long)N * d >= (1LL << 31)) return VC_ERR_OVERFLOW;
  if (!V || !C_out || !labels || !perm || !offsets) return VC_ERR_NULL;
  if (k < 1 || k > VC_MAX_K || k > N) return VC_ERR_K;
  if (iters < 1) return VC_ERR_ITERS;
  const size_t need = vc_group_workspace_size(B, H, N, k);
  if (need > (size_t)VC_GROUP_STATIC_SCRATCH_BYTES) return VC_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return vc_hip_status(e);
  return vc_vsmooth_group(V, B, H, N, d, k, iters, C_init, C_out, labels, perm, offsets, objective, ws,
                          (size_t)VC_GROUP_STATIC_SCRATCH_BYTES, stream);
}
