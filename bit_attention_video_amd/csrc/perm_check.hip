// Validation of a caller's permutation pi (the joint key/value order of Sec. 3.2, Eq. 3): per
// (b, h), the number of entries that lie outside [0, N) or repeat a value already seen.  Zero
// means pi is a permutation of 0..N-1 (N entries, none out of range, none repeated).  Each
// repeated value with c occurrences adds c - 1 whatever the order in which the atomics land,
// so the count is deterministic.
#include "vc_common.h"
#include "vc_internal.h"

// Clears the bitmap and the counts (a fill kernel, not a memset, so a captured graph replays it).
__global__ void k_perm_clear(uint32_t* __restrict__ bits, int32_t* __restrict__ bad, size_t nwords, int BH) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < nwords; i += stride) bits[i] = 0u;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < (size_t)BH; i += stride) bad[i] = 0;
}

__global__ __launch_bounds__(256) void k_perm_mark(const int32_t* __restrict__ perm, int N, int words,
                                                   uint32_t* __restrict__ bits, int32_t* __restrict__ bad) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  bool fault = false;
  if (i < N) {
    const int v = perm[(size_t)bh * N + i];
    if ((unsigned)v >= (unsigned)N) {
      fault = true;
    } else {
      const uint32_t m = 1u << (v & 31);
      fault = (atomicOr(&bits[(size_t)bh * words + (v >> 5)], m) & m) != 0u;
    }
  }
  const uint64_t b = __ballot(fault);
  if ((threadIdx.x & 63) == 0 && b) atomicAdd(&bad[bh], (int)__popcll(b));
}

hipError_t vc_launch_validate_perm(const int32_t* perm, int BH, int N, uint32_t* bits, int32_t* bad, hipStream_t s) {
  const int words = (N + 31) / 32;
  const size_t nwords = (size_t)BH * words;
  size_t g = (nwords + 255) / 256;
  if (g < 1) g = 1;
  if (g > 4096) g = 4096;
  hipLaunchKernelGGL(k_perm_clear, dim3((unsigned)g), dim3(256), 0, s, bits, bad, nwords, BH);
  hipLaunchKernelGGL(k_perm_mark, dim3((N + 255) / 256, BH), dim3(256), 0, s, perm, N, words, bits, bad);
  return hipGetLastError();
}
