// The rotated (Hadamard) no-mean instantiation of the 6-bit VC-Attention forward, in a
// translation unit of its own because the library builds it at -O2: the -O3 code of this one
// instantiation gave wrong outputs on the device (the other seven, and this one at -O2, match
// the emulated reference), and -O2 for the whole kernel file would slow the default 6-bit kernel
// by about 3%.
#include "attn_fwd_mx_kernel.h"

hipError_t vc_launch_attn_fwd_mx6_rn(const uint16_t* Q, const uint8_t* Kq6, const uint8_t* sK6,
                                     const uint8_t* Rq6, const uint8_t* sR6, const uint16_t* mu, int BH, int N, float L4,
                                     uint16_t* O, hipStream_t s) {
  return launch_attn_mx<6, true, true>(Q, Kq6, sK6, Rq6, sR6, mu, BH, N, L4, O, s);
}
