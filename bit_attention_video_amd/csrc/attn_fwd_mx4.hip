// Launcher of the 4-bit and 6-bit VC-Attention forward (the kernel is in attn_fwd_mx_kernel.h).
#include "attn_fwd_mx_kernel.h"

hipError_t vc_launch_attn_fwd_mx4(const uint16_t* Q, const uint8_t* Kq4, const uint8_t* sK4,
                                  const uint8_t* Rq4, const uint8_t* sR4, const uint16_t* mu,
                                  int BH, int N, float L4, unsigned flags, uint16_t* O,
                                  int bits, hipStream_t s) {
  const bool no_mean = flags & VC_ATTN_NO_MEAN, had = flags & VC_ATTN_HADAMARD;
  if (bits == 6) {
    if (no_mean && had) return vc_launch_attn_fwd_mx6_rn(Q, Kq4, sK4, Rq4, sR4, mu, BH, N, L4, O, s);
    if (no_mean) return launch_attn_mx<6, true, false>(Q, Kq4, sK4, Rq4, sR4, mu, BH, N, L4, O, s);
    if (had) return launch_attn_mx<6, false, true>(Q, Kq4, sK4, Rq4, sR4, mu, BH, N, L4, O, s);
    return launch_attn_mx<6, false, false>(Q, Kq4, sK4, Rq4, sR4, mu, BH, N, L4, O, s);
  }
  if (no_mean && had) return launch_attn_mx<4, true, true>(Q, Kq4, sK4, Rq4, sR4, mu, BH, N, L4, O, s);
  if (no_mean) return launch_attn_mx<4, true, false>(Q, Kq4, sK4, Rq4, sR4, mu, BH, N, L4, O, s);
  if (had) return launch_attn_mx<4, false, true>(Q, Kq4, sK4, Rq4, sR4, mu, BH, N, L4, O, s);
  return launch_attn_mx<4, false, false>(Q, Kq4, sK4, Rq4, sR4, mu, BH, N, L4, O, s);
}
