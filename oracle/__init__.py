"""CPU oracle for VC-Attention (test infrastructure only).

A plain, slow, obviously-correct numpy implementation of what the VC-Attention
hot path computes, written from the paper "VC-Attention: Value Smoothing and
Softmax Casting for Low-bit Attention" (arXiv 2609.15810).  It shares no code
with the HIP library: it imports neither the package ``bit_attention_video_amd``
nor anything it builds.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.

Floating point is float64 unless the method fixes a precision.  Where a float
decides an integer (an E4M3 code, an ExpCast code) the decision is taken in
float32 with the operation order the kernels use, so both sides round the
same number.

Modules
  formats   E4M3 (OCP E4M3FN), E2M1 and E2M3 codecs, bf16 rounding, float32 rounding
  expcast   ExpCast-FP8 code c(u) (Sec. 3.3, Eq. 7) and the exp-then-cast code
  analysis  closed forms of App. C/D (Mitchell error, ratio bounds, TV bound)
  vsmooth   k-means grouping, stable label sort, K smoothing and V block
            demeaning with E4M3 quantisation (Sec. 3.2, Eq. 3-5; App. B)
  rotation  the QK Hadamard rotation fused into the Q/K quantisers (Sec. 4.1, App. B)
  mx4       4-bit V-Smooth on MX E2M1 elements (and 6-bit on E2M3) with per-32
            power-of-two scales (Sec. 3.2 after Eq. 4, Sec. 4.1 "Implementation", App. A,
            App. B)
  attention exact softmax attention and the emulated tiled VC attention
            (Sec. 3.1 Eq. 1, Sec. 3.2 Eq. 6, Sec. 3.3 Eq. 7)
  diagnostics  the error split of Eq. 2, block-mean energy shares and value error by
            token order (Sec. 3.2, Eq. 5, Table 1), row total variation (Sec. 3.3)

Parity pins live in tests/test_oracle_*.py.  The emulated tiled attention has
no printed worked example on the pages; it is pinned by its reductions (exact
arithmetic -> exact attention; ExpCast row bound of Prop. 3.1; mean-restore
identity), not by printed values.
"""
from . import formats, expcast, analysis, rotation, vsmooth, attention, mx4, diagnostics  # noqa: F401
