/*
 * vc_attn.h -- C ABI of the VC-Attention hot path for AMD Instinct MI355X (gfx950).
 *
 * Method: "VC-Attention: Value Smoothing and Softmax Casting for Low-bit Attention"
 * (arXiv 2609.15810).  Non-causal FP8 attention forward with
 *   V-Smooth   -- k-means grouping of value tokens, joint K/V permutation, 128-row
 *                 block demeaning, E4M3 residuals, mean restored from the softmax
 *                 row sum (Sec. 3.2, Eq. 3-6; App. B), and
 *   ExpCast-FP8 -- the E4M3 probability byte written from the log-domain score by one
 *                 FMA and one integer conversion (Sec. 3.3, Eq. 7).
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *     allocates or frees device memory; scratch space comes in through `ws`.
 *   - Layout is [B, H, N, d] row-major and contiguous unless stated otherwise.
 *     bf16 tensors are passed as their 16-bit patterns (uint16_t).
 *   - d must be 128 (VC_HEAD_DIM) and N a multiple of 128 (VC_BLOCK): the method's
 *     hardware block is 128 rows (Sec. 3.2, Eq. 4) and padding is the caller's job
 *     (App. B fuses it into the quantisers upstream).
 *   - B * H * N * d must be below 2^31.
 *   - B == 0, H == 0 or N == 0 is an empty problem: VC_OK, nothing touched.
 *   - Every call validates its arguments on the host before any HIP call and
 *     returns VC_OK (0) or a negative vc_status.  Work is enqueued asynchronously on
 *     `stream`; nothing synchronises.  A failed launch returns VC_ERR_HIP and the
 *     hipError_t is available from vc_last_hip_error() (per calling thread).
 *   - Calls are re-entrant; there is no global state besides that error slot.
 *   - Results are deterministic: no floating-point atomics, fixed reduction orders.
 */
#ifndef VC_ATTN_H
#define VC_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum vc_status {
  VC_OK = 0,
  VC_ERR_NULL = -1,       /* a required pointer is NULL */
  VC_ERR_SHAPE = -2,      /* negative size, d != 128 or N % 128 != 0 */
  VC_ERR_K = -3,          /* k outside [1, min(256, N)] */
  VC_ERR_ITERS = -4,      /* iters < 1 */
  VC_ERR_WORKSPACE = -5,  /* ws_bytes below the size the matching *_workspace_size returns */
  VC_ERR_OVERFLOW = -6,   /* B * H * N * d >= 2^31 */
  VC_ERR_FLAGS = -7,      /* unknown flag bits */
  VC_ERR_HIP = -8         /* a HIP call failed; see vc_last_hip_error() */
};

#define VC_HEAD_DIM 128
#define VC_BLOCK 128
#define VC_MAX_K 256

/* vc_attn_fwd flags */
#define VC_ATTN_NO_MEAN 0x1u     /* drop the r * mu term of Eq. 6 (the plain low-bit kernel) */
#define VC_ATTN_EXP_THEN_CAST 0x2u  /* P by exp2 then an E4M3 cast instead of ExpCast (Sec. 3.3's
                                       "exp-then-cast" comparator, Table 4's naive FP8) */
#define VC_ATTN_HADAMARD 0x4u    /* rotate Q L by H before quantising (App. B's Q pass, the fused
                                    QK Hadamard of Sec. 4.1); pair with VC_DQ_HADAMARD keys */
/* vc_workspace_size operations */
#define VC_OP_GROUP 1             /* vc_vsmooth_group (uses k) */
#define VC_OP_DEMEAN_QUANT 2      /* vc_vsmooth_demean_quant */
#define VC_OP_DEMEAN_QUANT_MX4 3  /* vc_vsmooth_demean_quant_mx4 */
#define VC_OP_ATTN_FWD 4          /* vc_attn_fwd (needs none: 0) */
#define VC_OP_ATTN_FWD_MX4 5      /* vc_attn_fwd_mx4 (needs none: 0) */
#define VC_OP_VALIDATE_PERM 6     /* vc_validate_perm */
#define VC_OP_DEMEAN_QUANT_MX6 7  /* vc_vsmooth_demean_quant_mx6 */
#define VC_OP_ATTN_FWD_MX6 8      /* vc_attn_fwd_mx6 (needs none: 0) */
/* vc_vsmooth_demean_quant flags */
#define VC_DQ_NO_DEMEAN 0x1u     /* mu = 0: quantise V' itself (unsmoothed per-channel baseline) */
#define VC_DQ_HADAMARD 0x2u      /* quantise the rotated keys K' H, scale / 128 (App. B's K pass) */

/* Human-readable name of a vc_status. Never NULL. */
const char* vc_strerror(int status);

/* hipError_t of the last VC_ERR_HIP returned on the calling thread (0 if none). */
int vc_last_hip_error(void);

/* Bytes of scratch the call `op` (VC_OP_*) needs for this shape, 256-byte aligned; one entry for
 * all calls (the per-call *_workspace_size functions give the same numbers).  0 when the call
 * needs none, for an empty shape, for d != 128 or for an unknown op.  k is used by VC_OP_GROUP
 * only (an invalid k sizes for k = 256; the call itself then rejects it). */
size_t vc_workspace_size(int op, int B, int H, int N, int d, int k);

/* ------------------------------------------------------------------------------------------
 * Grouping: k-means over value tokens and the label sort (Sec. 3.2, "Value-guided
 * permutation", Eq. 3).
 *
 * Per (b, h), batch Lloyd k-means over the N value rows: `iters` rounds of
 *   assign: z_t = argmin_c ||v_t - c_c||^2 (ties to the lowest c), then
 *   update: c_c = mean of the rows labelled c (an empty cluster keeps its centroid).
 * Start: C_init when non-NULL (warm start, [B,H,k,d] float32), else the rows
 * floor((c + 1/2) N / k) of V.  Then pi = stable argsort(z) (ties keep token order).
 *
 *   V        in   bf16 [B,H,N,d]
 *   C_init   in   float32 [B,H,k,d] or NULL
 *   C_out    out  float32 [B,H,k,d]   centroids after the last update (may alias C_init)
 *   labels   out  int32 [B,H,N]       labels of the last assignment
 *   perm     out  int32 [B,H,N]       pi: perm[i] = token at sorted position i
 *   offsets  out  int32 [B,H,k+1]     start of each cluster's run in pi; offsets[k] = N
 *   objective out float64 [B,H]       J = sum_t ||v_t - c_{z_t}||^2 with the final labels and
 *                                     centroids (may be NULL)
 *   ws       scratch of at least vc_group_workspace_size(B,H,N,k) bytes, 256-byte aligned
 * The assignment takes the argmax of v.c - ||c||^2 / 2 (the same order as the distance),
 * accumulated in float32 from -||c||^2 / 2 and bf16 x (bf16 hi + bf16 lo split of the float32
 * centroid) matrix products; centroid sums are float64 in a fixed order, and J is formed in
 * float64 from the last update's own sums (sum ||v||^2 - 2 c.S + n ||c||^2 per cluster).
 * -------------------------------------------------------------------------------------- */
size_t vc_group_workspace_size(int B, int H, int N, int k);
int vc_vsmooth_group(const uint16_t* V, int B, int H, int N, int d, int k, int iters,
                     const float* C_init, float* C_out, int32_t* labels, int32_t* perm,
                     int32_t* offsets, double* objective, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* vc_vsmooth_group without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, results and errors as vc_vsmooth_group minus ws / ws_bytes; the scratch is a
 * library-held device array of VC_GROUP_STATIC_SCRATCH_BYTES (16 MiB) per GPU, kept until the
 * process ends.  A shape whose grouping workspace (vc_group_workspace_size) exceeds it returns
 * VC_ERR_WORKSPACE before any HIP call (e.g. B*H = 40, N = 70,016, k = 128 needs 5.5 MB;
 * B*H = 24, N = 115,200, k = 256 needs 6.0 MB).  No call allocates or frees.  The first call on a
 * device resolves the array's address (hipGetSymbolAddress; make it outside graph capture).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (different streams
 * or threads without ordering) race and must be serialised by the caller. */
#define VC_GROUP_STATIC_SCRATCH_BYTES (16u << 20)
int vc_vsmooth_group_static(const uint16_t* V, int B, int H, int N, int d, int k, int iters,
                            const float* C_init, float* C_out, int32_t* labels, int32_t* perm,
                            int32_t* offsets, double* objective, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Smoothing and quantisation of K and V in permuted order (Sec. 3.2 Eq. 3-4; App. B).
 *
 * K path: kbar = float32(sum_t K[t] / N) (key channel mean, sum exact in float64);
 *   K' = K[pi] - kbar (float32); per 128-row block j: sK[j] = 2^E, the smallest power of two
 *   with amax|K'_j| <= 448 sK[j] (1 if 0, E >= -100); Kq = E4M3_RNE(K' / sK[j]) in
 *   [B,H,N,d], rows in permuted order (the division by a power of two is exact).
 * V path: V' = V[pi]; mu_j = float32(sum of the 128 rows of block j / 128);
 *   R = V' - mu_j (float32); sV[c] = amax_t |R[t,c]| / 448 over all N rows (1 if 0);
 *   Rq = E4M3_RNE(R / sV[c]); mu_out[j][c] = bf16_RNE(mu_j[c] / sV[c]).
 *   Flag VC_DQ_NO_DEMEAN sets mu = 0 (quantise V' itself).
 * Flag VC_DQ_HADAMARD (App. B's K pass with the QK rotation; Sec. 4.1 "Baselines"): the
 *   blocks of Y = float32(K' H) are quantised instead of K', with H the Sylvester Hadamard
 *   matrix of order 128 (H[r][c] = (-1)^popcount(r & c)); each Y element is the float32
 *   rounding of the signed sum of 128 float32 terms, taken in float64 (exact unless a row's
 *   terms span more than about 22 binades).  sK[j] = 2^(E-7) with 2^E the scale of block j
 *   of Y, so Kq * sK = K' H / 128 = K' H^-T and the scores are those of unrotated keys once
 *   the queries are rotated by H (vc_attn_fwd's VC_ATTN_HADAMARD).
 * Every division is one correctly rounded float32 division; E4M3 is OCP E4M3FN with
 * round-to-nearest-even (|x| <= 448 by construction).
 *
 *   K, V     in   bf16 [B,H,N,d]
 *   perm     in   int32 [B,H,N] permutation of 0..N-1 per (b,h), or NULL for identity.
 *                 Entries are not validated here (vc_validate_perm does that); an entry outside
 *                 [0, N) is read as token 0, so every gather stays inside the head's rows, and a
 *                 repeated entry repeats its token: the outputs are then not those of any
 *                 permutation, but nothing outside K and V is read.
 *   Kq       out  E4M3 bytes [B,H,N,d]
 *   sK       out  float32 [B,H,N/128]
 *   Rq       out  E4M3 bytes, TILE-TRANSPOSED: [B,H,N/128][d][128 slots].  Within tile j,
 *                 slot s of channel c holds residual code of permuted row 128 j + key(s) with
 *                 key(s) = 64 p + 32 (i / 16) + 8 ((i % 16) / 4) + 4 g + (i % 4) for
 *                 s = 64 p + 32 g + i (p, g in {0,1}, i in [0,32)).  This is the operand order
 *                 of the PV matrix instruction in vc_attn_fwd.
 *   mu_out   out  bf16 [B,H,N/128,d]  block means divided by sV (App. B)
 *   sV       out  float32 [B,H,d]
 *   ws       scratch of at least vc_demean_quant_workspace_size(B,H,N) bytes, 256-byte aligned
 * -------------------------------------------------------------------------------------- */
size_t vc_demean_quant_workspace_size(int B, int H, int N);
int vc_vsmooth_demean_quant(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                            int B, int H, int N, int d, unsigned flags,
                            uint8_t* Kq, float* sK, uint8_t* Rq, uint16_t* mu_out, float* sV,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * FP8 attention forward with ExpCast-FP8 and the online mean restore
 * (Sec. 3.1 Eq. 1; Sec. 3.2 Eq. 6; Sec. 3.3 Eq. 7; App. B).
 *
 * Per (b,h) and query row i (original order; Q is never permuted), over key tiles
 * j = 0 .. N/128-1 of the permuted keys:
 *   L = float32(8 log2(e) softmax_scale);  per Q block of 128 rows: X = float32(Q L)
 *   (VC_ATTN_HADAMARD: X = float32(float32(Q L) H), H and its rounding as for VC_DQ_HADAMARD),
 *   sQ = 2^E the smallest power of two with amax|X| <= 448 sQ (1 if 0, E >= -100),
 *   Qq = E4M3_RNE(X / sQ)
 *   s = Qq . Kq_j (FP8 matrix instruction, float32 accumulate);  a = sQ sK[j] (exact)
 *   m' = max(m, a max_k s);  b = float32(119.65 - m')
 *   code = clip(RNE(a s + b), 0, 120)  -- the E4M3 byte of P, 2^8 = row maximum
 *     (VC_ATTN_EXP_THEN_CAST: code = E4M3_RNE(2^((a s - m')/8 + 8)))
 *   r = sum of decoded codes;  alpha = 2^((m - m')/8)
 *   A = alpha A + P Rq_j + r mu_j;  l = alpha l + r     (mu term dropped by VC_ATTN_NO_MEAN)
 *   O = bf16_RNE(sV * A / l)
 * a s + b is the accumulator of the scaled FP8 matrix instruction seeded with b (one float32
 * result per element), so it matches the float32 FMA of the formula up to the instruction's
 * internal summation order.
 *
 *   Q        in   bf16 [B,H,N,d]
 *   Kq, sK, Rq, mu, sV   in   as written by vc_vsmooth_demean_quant
 *   softmax_scale        0 means 1/sqrt(d); must be finite and >= 0 (else VC_ERR_SHAPE)
 *   flags    VC_ATTN_NO_MEAN | VC_ATTN_EXP_THEN_CAST | VC_ATTN_HADAMARD (others: VC_ERR_FLAGS).
 *            VC_ATTN_HADAMARD needs keys written with VC_DQ_HADAMARD and the reverse; a mixed
 *            pair is not detected and gives the scores of a different operator.
 *   O        out  bf16 [B,H,N,d]
 * -------------------------------------------------------------------------------------- */
int vc_attn_fwd(const uint16_t* Q, const uint8_t* Kq, const float* sK, const uint8_t* Rq,
                const uint16_t* mu, const float* sV, int B, int H, int N, int d,
                float softmax_scale, unsigned flags, uint16_t* O, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * 4-bit V-Smooth on MX formats (Sec. 3.2 after Eq. 4: the residual goes through the host
 * kernel's 4-bit value quantiser; Sec. 4.1 "Implementation" and App. A "Scope of ExpCast-FP8":
 * 4 bits run V-Smooth alone, P by exponentiation; App. B: the microscales act inside the
 * matrix instruction, so the means are added unscaled).  The pages' 4-bit format is NVFP4;
 * MI355X's matrix instructions take MX scales, so this path uses E2M1 elements with one E8M0
 * scale per 32 elements along each product's reduction axis.
 *
 * E2M1: sign, 2-bit exponent (bias 1), 1-bit mantissa; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 * Group scale 2^E: the smallest power of two with amax <= 6 * 2^E (E >= -100, E = 0 for an
 * all-zero group), stored as the byte E + 127; elements E2M1_RNE(x / 2^E), two per byte, the
 * even index in the low nibble.
 *
 * vc_vsmooth_demean_quant_mx4: the K and V paths of vc_vsmooth_demean_quant with 4-bit outputs.
 *   K' = float32(K[pi] - kbar) (VC_DQ_HADAMARD: float32(K' H), exponent stored minus 7);
 *     Kq4 [B,H,N,64]: codes of each permuted row; sK4 [B,H,N,4]: the scale byte of channel
 *     group c/32.
 *   V' = V[pi]; mu_j = float32(block sum / 128) (0 with VC_DQ_NO_DEMEAN); R = V' - mu_j;
 *     Rq4 [B,H,N/128][128 channels][64]: tile-transposed like Rq (slot s of channel c holds
 *     the residual of row 128 j + key(s), two slots per byte); sR4 [B,H,N/128][128][4]: the
 *     scale of slots 32 g .. 32 g + 31 (in key terms: the keys of one 64-key half with equal
 *     index bit 2); mu_out bf16 [B,H,N/128,128] = bf16_RNE(mu_j), unscaled.
 *   ws: vc_demean_quant_workspace_size(B,H,N) bytes.  flags: VC_DQ_NO_DEMEAN | VC_DQ_HADAMARD.
 *
 * vc_attn_fwd_mx4: per (b,h) and query row, over key tiles j of 128 permuted keys:
 *   L4 = float32(log2(e) softmax_scale); X = float32(Q L4) (rotated by H with
 *   VC_ATTN_HADAMARD), E2M1 per 32-channel group of the row;
 *   S = sum over the 4 channel groups of (decoded Q x its scale)(decoded K x its scale), float32
 *   matrix-instruction accumulation; m' = max(m, max S); P = 2^(S - m'), float32 exp2;
 *   P in E2M1 per 32-key group (the groups of Rq4); r = sum of the dequantised P;
 *   alpha = 2^(m - m'); A = alpha A + P Rq_j + r mu_j; l = alpha l + r; O = bf16_RNE(A / l).
 *   flags: VC_ATTN_NO_MEAN | VC_ATTN_HADAMARD (others: VC_ERR_FLAGS); mu may be NULL only with
 *   VC_ATTN_NO_MEAN; softmax_scale as vc_attn_fwd.
 * -------------------------------------------------------------------------------------- */
int vc_vsmooth_demean_quant_mx4(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                int B, int H, int N, int d, unsigned flags,
                                uint8_t* Kq4, uint8_t* sK4, uint8_t* Rq4, uint8_t* sR4,
                                uint16_t* mu_out, void* ws, size_t ws_bytes, hipStream_t stream);
int vc_attn_fwd_mx4(const uint16_t* Q, const uint8_t* Kq4, const uint8_t* sK4, const uint8_t* Rq4,
                    const uint8_t* sR4, const uint16_t* mu, int B, int H, int N, int d,
                    float softmax_scale, unsigned flags, uint16_t* O, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * 6-bit V-Smooth on MX formats: the 4-bit path above with E2M3 elements (OCP MX FP6) instead
 * of E2M1, on the same matrix instructions (App. B's microscaled value quantiser, Sec. 3.2
 * after Eq. 4; the MX element width MI355X offers between FP4 and FP8).
 *
 * E2M3: sign, 2-bit exponent (bias 1), 3-bit mantissa; magnitudes m/8 (m < 8), then 1 to 1.875,
 * 2 to 3.75, 4 to 7.5 in steps of 1/8, 1/4, 1/2.  Group scale 2^E: the smallest power of two
 * with amax <= 7.5 * 2^E (E >= -100, E = 0 for an all-zero group), stored as the byte E + 127;
 * elements E2M3_RNE(x / 2^E).  A group of 32 elements has 24 code bytes, element k in bits
 * 6k .. 6k + 5 of its 192-bit little-endian field.  The four groups of a 128-byte operand row are
 * stored with the first 16 code bytes of group g at byte 16 g and its last 8 at byte
 * 64 + 16 (g % 2) + 8 (g / 2) (the last 8 of groups 0 and 2 in bytes 64 .. 79, of groups 1 and 3
 * in bytes 80 .. 95); bytes 96 .. 127 are zero.
 *
 * vc_vsmooth_demean_quant_mx6: as vc_vsmooth_demean_quant_mx4, with
 *   Kq6 [B,H,N,128]: the four 32-channel groups of each permuted row; sK6 [B,H,N,4];
 *   Rq6 [B,H,N/128][128 channels][128]: the four 32-slot groups of each channel (slot order
 *     as Rq4); sR6 [B,H,N/128][128][4]; mu_out bf16 [B,H,N/128,128] = bf16_RNE(mu_j).
 *   ws: vc_demean_quant_workspace_size(B,H,N) bytes.  flags: VC_DQ_NO_DEMEAN | VC_DQ_HADAMARD.
 *
 * vc_attn_fwd_mx6: vc_attn_fwd_mx4's recurrence with E2M3 operands (Q per 32 channels, P per
 *   32-key group); flags, mu and softmax_scale as vc_attn_fwd_mx4.
 * -------------------------------------------------------------------------------------- */
int vc_vsmooth_demean_quant_mx6(const uint16_t* K, const uint16_t* V, const int32_t* perm,
                                int B, int H, int N, int d, unsigned flags,
                                uint8_t* Kq6, uint8_t* sK6, uint8_t* Rq6, uint8_t* sR6,
                                uint16_t* mu_out, void* ws, size_t ws_bytes, hipStream_t stream);
int vc_attn_fwd_mx6(const uint16_t* Q, const uint8_t* Kq6, const uint8_t* sK6, const uint8_t* Rq6,
                    const uint8_t* sR6, const uint16_t* mu, int B, int H, int N, int d,
                    float softmax_scale, unsigned flags, uint16_t* O, hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Validation of a caller's permutation (Sec. 3.2, Eq. 3: pi must reorder the N keys and values
 * of each (b,h) jointly, without loss or repetition).
 *
 *   perm  in   int32 [B,H,N]
 *   bad   out  int32 [B,H] (device): per (b,h) the number of entries outside [0, N) plus, for
 *              every value that occurs c > 1 times, c - 1.  0 exactly when perm[b,h] is a
 *              permutation of 0..N-1.  Deterministic.
 *   ws    scratch of vc_workspace_size(VC_OP_VALIDATE_PERM, B, H, N, 128, 0) bytes
 * Errors: VC_ERR_SHAPE for negative sizes, VC_ERR_OVERFLOW for B*H*N >= 2^31, VC_ERR_NULL,
 * VC_ERR_WORKSPACE.  Every read stays inside perm.
 * -------------------------------------------------------------------------------------- */
int vc_validate_perm(const int32_t* perm, int B, int H, int N, int32_t* bad, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* ------------------------------------------------------------------------------------------
 * Test hooks: single stages of the path, exposed so each can be checked on its own.
 * -------------------------------------------------------------------------------------- */

/* ExpCast code of Eq. 7 for float32 u: clip(RNE(fma(8, u, 119.65f)), 0, 120); NaN -> 0.
 * Same rounding and clip instruction sequence as vc_attn_fwd.  u, codes: device, n elements. */
int vc_test_expcast(const float* u, uint8_t* codes, size_t n, hipStream_t stream);

/* E4M3 (OCP E4M3FN) round-to-nearest-even of float32 x, saturating to +-448, as the
 * quantisers of vc_vsmooth_demean_quant and vc_attn_fwd do it. */
int vc_test_e4m3_encode(const float* x, uint8_t* codes, size_t n, hipStream_t stream);

/* E2M1 codes of float32 pairs as the 4-bit quantisers pack them: codes[i] holds x[2i] in the
 * low and x[2i+1] in the high nibble (round to nearest even, |x| <= 6 expected: the callers
 * divide by the group scale first).  n (the number of floats) must be even (VC_ERR_SHAPE). */
int vc_test_fp4_encode(const float* x, uint8_t* codes, size_t n, hipStream_t stream);

/* E2M3 codes of groups of 32 float32 values as the 6-bit paths pack them: words[6i .. 6i+5]
 * (uint32, device) hold the codes of x[32i .. 32i+31], value k in bits 6k .. 6k+5 of the
 * 192-bit little-endian field.  With scale NULL the values are converted as they are (the
 * quantisers divide by the group scale first, |x| <= 7.5 expected); otherwise scale[i]
 * (float32, device, a power of two) is the conversion's own scale operand, which divides
 * (the 6-bit attention converts P that way).  Round to nearest even. */
int vc_test_fp6_encode(const float* x, const float* scale, uint32_t* words, size_t ngroups, hipStream_t stream);

/* One k-means assignment with given centroids C [B,H,k,d] float32 (the assign step of
 * vc_vsmooth_group): labels int32 [B,H,N]; mindist float32 [B,H,N] (||v - c_z||^2 as the
 * kernel computed it, may be NULL).  ws: at least vc_group_workspace_size(B,H,N,k) bytes. */
int vc_test_kmeans_assign(const uint16_t* V, const float* C, int B, int H, int N, int d, int k,
                          int32_t* labels, float* mindist, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Stable counting sort of labels int32 [B,H,N] with values in [0,k): perm, offsets as in
 * vc_vsmooth_group.  ws: at least vc_group_workspace_size(B,H,N,k) bytes. */
int vc_test_label_sort(const int32_t* labels, int B, int H, int N, int k, int32_t* perm,
                       int32_t* offsets, void* ws, size_t ws_bytes, hipStream_t stream);

/* Dense FP8 matrix-instruction rate, for quoting the attention kernel's fraction of the FP8
 * peak this device actually attains beside the vendor figure: `workgroups` workgroups of 512
 * threads, each of whose 8 waves issues `iters` x 4 independent 32x32x64 E4M3 products (the
 * instruction vc_attn_fwd uses) on fixed pseudo-random operands (data that toggles the
 * multipliers as real operands do), i.e. workgroups x iters x 4,194,304 FLOP.  The caller times
 * the call on `stream`.  out: device float32 [workgroups * 512], written (one value per
 * thread keeps the products live).  clock_mhz: NULL, or device float32 [workgroups] that
 * receives, per workgroup, the shader clock in MHz over its first wave's loop (shader-cycle
 * counter over the constant-rate counter, scaled by hipDeviceAttributeWallClockRate): the
 * clock the matrix unit sustained.  VC_ERR_NULL for a null out, VC_ERR_SHAPE for
 * workgroups < 1, iters < 1 or a FLOP count beyond 2^62, VC_ERR_HIP if the counter rate
 * cannot be read. */
int vc_test_mfma_fp8_rate(float* out, int workgroups, int iters, float* clock_mhz, hipStream_t stream);

/* The query prologue of vc_attn_fwd run on its own (App. B's Q pass; row a8 of the path): per
 * 128-row block of X = float32(Q L) (rotated by H with VC_ATTN_HADAMARD), sQ = 2^E the smallest
 * power of two with amax|X| <= 448 sQ, Qq = E4M3_RNE(X / sQ), with the kernel's own code.
 *   Qq out E4M3 bytes [B,H,N,d] (natural layout);  sQ out float32 [B,H,N/128].
 * flags: VC_ATTN_HADAMARD only.  softmax_scale as vc_attn_fwd. */
int vc_test_quantize_q(const uint16_t* Q, int B, int H, int N, int d, float softmax_scale, unsigned flags,
                       uint8_t* Qq, float* sQ, hipStream_t stream);

/* Clock probe of the attention kernel: vc_attn_fwd's kernel with its stamps switched on.  The
 * first wave of workgroup g reads the shader-cycle counter (s_memtime) and the constant-rate
 * counter (s_memrealtime, hipDeviceAttributeWallClockRate ticks per second) at its start and at
 * its end and writes them to clk[4 g .. 4 g + 3] = (cycles, ticks) at the start, then at the
 * end (uint64, device), so sum(cycles) / sum(ticks) x rate over the workgroups is the shader
 * clock the kernel ran at.  O and every other argument as vc_attn_fwd; clk needs
 * vc_test_attn_clock_slots(B,H,N) entries. */
size_t vc_test_attn_clock_slots(int B, int H, int N);
/* Rate of the constant-rate counter of the current device in kHz (hipDeviceAttributeWallClockRate),
 * into *khz.  VC_ERR_NULL for a null khz, VC_ERR_HIP if the attribute cannot be read. */
int vc_test_wall_clock_khz(int* khz);
int vc_test_attn_fwd_clock(const uint16_t* Q, const uint8_t* Kq, const float* sK, const uint8_t* Rq,
                           const uint16_t* mu, const float* sV, int B, int H, int N, int d,
                           float softmax_scale, unsigned flags, uint16_t* O, uint64_t* clk, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VC_ATTN_H */
