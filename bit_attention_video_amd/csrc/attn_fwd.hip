// FP8 VC-Attention forward on gfx950 (VC-Attention Sec. 3.1 Eq. 1, Sec. 3.2 Eq. 6,
// Sec. 3.3 Eq. 7, App. B).
//
// One workgroup = 8 waves in two groups of four; group g owns the 128-row query block
// 2 wb + g of one (b, h) and each of its waves owns 32 of those queries.  Keys/values stream
// in tiles of 128 (= B_v, so each tile has one key scale sK_j and one mean mu_j) through
// LDS, filled by direct global->LDS copies that every wave shares.
//
// Ping-pong between the two groups.  Per tile a wave has a matrix part M(j) -- the PV
// product and the row sum of tile j-1, then the QK product of tile j, then the bookkeeping of
// that row sum (l and the mean term's shift register) while the products run -- and a vector
// part V(j): the running maximum and the ExpCast codes of tile j, each key half of codes
// followed by the read of the next PV product's residual fragments for that half into the
// registers its scores just freed.  The groups run them in
// opposite phases separated by workgroup barriers (group 0: M(j) | V(j), group 1:
// V(j-1) | M(j)).  A SIMD holds one wave of each group, so while one of them keeps the
// matrix unit busy the other does the vector work; with one workgroup per CU nothing else
// competes.  K and R tiles are copied three steps ahead into a four-deep LDS ring whose slots
// hold a K and an R tile side by side; each wave issues its share of the copies in its vector
// phase, away from the matrix instructions.
//
// Layouts.  Both products use the FP8 32x32x64 matrix instruction with the key index as the
// reduction dimension of PV, computed transposed so one lane owns one query row:
//   S^T (keys x queries) = Kq_j (keys x d) . Qq^T (d x queries)
//   O^T (d x queries)   += Rq_j^T (d x keys) . P^T (keys x queries)
// In the 32x32 result layout lane (q = lane%32, h = lane/32) holds column q and rows
// 8(i/4) + 4h + i%4 (i = 0..15), so every score, row statistic and output element of a
// lane belongs to query q; the lanes q and q+32 share a row and exchange one value.
// The P bytes a lane produces are exactly its B-operand bytes for PV once the residual
// tile is stored in the matching key order (vc_vsmooth_demean_quant's tile-transposed Rq).
//
// ExpCast inside the matrix unit.  The query block is quantised as E4M3(Q L / sQ) with
// L = float32(8 log2(e) softmax_scale), and sQ, sK_j are powers of two (E8M0), so the scaled
// FP8 instruction with block scales sK_j and sQ already returns a*s = 8 log2(e) S, the
// score in Eq. 7's units.  Its accumulator input is b = 119.65 - m (the row maximum folded
// into the constant, Fig. 2 caption), so it returns t = a*s + b and Eq. 7 is left with
// Round and clip: one v_cvt_pk_u8_f32 per element (RNE, saturating; t <= 119.65 + ulp, so
// the saturation at 0 is the clip and 120 is never exceeded).
//
// Running maximum (Eq. 1).  With t = a s + C - m, rowmax(t) - C = a*max(s) - m, so a row's
// maximum grows by delta = max(0, rowmax(t) - C); then t, b and m move by -delta, +delta
// and alpha = 2^(-delta/8) rescales A and l.  Rows that do not grow skip all of it: the
// branch is taken per wave only when some row of the wave grew.
//
// Row sum (Eq. 6, r = sum of the decoded codes) on the matrix unit as well: a 16x16x128 FP8
// product of a constant 0/1 operand with the P bytes returns each lane the sum of its
// query's 128 codes (see rowsum_ones).  l += r.  The rank-one mean term r mu~_j^T runs on
// the matrix unit too: each row keeps the r of the current 16-tile group (rescaled with A
// when the maximum grows), and once per group A += mu~^T rho with the bf16 32x32x16
// instruction (mu~ is exact bf16; rho is split into bf16 hi + lo, 16 significant bits).
// Epilogue: O = bf16(A * sV / l) (App. B: one multiply by sV serves both terms).
//
// QK rotation (App. B's Q pass; the fused QK Hadamard of Sec. 4.1): with VC_ATTN_HADAMARD the
// prologue rotates each query row Q L by the Sylvester Hadamard matrix H before taking sQ and
// the codes; the key codes then come from vc_vsmooth_demean_quant's matching K H / 128.
#include "vc_common.h"
#include "vc_internal.h"
#include "vc_attn.h"
#include "attn_common.h"

#include <type_traits>

namespace {

using namespace vc_attn;

constexpr int TILE_BYTES = 128 * 128;
constexpr float EC_C = 119.65f;    // 120 + beta, beta = -0.35 (Eq. 7)
constexpr int NWAVE = 8;           // two groups of four waves
constexpr int MRING = 32;          // LDS ring of mean rows: two 16-tile groups
constexpr int NBUF = 4;            // K and R tile buffers each (prefetch depth NBUF - 1 tiles)

// Byte offset of 16-byte chunk c16 (0..7) of row `row` in a 128 x 128-byte LDS tile.  The
// chunk index is XORed with (row % 8) ^ (row / 8 % 2): rows r..r+7 then hit 8 different
// 16-byte bank groups of a 128-byte bank period, and rows r..r+15 hit 16 different groups
// of a 256-byte period, so the lanes one LDS cycle serves never share a bank.
__device__ __forceinline__ int swz_phys(int row, int c16) { return c16 ^ (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int c16) { return row * 128 + (swz_phys(row, c16) << 4); }

// Source offset (bytes, within a 16 KB tile) of the chunk a lane copies with instruction i
// of wave w: the instruction fills LDS chunks (2w + i) * 64 + lane of the swizzled tile, so
// each lane fetches the global chunk that belongs there (the XOR is an involution).
__device__ __forceinline__ int stage_src(int w, int i, int lane) {
  const int P = (2 * w + i) * 64 + lane;
  const int row = P >> 3;
  return row * 128 + (swz_phys(row, P & 7) << 4);
}

// E4M3 x E4M3 -> float32, operands scaled by 2^(sa-127) and 2^(sb-127) (E8M0 block scales).
__device__ __forceinline__ v16f mfma_fp8(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ v4f mfma_fp8_16(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Constant A operand of the row-sum product D = A . B (16x16x128, FP8).  In that instruction
// lane l holds row / column l%16 and k-block G = l/16 of A / B; the P bytes of lane l (query
// l%32, key half l/32) therefore form k-block G of column n = l%16 with query n + 16 (G%2).
// Rows 0 and 8 of A are ones on k-blocks 0 and 2 (query n), rows 4 and 12 on k-blocks 1 and
// 3 (query n + 16), all else zero; lane l reads row 4 (l/16) in result register 0, which is
// then the sum of its own query's 128 codes.  The codes are multiples of 2^-9 below 2^8, so
// the sum (< 2^15) is exact in float32.
__device__ __forceinline__ int rowsum_ones_word(int lane) {
  const int i = lane & 15, G = lane >> 4;
  const bool one = (G & 1) ? (i == 4 || i == 12) : (i == 0 || i == 8);
  return one ? 0x38383838 : 0;   // four E4M3 1.0
}
// The operand itself: eight copies of the lane's word, built once and kept in registers for
// the whole key loop (opaque, so the compiler keeps it rather than rebuilding it per tile).
__device__ __forceinline__ v8i rowsum_ones(int lane) {
  const int word = rowsum_ones_word(lane);
  v8i r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = word;
  asm volatile("" : "+v"(r));
  return r;
}

}  // namespace

// ETC: P by exp-then-cast (the comparator of Sec. 3.3): the accumulator input is -m instead
// of 119.65 - m, so the instruction returns y = a s - m, and P = E4M3_RNE(2^(y/8 + 8)) with
// v_exp_f32 and the hardware FP8 conversion (y <= 0, so P <= 256 needs no saturation).
template <bool NO_MEAN, bool ETC, bool HAD>
__global__ __launch_bounds__(512) void k_attn_fwd(const uint16_t* __restrict__ Q,
                                                  const uint8_t* __restrict__ Kq,
                                                  const float* __restrict__ sK,
                                                  const uint8_t* __restrict__ Rq,
                                                  const uint16_t* __restrict__ mu,
                                                  const float* __restrict__ sV, int N, int nqb,
                                                  int nwb, uint32_t G, float L, uint16_t* __restrict__ O,
                                                  uint64_t* __restrict__ clk) {
  // ring slot s holds K tile at tiles[s][0] and R tile at tiles[s][1]: one slot base serves both
  __shared__ __attribute__((aligned(1024))) uint8_t tiles[NBUF][2][TILE_BYTES];
  __shared__ __attribute__((aligned(256))) uint16_t mring[MRING][128];
  // first-half row sums of each query row, and b at the time they were saved
  __shared__ float rsnap[9][NWAVE * 32];   // [slot][query of the workgroup]
  __shared__ float red[NWAVE];

  const int t = threadIdx.x, lane = t & 63, q = lane & 31, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = w >> 2;
  // the clock probe (clk non-null): wave 0 stamps the workgroup's start and end
  if (w == 0) clock_stamp(clk ? clk + 4 * blockIdx.x : nullptr);
  const uint32_t item = xcd_remap(blockIdx.x, G);
  const int bh = (int)(item / (uint32_t)nwb), qb = 2 * (int)(item % (uint32_t)nwb) + grp;
  const bool valid = qb < nqb;   // the last block of a head may have no second query block
  const int T = N / 128;
  const size_t headN = (size_t)bh * N;
  const int qi = (valid ? qb : nqb - 1) * 128 + (w & 3) * 32 + q;
  const uint8_t* Kh = Kq + headN * VC_D;
  const uint8_t* Rh = Rq + (size_t)bh * T * TILE_BYTES;
  const uint16_t* muh = mu + (size_t)bh * T * VC_D;
  const float* sKh = sK + (size_t)bh * T;

  // this wave's share of every tile copy: per-lane source offsets, LDS chunk offsets
  const uint32_t so0 = stage_src(w, 0, lane), so1 = stage_src(w, 1, lane);
  const uint32_t kt0 = lds_addr(&tiles[0][0][0]) + 2 * w * 1024, rt0 = kt0 + TILE_BYTES;
  auto stage = [&](const uint8_t* gtile, uint32_t lbase) {
    dma16(gtile, so0, lbase);
    dma16(gtile, so1, lbase + 1024);
  };
  // Copies of step j: K tile j+D, R tile j+D-1 and mean row j+D-1 (D = NBUF-1), with tile
  // indices clamped to T-1 so every step issues the same number of copies per wave (a
  // clamped copy rewrites a buffer whose tile has been used up, or a mean-ring row whose
  // rho is zero).
  constexpr int D = NBUF - 1;
  constexpr int NSET = 4;   // copies per wave and step, plus the mean row on wave 0
  const uint32_t mr0 = lds_addr(&mring[0][0]);
  auto mean_row = [&](int i) {
    if (!NO_MEAN && w == 0) dma4(muh + (size_t)i * VC_D, 4 * lane, mr0 + (i % MRING) * 256);
  };
  auto clampT = [&](int i) { return i < T ? i : T - 1; };
  auto issue = [&](int j) {
    stage(Kh + (size_t)clampT(j + D) * TILE_BYTES, kt0 + ((j + D) % NBUF) * 2 * TILE_BYTES);
    stage(Rh + (size_t)clampT(j + D - 1) * TILE_BYTES, rt0 + ((j + D - 1) % NBUF) * 2 * TILE_BYTES);
    mean_row(clampT(j + D - 1));
  };
  // the end of phase 2j+1: the copies of step j-1 and before (up to K tile j+2, R tile j+1)
  // have landed; step j may still be in flight.  So R tile j+1 is readable from phase 2j+2
  // on, in time for V(j+1), which reads the fragments of PV(j+1) ahead of M(j+2).
  auto wait_step = [&]() {
    if (!NO_MEAN && w == 0) wait_dma_barrier<(D - 2) * (NSET + 1)>();
    else wait_dma_barrier<(D - 2) * NSET>();
  };

  // K tiles 0..D-1, R tiles and mean rows 0..D-2; clear the mean ring first (rows past the
  // last tile multiply rho = 0 and must be finite)
  if (!NO_MEAN)
    for (int i = t; i < MRING * 128 / 2; i += NWAVE * 64) ((uint32_t*)&mring[0][0])[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < D; ++i) stage(Kh + (size_t)clampT(i) * TILE_BYTES, kt0 + i * 2 * TILE_BYTES);
#pragma unroll
  for (int i = 0; i < D - 1; ++i) {
    stage(Rh + (size_t)clampT(i) * TILE_BYTES, rt0 + i * 2 * TILE_BYTES);
    mean_row(clampT(i));
  }

  // ---- prologue: Q L (rotated by H when HAD), its block scale sQ = 2^E (amax over the
  // 128 x 128 block), E4M3 ----
  const uint16_t* qrow = Q + (headN + qi) * VC_D;
  float qs[64];
  q_row_scaled<HAD>(qrow, hl, L, qs);
  float amax = wave_max(q_row_absmax(qs));
  if (lane == 0) red[w] = amax;
  __syncthreads();   // red[] and the cleared ring
  const int r0 = 4 * grp;
  amax = fmaxf(fmaxf(red[r0], red[r0 + 1]), fmaxf(red[r0 + 2], red[r0 + 3]));
  const int EQ = pow2_block_exponent(amax);
  const int sb = 127 + EQ;                         // E8M0 of sQ
  v8i qf[2];
  q_row_codes(qs, __builtin_ldexpf(1.0f, -EQ), qf);
  wait_dma_barrier<0>();   // the first copies have landed

  const v8i ones = rowsum_ones(lane);
  // byte offsets of this lane's 16-byte chunks 2hl, 2hl+1, 4+2hl, 5+2hl in row q of a tile (row
  // 32 i + q adds 4096 i, an instruction offset), so a fragment address is one add
  const uint32_t co0 = swz(q, 2 * hl), co1 = swz(q, 2 * hl + 1), co2 = swz(q, 4 + 2 * hl), co3 = swz(q, 5 + 2 * hl);
  auto frag = [&](const uint8_t* t, uint32_t oa, uint32_t ob, int blk) {
    const uint4 lo = *(const uint4*)(t + oa + 4096 * blk);
    const uint4 hi = *(const uint4*)(t + ob + 4096 * blk);
    v8i r;
    r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
    r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
    return r;
  };
  float b = 0.0f, l_run = 0.0f;   // b = 119.65 - m; set on the first tile
  // b in every element: the QK accumulator input, kept in registers and rebuilt only when b
  // changes (a running-maximum update), not once per tile
  v16f bsplat = {};
  // E8M0 exponent of sK of the tile of this wave's next QK product.  It is loaded at the start
  // of the vector phase before and taken before that phase's LDS reads: a scalar load shares its
  // wait counter with the LDS reads, so waiting for it later (or inside the matrix phase) would
  // also wait for every fragment in flight.
  auto e8m0_sk = [&](int i) { return (int)((__float_as_uint(sKh[i]) >> 23) & 0xFFu); };
  int sa = e8m0_sk(0);
  // Row sums of the current 16-tile group (query q), kept as a shift register: each tile's r
  // enters rA[7] and pushes the older ones down.  After the group's 8th tile rA is saved to
  // LDS (rsnap, one dword per slot and query, so the stores need no register quad; with the b
  // of that moment) and restarts; the saved half is rescaled once, at
  // the group end, by 2^((b_end - b_snap)/8), the product of the maximum updates since.  At
  // the group end the saved half holds tiles t0 .. t0+7 and rA[k] tile e-7+k (zero for tiles
  // before t0+8): the bf16 instruction's K-slots of the lane halves 0 and 1.
  float rA[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rA[k] = 0.0f;
  bool snapped = false;   // a first half of the current group is in rsnap
  float* my_snap = &rsnap[0][w * 32 + q];   // slot i at my_snap[i * NWAVE * 32]
  auto push_r = [&](float r, int e) {   // r of tile e
#pragma unroll
    for (int k = 0; k < 7; ++k) rA[k] = rA[k + 1];
    rA[7] = r;
    if ((e & 15) == 7) {
#pragma unroll
      for (int k = 0; k < 8; ++k) my_snap[k * NWAVE * 32] = rA[k];
#pragma unroll
      for (int k = 0; k < 8; ++k) rA[k] = 0.0f;
      my_snap[8 * NWAVE * 32] = b;
      snapped = true;
    }
  };
  v16f acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = v16f{};
  v16f s[4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) s[kb] = v16f{};
  v8i pw[2] = {};
  v8i rf[8];   // residual fragments of the next PV product, read at the end of the vector phase
#pragma unroll
  for (int i = 0; i < 8; ++i) rf[i] = v8i{};
  v4f rs = {};

  // Eq. 6's mean term of the 16-tile group that ends with tile e: A += mu~^T rho
  auto mean_group = [&](int e) {
    float rB[8];
    if (snapped) {
      const float f = __builtin_amdgcn_exp2f(0.125f * (b - my_snap[8 * NWAVE * 32]));
#pragma unroll
      for (int k = 0; k < 8; ++k) rB[k] = my_snap[k * NWAVE * 32] * f;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) rB[k] = 0.0f;
    }
    snapped = false;
    // rho = bf16 hi + bf16 lo, two values per hardware conversion (round to nearest even)
    typedef float v2f_ __attribute__((ext_vector_type(2)));
    typedef __bf16 v2bf_ __attribute__((ext_vector_type(2)));
    v8s bhi, blo;
#pragma unroll
    for (int k = 0; k < 8; k += 2) {
      const v2f_ x = {hl ? rA[k] : rB[k], hl ? rA[k + 1] : rB[k + 1]};
      const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, v2bf_));
      const v2f_ rest = {x[0] - __uint_as_float(hw << 16), x[1] - __uint_as_float(hw & 0xFFFF0000u)};
      const uint32_t lw = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, v2bf_));
      bhi[k] = (short)(hw & 0xFFFFu); bhi[k + 1] = (short)(hw >> 16);
      blo[k] = (short)(lw & 0xFFFFu); blo[k + 1] = (short)(lw >> 16);
      rA[k] = 0.0f; rA[k + 1] = 0.0f;
    }
    const int t0 = hl ? e - 7 : (e & ~15);   // tile of this lane's first K-slot
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      v8s am;
#pragma unroll
      for (int k = 0; k < 8; ++k) am[k] = (short)mring[(t0 + k) & (MRING - 1)][32 * db + q];
      acc[db] = mfma_bf16(am, bhi, acc[db]);
      acc[db] = mfma_bf16(am, blo, acc[db]);
    }
  };

  // M(j): A += P R and the row sum of tile j-1, then S^T of tile j (t = a s + b), then r of
  // tile j-1 into l and rho (vector work that fills the wave's idle issue slots while its
  // products run, taken off the vector phase).  All
  // fragments of the residual tile are requested first and two key fragments after each PV
  // instruction, so the matrix unit never waits for an LDS round trip inside the phase.
  auto mphase = [&](int j, auto qk, auto pv) {
    constexpr bool QK = decltype(qk)::value, PV = decltype(pv)::value;
    v8i kf[8];
    if constexpr (QK) {
      const uint8_t* kb_ = tiles[j % NBUF][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) kf[2 * kb] = frag(kb_, co0, co1, kb);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        kf[2 * kb + 1] = frag(kb_, co2, co3, kb);
      }
    }
    if constexpr (PV) {
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[db] = mfma_fp8(rf[4 * p + db], pw[p], acc[db], 127, 127);
      rs = mfma_fp8_16(ones, pw[0], v4f{});
      rs = mfma_fp8_16(ones, pw[1], rs);
    }
    if constexpr (QK) {
      // the first halves of the four chains, then the second halves: no product waits on the
      // one issued just before it (the key fragments are read in that order too)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb] = mfma_fp8(kf[2 * kb], qf[0], bsplat, sa, sb);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) s[kb] = mfma_fp8(kf[2 * kb + 1], qf[1], s[kb], sa, sb);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) keep(s[kb]);
    }
    if constexpr (PV) keep(rs);
    if constexpr (PV && QK) {
      // key fragments two at a time behind the products, so at most four are in registers:
      // PV 0-3 with K fragments 0-3, PV 4-7 and the row sums, QK 0-3 (chains 0, 1) with K
      // fragments 4-7, QK 4-7
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    // the group that ended at tile j-2 has all its row sums in rho since M(j-1)
    if constexpr (PV) {
      if (!NO_MEAN && j >= 2 && ((j - 2) & 15) == 15) mean_group(j - 2);
      const float r = rs[0];   // r of tile j-1 into l and rho
      l_run += r;
      if (!NO_MEAN) push_r(r, j - 1);
    }
  };
  constexpr std::true_type Y{};
  constexpr std::false_type X{};

  // V(j): running maximum of tile j, its ExpCast codes, the residual fragments of PV(j)
  auto vphase = [&](int j) {
    const int sa_next = e8m0_sk(j + 1 < T ? j + 1 : T - 1);   // for QK of tile j+1
    float tm;
    if constexpr (ETC) {
      tm = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) tm = fmaxf(tm, s[kb][i]);
    } else {
      float tmA, tmB;
      max16_2chains<true>(tmA, tmB, s[0]);
      max16_2chains<false>(tmA, tmB, s[1]);
      max16_2chains<false>(tmA, tmB, s[2]);
      max16_2chains<false>(tmA, tmB, s[3]);
      tm = fmaxf(tmA, tmB);
    }
    tm = pair_max(tm);
    const bool first = j == 0;
    constexpr float C0 = ETC ? 0.0f : EC_C;
    const float delta = first ? tm - C0 : fmaxf(tm - C0, 0.0f);
    if (first || __ballot(delta > 0.0f) != 0ull) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] -= delta;
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(-0.125f * delta);
        l_run *= alpha;
#pragma unroll
        for (int k = 0; k < 8; ++k) rA[k] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
      b -= delta;
      {   // eight 64-bit copies of the pair (b, b): 16 moves where a float splat takes 23
        typedef double v8d __attribute__((ext_vector_type(8)));
        double bb = __builtin_bit_cast(double, ((uint64_t)__float_as_uint(b) << 32) | __float_as_uint(b));
        asm("" : "+v"(bb));   // opaque, so the compiler does not turn it back into a float splat
        const v8d w = {bb, bb, bb, bb, bb, bb, bb, bb};
        bsplat = __builtin_bit_cast(v16f, w);
      }
      asm volatile("" : "+v"(bsplat));   // opaque: kept, not rebuilt from b where it is used
    }
    // ExpCast Round + clip: one saturating RNE byte conversion per element.  Byte jj of the
    // PV B-operand for key half p is element (kb = 2p + jj/16, i = jj%16) of S^T.
    // key half 0's codes free the scores of key blocks 0-1, whose registers then receive the
    // residual fragments of PV half 0 (the reads are requested in key-half order)
    sa = sa_next;   // its wait precedes the fragment reads
    keep(sa);
    const uint8_t* rb = tiles[j % NBUF][1];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int kb = 2 * p + (wd >> 2), i0 = 4 * (wd & 3);
        uint32_t word = 0;
        if constexpr (ETC) {
          float e[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) e[x] = __builtin_amdgcn_exp2f(fmaf(s[kb][i0 + x], 0.125f, 8.0f));
          int w2 = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
          w2 = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w2, true);
          word = (uint32_t)w2;
        } else {
          word = expcast_byte(s[kb][i0 + 0], 0, word);
          word = expcast_byte(s[kb][i0 + 1], 1, word);
          word = expcast_byte(s[kb][i0 + 2], 2, word);
          word = expcast_byte(s[kb][i0 + 3], 3, word);
        }
        pw[p][wd] = (int)word;
      }
      keep(pw[p]);
      // the residual fragments of PV(j) half p, the first products of M(j+1)
#pragma unroll
      for (int db = 0; db < 4; ++db) rf[4 * p + db] = frag(rb, p ? co2 : co0, p ? co3 : co1, db);
    }
  };

  // Phases 2j and 2j+1.  Group 0 runs M(j) | V(j), group 1 V(j-1) | M(j); each wave issues
  // its copies of step j at the start of its vector phase (phase 2j+1 in group 0, 2j in group
  // 1), keeping them out of the matrix-instruction stream, and every wave waits at the end of
  // phase 2j+1 for step j-1 (K tile j+1, R tile j, first read in phase 2j+2).  Buffer reuse:
  // step j overwrites K tile j-1 and R tile j-2, whose last reads were in phase 2j-1.
  // A wave without queries only copies.
  // The ExpCast loops run four steps per iteration: the copy ring is four deep, so every
  // slot index inside the body is a constant.  The body is a macro because a lambda called
  // there is not inlined and would put the loop state on the stack.  The exp-then-cast
  // variant keeps the rolled loop, which allocates no scratch.
  if (!valid) {
    for (int j = 0; j < T; ++j) {
      issue(j);
      phase_barrier();
      wait_step();
    }
    phase_barrier();
    wait_dma_barrier<0>();
    return;
  }
  if (grp == 0) {
    mphase(0, Y, X);
    phase_barrier();
    issue(0);
    vphase(0);
    wait_step();
#define VC_STEP0(J) { mphase(J, Y, Y); phase_barrier(); issue(J); vphase(J); wait_step(); }
    int j = 1;
    if constexpr (!ETC)
      for (; j + 3 < T; j += 4) {
        VC_STEP0(j)
        VC_STEP0(j + 1)
        VC_STEP0(j + 2)
        VC_STEP0(j + 3)
      }
    for (; j < T; ++j) VC_STEP0(j)
#undef VC_STEP0
    mphase(T, X, Y);
    phase_barrier();
    wait_dma_barrier<0>();
  } else {
    issue(0);
    phase_barrier();
    mphase(0, Y, X);
    wait_step();
#define VC_STEP1(J) { issue(J); vphase(J - 1); phase_barrier(); mphase(J, Y, Y); wait_step(); }
    int j = 1;
    if constexpr (!ETC)
      for (; j + 3 < T; j += 4) {
        VC_STEP1(j)
        VC_STEP1(j + 1)
        VC_STEP1(j + 2)
        VC_STEP1(j + 3)
      }
    for (; j < T; ++j) VC_STEP1(j)
#undef VC_STEP1
    vphase(T - 1);
    phase_barrier();
    mphase(T, X, Y);
    wait_dma_barrier<0>();
  }

  // ---- epilogue: the last mean group, O = A * sV / l -> bf16 ----
  if (!NO_MEAN) mean_group(T - 1);
  const float inv_l = 1.0f / l_run;
  const float* sv = sV + (size_t)bh * VC_D;
  uint16_t* orow = O + (headN + qi) * VC_D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int d0 = 32 * db + 8 * ig + 4 * hl;
      const float4 s4 = *(const float4*)(sv + d0);
      const uint32_t o0 = f32_to_bf16_rne(acc[db][4 * ig + 0] * s4.x * inv_l);
      const uint32_t o1 = f32_to_bf16_rne(acc[db][4 * ig + 1] * s4.y * inv_l);
      const uint32_t o2 = f32_to_bf16_rne(acc[db][4 * ig + 2] * s4.z * inv_l);
      const uint32_t o3 = f32_to_bf16_rne(acc[db][4 * ig + 3] * s4.w * inv_l);
      *(uint2*)(orow + d0) = make_uint2(o0 | (o1 << 16), o2 | (o3 << 16));
    }
  if (w == 0) clock_stamp(clk ? clk + 4 * blockIdx.x + 2 : nullptr);
}

// The query prologue of k_attn_fwd on its own: one workgroup of four waves per 128-row block,
// each wave 32 rows in the kernel's lane layout, the same helpers; writes the E4M3 codes in
// natural layout Qq [BH][N][128] and the block scales sQ [BH][N/128] (2^EQ).
template <bool HAD>
__global__ __launch_bounds__(256) void k_test_qquant(const uint16_t* __restrict__ Q, int N, float L,
                                                     uint8_t* __restrict__ Qq, float* __restrict__ sQ) {
  __shared__ float red[4];
  const int t = threadIdx.x, lane = t & 63, q = lane & 31, hl = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const size_t row = (size_t)blockIdx.y * N + (size_t)blockIdx.x * 128 + 32 * w + q;
  float qs[64];
  q_row_scaled<HAD>(Q + row * VC_D, hl, L, qs);
  float amax = wave_max(q_row_absmax(qs));
  if (lane == 0) red[w] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const int EQ = pow2_block_exponent(amax);
  v8i qf[2];
  q_row_codes(qs, __builtin_ldexpf(1.0f, -EQ), qf);
  uint8_t* out = Qq + row * VC_D;
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int d4 = 0; d4 < 8; ++d4) *(int*)(out + 64 * c + 32 * hl + 4 * d4) = qf[c][d4];
  if (t == 0) sQ[(size_t)blockIdx.y * (N / 128) + blockIdx.x] = __builtin_ldexpf(1.0f, EQ);
}

uint32_t vc_attn_fwd_workgroups(int BH, int N) { return (uint32_t)BH * (uint32_t)((N / 128 + 1) / 2); }

hipError_t vc_launch_test_qquant(const uint16_t* Q, int BH, int N, float L, bool hadamard, uint8_t* Qq, float* sQ,
                                 hipStream_t s) {
  if (hadamard)
    hipLaunchKernelGGL(k_test_qquant<true>, dim3(N / 128, BH), dim3(256), 0, s, Q, N, L, Qq, sQ);
  else
    hipLaunchKernelGGL(k_test_qquant<false>, dim3(N / 128, BH), dim3(256), 0, s, Q, N, L, Qq, sQ);
  return hipGetLastError();
}

hipError_t vc_launch_attn_fwd(const uint16_t* Q, const uint8_t* Kq, const float* sK,
                              const uint8_t* Rq, const uint16_t* mu, const float* sV,
                              int BH, int N, float L, unsigned flags, uint16_t* O,
                              uint64_t* clk, hipStream_t s) {
  const int nqb = N / 128, nwb = (nqb + 1) / 2;
  const uint32_t G = vc_attn_fwd_workgroups(BH, N);
  auto launch = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(G), dim3(NWAVE * 64), 0, s, Q, Kq, sK, Rq, mu, sV, N, nqb, nwb, G, L, O, clk);
  };
  const bool no_mean = flags & VC_ATTN_NO_MEAN, etc = flags & VC_ATTN_EXP_THEN_CAST;
  if (flags & VC_ATTN_HADAMARD) {
    if (no_mean && etc) launch(k_attn_fwd<true, true, true>);
    else if (no_mean) launch(k_attn_fwd<true, false, true>);
    else if (etc) launch(k_attn_fwd<false, true, true>);
    else launch(k_attn_fwd<false, false, true>);
  } else {
    if (no_mean && etc) launch(k_attn_fwd<true, true, false>);
    else if (no_mean) launch(k_attn_fwd<true, false, false>);
    else if (etc) launch(k_attn_fwd<false, true, false>);
    else launch(k_attn_fwd<false, false, false>);
  }
  return hipGetLastError();
}
