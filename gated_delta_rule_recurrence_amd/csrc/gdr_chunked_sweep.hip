// Chunked sweeps of the gated delta rule on gfx950 (matrix cores): the
// forward state recurrence and the reverse recurrence of its state gradient.
//
// Notation: a chunk has n <= 64 steps, local t = 0..n-1, and Gam(a,b] is the
// product of g over the steps a+1..b.  It is always formed as a running
// product and never by division.  Unrolling the recurrence of mlx issue #4614
// (the recurrence statement under the accuracy table) over one chunk gives:
//
// Forward, with S0 the state before the chunk:
//   e_t   = v_t - Gam(-1,t] S0 k_t - sum_{r<t} Gam(r,t] (k_t . k_r) beta_r e_r
//   y_t   = Gam(-1,t] S0 q_t + sum_{r<=t} Gam(r,t] (q_t . k_r) beta_r e_r
//   S_end = Gam(-1,n-1] S0 + sum_r beta_r Gam(r,n-1] e_r k_r^T
// For the rows of one value head, with E = [e_t] and U = V - diag(gam) K S0^T:
//   (I + A) E = U,            A[t][r] = Gam(r,t] (k_t . k_r) beta_r  (r < t)
//   Y = diag(gam) Q S0^T + M E,  M[t][r] = Gam(r,t] (q_t . k_r) beta_r (r <= t)
//   S_end = gend S0 + E^T diag(ks) K,  gam_t = Gam(-1,t], ks_r = beta_r Gam(r,n-1].
//
// Reverse, with H the gradient of the loss with respect to the state after
// step t.  The per-step form is
//   G_t = H_t + dy_t q_t^T,  c_t = G_t k_t,  H_{t-1} = g_t (G_t - beta_t c_t k_t^T).
// With Hend the gradient after the chunk:
//   c_t = Gam(t,n-1] Hend k_t + sum_{s>=t} Gam(t,s] (q_s . k_t) dy_s
//         - sum_{s>t} Gam(t,s] beta_s (k_s . k_t) c_s
//   H_start = Gam(-1,n-1] Hend + sum_s Gam(-1,s] (dy_s q_s^T - beta_s c_s k_s^T)
// For C = [c_t]:
//   (I + Bm) C = diag(suf) K Hend^T + Mq DY,
//     Bm[t][s] = Gam(t,s] beta_s (k_s . k_t)  (s > t),
//     Mq[t][s] = Gam(t,s] (q_s . k_t)  (s >= t),
//     suf_t = Gam(t,n-1],
//   H_start = pre_{n-1} Hend + DY^T diag(pre) Q - C^T diag(beta pre) K,  pre_s = Gam(-1,s].
//
// A prep kernel forms, once per (batch row, value head, chunk), the two
// Gram matrices and Gam, and from them:
//   * forward: T = (I + A)^-1 (column-wise forward substitution) and M;
//   * reverse: Tb = (I + Bm)^-1 (column-wise back substitution) and Mq.
// Each substitution forms the same sums as the sequential recurrence.  The
// sweep kernels then run a value head's chunks in order (reverse order for
// the gradient), 32 state rows per workgroup.  Rows are independent.  With
// fp32 inputs every product runs on fp32 MFMA (Dk <= 192); with bf16 inputs
// (the *_bf16_kernel sweeps, Dk <= 256) on bf16 MFMA over exact three-piece
// splits of the fp32 operands.  A replay mode of the forward (FwdSweepArgs::seg) rebuilds
// the tile states and residuals for the backward from states saved every
// few tiles.
//
// Outputs match the sequential sweeps:
//   * forward: y, S_T, the state checkpoint at every chunk start, and the
//     residuals e_t;
//   * reverse: dv, c_t, the gradient at every chunk end, and dS0.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kSwThreads = 512;  // sweep workgroup: eight waves, two per SIMD
constexpr int kN = 64;
constexpr int kNP = kN + 1;   // row stride of the Gram matrices in the prep
constexpr int kGP = kN + 4;   // row stride of the per-head matrix (16-byte rows)
constexpr int kDS = 32;       // state rows per sweep workgroup
constexpr int kUBS = 36;      // row stride of the [kN][kDS] step-by-row stages
constexpr int kMaxJT = 12;    // Dk <= 192: the fp32-operand sweeps (their LDS); the
                              // prep's bf16 Gram stage takes Dk in passes of this width
constexpr int kMaxJTB = 16;   // Dk <= 256: the bf16-product sweeps

// The products over the steps of a chunk (E = T U, Y = M E, C = Tb U,
// U += Mq DY and the state updates) use step rstep(ks, lq) as the k index
// of MFMA k-step ks in lane quarter lq.  That step is
// 16 (ks / 4) + 4 lq + ks % 4, which keeps the LDS reads of those products
// free of bank conflicts.
__device__ __forceinline__ int rstep(int ks, int lq) {
  return 16 * (ks >> 2) + 4 * lq + (ks & 3);
}

// The bf16-product sweeps (and the bf16-piece prep records they read) take
// bf16 inputs whose k, q rows come in 8-element groups and whose value rows
// come in 4-element blocks.
__host__ __device__ constexpr bool bf16_products(bool bf16_vec, int Dk, int Dv) {
  return bf16_vec && Dk % 8 == 0 && Dv % 4 == 0;
}

// Prep record layouts (floats; the stride is kChunkPrepStride).
// Forward record:
constexpr int kPrT = 0, kPrM = 4096, kPrGam = 8192, kPrKs = 8256, kPrGend = 8320;
// Reverse record:
constexpr int kPbT = 0, kPbM = 4096, kPbSuf = 8192, kPbPre = 8256, kPbBeta = 8320;
// With bf16 inputs (the bf16-product sweeps), the two matrices as three
// bf16 pieces each in 16x16x32 A-fragment order (pieces_to_record):
constexpr int kBrT = 0, kBrM = 6144, kBrGam = 12288, kBrKs = 12352, kBrGend = 12416;
constexpr int kBbT = 0, kBbM = 6144, kBbSuf = 12288, kBbPre = 12352, kBbBeta = 12416;
// All: 64 floats that nothing reads, the target of the sweeps' stores for
// lanes outside the tensors, so that no store needs a branch around it (a
// branch makes the compiler's wait counts for later loads conservative).
constexpr int kPrSink = 12480;
static_assert(kPbBeta + kN <= kPrSink && kBbBeta + kN <= kPrSink &&
                  kPrSink + 64 <= kChunkPrepStride, "record");

// A [64][64] triangular matrix, given elementwise, to a record as three bf16
// pieces in 16x16x32 A-fragment order: block (tb, ks, piece) holds for lane l
// the 16 bytes of row 16 tb + l % 16, columns 32 ks + 8 (l / 16) .. +7; block
// b = 2 tb + ks starts at float (3 b * 64 + l) * 4.  The two blocks past the
// diagonal (lower triangle: tb < 2, ks = 1; UPPER: tb >= 2, ks = 0) are zero;
// they are not written, and the readers skip them (pieces_from_record).  The
// other six are numbered 0..5 in record order; this writes blocks I0..I1-1.
template <bool UPPER, int I0 = 0, int I1 = 6, typename Elem>
__device__ __forceinline__ void pieces_to_record(float* __restrict__ dst, int l, Elem elem) {
  const int lr = l & 15, lq = l >> 4;
#pragma unroll 2
  for (int i = I0; i < I1; ++i) {
    const int b = UPPER ? (i < 4 ? i : 2 * i - 3) : (i < 2 ? 2 * i : i + 2);
    const int t = 16 * (b >> 1) + lr, s0 = 32 * (b & 1) + 8 * lq;
    f4 x, y;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = elem(t, s0 + e), y[e] = elem(t, s0 + 4 + e);
    uint2 x0, x1, x2, y0, y1, y2;
    split3_quad(x, x0, x1, x2);
    split3_quad(y, y0, y1, y2);
    *reinterpret_cast<uint4*>(dst + ((3 * b + 0) * 64 + l) * 4) = uint4{x0.x, x0.y, y0.x, y0.y};
    *reinterpret_cast<uint4*>(dst + ((3 * b + 1) * 64 + l) * 4) = uint4{x1.x, x1.y, y1.x, y1.y};
    *reinterpret_cast<uint4*>(dst + ((3 * b + 2) * 64 + l) * 4) = uint4{x2.x, x2.y, y2.x, y2.y};
  }
}

// The pieces of k-steps 0, 1 of step tile tb (lane l), as written above,
// except k-step `zero` (wave-uniform; -1: none), a block of zeros that the
// products skip (the triangular matrices' blocks past the diagonal)
__device__ __forceinline__ void pieces_from_record(const float* __restrict__ src, int tb, int l,
                                                   int zero, uint4 (&f)[2][3]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks == zero) continue;
#pragma unroll
    for (int p = 0; p < 3; ++p)
      f[ks][p] = *reinterpret_cast<const uint4*>(src + ((3 * (2 * tb + ks) + p) * 64 + l) * 4);
  }
}

// acc += A B over the 64 steps with both operands as three bf16 pieces: the
// six piece products down to the order of fp32 rounding.  a: A pieces per
// k-step (registers); b(ks, p): B piece p of k-step ks; k-step `zero` of A
// is zero and skipped.
template <typename BFn>
__device__ __forceinline__ f4 mfma_pieces6(const uint4 (&a)[2][3], BFn b, int zero, f4 acc) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks == zero) continue;
    const uint4 b0 = b(ks, 0), b1 = b(ks, 1), b2 = b(ks, 2);
    acc = mfma_bf16(a[ks][0], b0, acc);
    acc = mfma_bf16(a[ks][0], b1, acc);
    acc = mfma_bf16(a[ks][1], b0, acc);
    acc = mfma_bf16(a[ks][0], b2, acc);
    acc = mfma_bf16(a[ks][2], b0, acc);
    acc = mfma_bf16(a[ks][1], b1, acc);
  }
  return acc;
}

// A [64][64] record matrix in MFMA A-fragment order: the A operand of k-step
// ks (k index rstep(ks, lq)) of the 16 x 16 tile of rows 16 tb.. sits in
// lane (t % 16) + 16 lq; each group of four k-steps is one 16-byte block per
// lane, the 64 lanes' blocks consecutive, so a lane loads its 16 operands
// with four fully coalesced 16-byte loads.  Block (tb, x) starts at float
// ((tb * 4 + x) * 64 + lane) * 4.
__device__ __forceinline__ void load_frags(const float* __restrict__ m, int tb, int l,
                                           float (&f)[16]) {
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const f4 v = *reinterpret_cast<const f4*>(m + ((tb * 4 + x) * 64 + l) * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) f[4 * x + e] = v[e];
  }
}

// Writes a matrix held in LDS (element (t, r) at src[t * ld + r]) to a record
// in the order above; lane l writes block (tb, x) = bx of itself, for bx in
// [bx0, bx1).
__device__ __forceinline__ void store_frags(const float* src, int ld, float* __restrict__ m,
                                            int l, int bx0 = 0, int bx1 = 16) {
  const int lr = l & 15, lq = l >> 4;
#pragma unroll 4
  for (int bx = bx0; bx < bx1; ++bx) {
    const int tb = bx >> 2, x = bx & 3, t = 16 * tb + lr;
    f4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = src[t * ld + rstep(4 * x + e, lq)];
    *reinterpret_cast<f4*>(m + (bx * 64 + l) * 4) = v;
  }
}

// T = (I + A)^-1 for a unit lower (UPPER: upper) triangular I + A of size
// 64 whose strict triangle is held in the [64][kGP] LDS matrix G, by one
// wave, in 16 x 16 blocks:
//   the diagonal blocks T_ii = (I + A_ii)^-1 by substitution, the four blocks
//   at once (lane l: block l / 16, column l % 16);
//   L_ik = -T_ii A_ik for the off-diagonal blocks of the triangle (MFMA);
//   T_ij = sum_k L_ik T_kj, k from j to i - 1 (UPPER: i + 1 to j), block
//   row by block row (MFMA), from the block-row equations of (I + A) T = I.
// T replaces A in G (all of it: the other triangle is zeroed).  Stage
// STG 0 does all of it; with several waves on the matrix, stage 1 forms the
// diagonal blocks, stage 2 (every wave, its share nw of the six products,
// from wave iw) the L blocks, and stage 3 the rest, a barrier between the
// stages: each block takes the same operations either way.
template <bool UPPER, int STG = 0>
__device__ __forceinline__ void invert_unit_triangular(float* G, int l, int iw = 0, int nw = 1) {
  const int lr = l & 15, lq = l >> 4;
  if (STG == 0 || STG == 1) {
    const int base = 16 * lq, c = lr;
    float x[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = UPPER ? 15 - u : u;
      float acc[4] = {t == c ? 1.f : 0.f, 0.f, 0.f, 0.f};
      const float* row = G + (base + t) * kGP + base;
#pragma unroll
      for (int r4 = 0; r4 < 16; r4 += 4) {
        if (UPPER ? r4 + 3 <= t : r4 >= t) continue;
        const f4 a4 = *reinterpret_cast<const f4*>(row + r4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (UPPER ? r4 + e > t : r4 + e < t) acc[e] = fmaf(-a4[e], x[r4 + e], acc[e]);
      }
      x[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) G[(base + t) * kGP + base + c] = x[t];
  }
  // 16 x 16 block product on fp32 MFMA: A operand block (ra, ca), B operand
  // block (rb, cb) of G
  auto prod = [&](int ra, int ca, int rb, int cb, f4 acc) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      acc = mfma(G[(16 * ra + lr) * kGP + 16 * ca + 4 * ks + lq],
                 G[(16 * rb + 4 * ks + lq) * kGP + 16 * cb + lr], acc);
    return acc;
  };
  auto put = [&](int rb, int cb, f4 v) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) G[(16 * rb + 4 * lq + e) * kGP + 16 * cb + lr] = v[e];
  };
  if (STG == 1) return;
  // L_ik = -T_ii A_ik in place of A_ik (product x of the six: this wave's
  // when x % nw == iw)
  if (STG == 0 || STG == 2) {
    int x = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (UPPER ? k <= i : k >= i) continue;
        if (x++ % nw == iw) put(i, k, -prod(i, i, i, k, f4{0.f, 0.f, 0.f, 0.f}));
      }
  }
  if (STG == 2) return;
  // T_ij, a block row at a time (its products read L of the same row, so
  // the row is written once all of it is formed)
#pragma unroll
  for (int u = 1; u < 4; ++u) {
    const int i = UPPER ? 3 - u : u;
    f4 acc[3];
#pragma unroll
    for (int d = 0; d < u; ++d) {
      const int j = UPPER ? i + 1 + d : d;
      acc[d] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (UPPER ? (k <= i || k > j) : (k < j || k >= i)) continue;
        acc[d] = prod(i, k, k, j, acc[d]);
      }
    }
#pragma unroll
    for (int d = 0; d < u; ++d) put(i, UPPER ? i + 1 + d : d, acc[d]);
  }
  // the other triangle's off-diagonal blocks
#pragma unroll
  for (int x = 0; x < 6; ++x) {
    const int blk = x * 64 + l;  // (block pair, row, 4-column group)
    const int pr = blk >> 6, row = (blk >> 2) & 15, cg = blk & 3;
    // block pairs (0,1) (0,2) (0,3) (1,2) (1,3) (2,3) of the upper triangle
    const int bi = pr < 3 ? 0 : (pr < 5 ? 1 : 2);
    const int bj = pr < 3 ? pr + 1 : (pr < 5 ? pr - 1 : 3);
    const int r = UPPER ? bj : bi, cb = UPPER ? bi : bj;
    *reinterpret_cast<f4*>(G + (16 * r + row) * kGP + 16 * cb + 4 * cg) = f4{0.f, 0.f, 0.f, 0.f};
  }
}

// ---------------------------------------------------------------- prep ----
// grid (nch, Hk, B), eight waves (two per SIMD).  MODE kPrepFwd / kPrepBwd:
// the forward (reverse) records of the kv head's value heads (or of a pair
// of them: a.pair_grid), two at a time, each formed by four waves (waves
// 4 s .. 4 s + 3 for head slot s): they build Gam as running products down
// the rows, a quarter of the rows each, split the M (Mq) record and the rows
// of A (Bm), the first forms the diagonal blocks of the inverse, all four its
// L blocks, the first its block rows, and they split the T (Tb) record (seven
// barriers per round).  The workgroup holds two per-head matrices, 51 KB of
// LDS, and three workgroups share a CU.  kPrepBoth: waves 0-3 the forward and waves 4-7 the reverse records of
// the same heads, each wave every step of its head alone (the Gram matrices
// formed once for both); the backward's replay uses it.  Every record element
// takes the same operations in every mode, so the records are bitwise the
// same whichever launch forms them.
constexpr int kPrepFwd = 0, kPrepBwd = 1, kPrepBoth = 2;
constexpr int kPrepThreads = 512;

// QK (q_t . k_r) and KK (k_t . k_r) in one [kN][kNP] matrix: QK on and below
// the diagonal, KK above it.  The records use QK[t][r] only for r <= t, and
// KK (symmetric) only off the diagonal, read as KK[min][max].
__device__ __forceinline__ int qk_at(int t, int r) { return t * kNP + r; }  // r <= t

// LDS of the prep: NG per-head matrices [kN][kGP] and their beta vectors,
// then the QK / KK matrix; the q, k stages alias all of it (the QK / KK
// matrix is written once the stages are no longer read).
template <int NG>
struct PL {
  static constexpr int QS = 0, KS = 64 * kN;          // q, k stage [16][kN][4]
  static constexpr int GW = 0;                         // NG x [kN][kGP] (alias)
  static constexpr int VB = NG * kN * kGP;             // NG x beta[kN]
  static constexpr int QK = VB + NG * kN;              // QK / KK [kN][kNP]
  static constexpr int SIZE = QK + kN * kNP;
  static_assert(2 * 64 * kN <= QK + kN * kNP, "stage fits the workgroup's LDS");
  // bf16 inputs: q, k rows as bf16 [kN][KGS] (alias the per-head arrays);
  // the row stride an odd number of 16-byte units, so the 16-byte operand
  // reads of 16 rows at one column group hit distinct banks
  static constexpr int KGS = 16 * kMaxJT + 8;
  static constexpr int BQ = 0, BK = kN * KGS / 2;
  static_assert((2 * KGS) % 32 == 16 && 2 * kN * KGS / 2 <= QK + kN * kNP, "bf16 stage");
  static_assert(SIZE * 4 <= 160 * 1024, "LDS");
};

template <typename TIn, int MODE, bool VEC>
__global__ __launch_bounds__(kPrepThreads, 1) void prep_kernel(
    ChunkedSweepShape a, float* __restrict__ prep_f, float* __restrict__ prep_b) {
  constexpr bool SPLIT = MODE != kPrepBoth;  // four waves per value head
  constexpr int NTH = kPrepThreads;
  using L = PL<SPLIT ? 2 : 8>;
  extern __shared__ __align__(16) float sm[];
  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ g = static_cast<const TIn*>(a.g);
  const TIn* __restrict__ beta = static_cast<const TIn*>(a.beta);
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk;
  const int rep = Hv / Hk;
  // SPLIT with a.pair_grid: grid y runs over (kv head, pair of its value
  // heads), one round per workgroup; else over the kv heads
  const int npair = (rep + 1) / 2;
  const bool pg = SPLIT && a.pair_grid;
  const int jc = blockIdx.x, b = blockIdx.z;
  const int hk = pg ? (int)blockIdx.y / npair : (int)blockIdx.y;
  const int hbase = pg ? 2 * ((int)blockIdx.y - hk * npair) : 0;  // first value head
  const int hend = pg ? min(rep, hbase + 2) : rep;
  const int t0 = jc * a.L;
  const int n = min(a.L, T - t0);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 15, lq = l >> 4;
  const int tw = 16 * (w & 3);
  const int half = w >> 2;  // this wave's Gram column tiles: 2 half, 2 half + 1
  // this wave's first value head, which records it forms, and (SPLIT) its
  // part of them: quarter q of the head's four waves (one wave does all of
  // it in kPrepBoth); r0: the wave that forms the inverse and the vectors
  const int wh = SPLIT ? w >> 2 : w & 3;
  const int qw = SPLIT ? w & 3 : 0;
  constexpr int HSTEP = SPLIT ? 2 : 4;  // value heads per round
  const bool bwd = MODE == kPrepBwd || (MODE == kPrepBoth && w >= 4);
  const bool r0 = qw == 0;

  // g, beta of this wave's first value head, issued before the k, q loads
  // (index clamped into the tensors; masked where used)
  auto gb_index = [&](int hh) {
    return ((int64_t)b * T + t0 + (l < n ? l : 0)) * Hv + hk * rep + hh;
  };
  const int hw0 = hbase + wh < rep ? hbase + wh : 0;
  TIn g_raw = g[gb_index(hw0)], b_raw = beta[gb_index(hw0)];

  // ---- QK[t][r] = q_t . k_r, KK[t][r] = k_t . k_r (MFMA over Dk) ----------
  // wave w: rows 16 (w % 4) .., column tiles 2 half, 2 half + 1 of both
  constexpr bool kBf16 = std::is_same<TIn, bf16>::value && VEC;
  f4 acc[4];  // QK tiles, then KK tiles
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f4{0.f, 0.f, 0.f, 0.f};
  if (kBf16 && Dk % 8 == 0) {
    // bf16 k, q: the rows staged as bf16 and multiplied on bf16 MFMA (the
    // products of two bf16 values are exact in fp32, as in the fp32 path).
    // The stage holds 192 columns: a wider Dk takes a second pass, the
    // accumulators carried over (the same k-steps in the same order).
    constexpr int PW = 16 * kMaxJT;                  // columns per pass
    constexpr int NCH = PW / 8;                      // 16-byte chunks per row
    constexpr int NL = (kN * NCH + NTH - 1) / NTH;
    uint16_t* const sq = reinterpret_cast<uint16_t*>(sm + L::BQ);
    uint16_t* const sk = reinterpret_cast<uint16_t*>(sm + L::BK);
    for (int j0 = 0; j0 < Dk; j0 += PW) {
      uint4 rq[NL], rk[NL];
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int ci = tid + NTH * u;
        const int s = ci / NCH, j = j0 + 8 * (ci % NCH);
        const bool ok = ci < kN * NCH && s < n && j < Dk;
        int64_t o = ok ? ((int64_t)(b * (int64_t)T + t0 + s) * Hk + hk) * Dk + j : 0;
        asm volatile("" : "+v"(o));  // keeps the select (no branch around the loads)
        rq[u] = *reinterpret_cast<const uint4*>(q + o);
        rk[u] = *reinterpret_cast<const uint4*>(k + o);
      }
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int ci = tid + NTH * u;
        const int s = ci / NCH, jl = 8 * (ci % NCH);
        const bool ok = ci < kN * NCH && s < n && j0 + jl < Dk;
        if (ci < kN * NCH) {
          uint4 xq = rq[u], xk = rk[u];
          xq.x = ok ? xq.x : 0u;  // component selects (a vector select goes through memory)
          xq.y = ok ? xq.y : 0u;
          xq.z = ok ? xq.z : 0u;
          xq.w = ok ? xq.w : 0u;
          xk.x = ok ? xk.x : 0u;
          xk.y = ok ? xk.y : 0u;
          xk.z = ok ? xk.z : 0u;
          xk.w = ok ? xk.w : 0u;
          *reinterpret_cast<uint4*>(sq + s * L::KGS + jl) = xq;
          *reinterpret_cast<uint4*>(sk + s * L::KGS + jl) = xk;
        }
      }
      __syncthreads();
      for (int ks = 0; ks < PW / 32 && j0 + 32 * ks < Dk; ++ks) {
        const int o = (tw + lr) * L::KGS + 32 * ks + 8 * lq;
        const uint4 aq = *reinterpret_cast<const uint4*>(sq + o);
        const uint4 ak = *reinterpret_cast<const uint4*>(sk + o);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int tb = 2 * half + x;
          const uint4 bk =
              *reinterpret_cast<const uint4*>(sk + (16 * tb + lr) * L::KGS + 32 * ks + 8 * lq);
          acc[x] = mfma_bf16(aq, bk, acc[x]);
          acc[2 + x] = mfma_bf16(ak, bk, acc[2 + x]);
        }
      }
      __syncthreads();  // the stage aliases the per-head arrays (and the next pass's)
    }
  } else {
    constexpr int NB = kMaxJT / 4, NU = 4 * 256 / NTH;
    Quad<TIn, VEC> rq[NB][NU], rk[NB][NU];
    uint64_t msk = 0;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int qi = tid + NTH * u;
        const int s = qi >> 4, j = 64 * jb + 4 * (qi & 15);
        const bool ok = s < n && j < Dk;
        const int64_t o = ok ? ((int64_t)(b * (int64_t)T + t0 + s) * Hk + hk) * Dk + j : 0;
        rq[jb][u].load(q, o, ok, Dk - j);
        rk[jb][u].load(k, o, ok, Dk - j);
        msk |= (uint64_t)Quad<TIn, VEC>::mask(ok, Dk - j) << (4 * (NU * jb + u));
      }
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      if (64 * jb >= Dk) break;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int qi = tid + NTH * u;
        const int s = qi >> 4, jq = qi & 15;
        const uint32_t mu = (uint32_t)(msk >> (4 * (NU * jb + u))) & 15u;
        *reinterpret_cast<f4*>(sm + L::QS + (jq * kN + s) * 4) = rq[jb][u].get(mu);
        *reinterpret_cast<f4*>(sm + L::KS + (jq * kN + s) * 4) = rk[jb][u].get(mu);
      }
      __syncthreads();
#pragma unroll 2
      for (int ks = 0; ks < 16; ++ks) {
        const int fw = ((ks * kN + tw + lr) << 2) + lq;
        const float aq = sm[L::QS + fw], ak = sm[L::KS + fw];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int tb = 2 * half + x;
          const float bk = sm[L::KS + ((ks * kN + 16 * tb + lr) << 2) + lq];
          acc[x] = mfma(aq, bk, acc[x]);
          acc[2 + x] = mfma(ak, bk, acc[2 + x]);
        }
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = tw + 4 * lq + v, j = 16 * (2 * half + x) + lr;
      sm[L::QK + i * kNP + j] = j <= i ? acc[x][v] : acc[2 + x][v];
    }
  __syncthreads();

  // ---- per value head ------------------------------------------------------
  // (SPLIT: the four waves of a head share its matrix G, and every wave runs
  // the same number of rounds, so that the barriers below match up)
  float* G = sm + L::GW + (SPLIT ? wh : w) * kN * kGP;  // [kN][kGP] per head
  float* vb = sm + L::VB + (SPLIT ? wh : w) * kN;        // beta_t
  const float* QK = sm + L::QK;  // QK on and below the diagonal, KK above
  // bf16 inputs in 8-element groups: the bf16-product sweeps read the
  // matrices as bf16 pieces
  const bool pieces = bf16_products(kBf16, Dk, a.Dv);
  // a record's six piece blocks: all of them (one wave per head), or this
  // wave's share of the four (blocks 0-1, 2-3, 4, 5)
  auto pieces_quarter = [&](float* dst, int ll, auto elem, auto upper)
                            __attribute__((always_inline)) {
    constexpr bool U = decltype(upper)::value;
    if (!SPLIT) pieces_to_record<U>(dst, ll, elem);
    else if (qw == 0) pieces_to_record<U, 0, 2>(dst, ll, elem);
    else if (qw == 1) pieces_to_record<U, 2, 4>(dst, ll, elem);
    else if (qw == 2) pieces_to_record<U, 4, 5>(dst, ll, elem);
    else pieces_to_record<U, 5, 6>(dst, ll, elem);
  };
  for (int h0 = hbase; h0 < hend; h0 += HSTEP) {
    // the lane indices again, from an opaque copy of the thread id: otherwise
    // the compiler evaluates the per-row lane masks of the loops below ahead
    // of the Gram phase and spills them (a lane read back per use)
    int lane = tid & 63;
    asm volatile("" : "+v"(lane));
    const int l = lane, lr = l & 15, lq = l >> 4;
    const int hh = h0 + wh;
    const bool act = hh < rep;
    const int h = hk * rep + (act ? hh : 0);
    float* __restrict__ rec =
        (bwd ? prep_b : prep_f) + (((int64_t)b * Hv + h) * a.nch + jc) * kChunkPrepStride;
    if (h0 > hbase) {
      g_raw = g[gb_index(act ? hh : 0)];
      b_raw = beta[gb_index(act ? hh : 0)];
    }
    // an identity step (mask byte 0) has g = 1, beta = 0
    const bool skip = l < n && skipped(a.mask, b, T, t0 + l);
    const float gl = l < n && !skip ? decay_of(to_f32(g_raw), a.log_g) : 1.f;
    const float bl = l < n && !skip ? to_f32(b_raw) : 0.f;
    // Gam(r,t] (lane l <-> t = l), held in G[r][t]: 1 on the diagonal, 0
    // below it (rows r > t), and above it running products down the rows,
    // Gam(r,t] = g_{r+1} Gam(r+1,t], in four quarters of 16 rows: rows
    // 63..48 from 1, each lower quarter from Gam(16 (z + 1), t] (a product
    // scan over the lanes) for its rows 16 z + 15 .. 16 z.  g_{r+1} is read
    // from lane r + 1, so the loops hold only LDS stores.  Every row takes the
    // same products in every mode (one quarter per wave of a head, or all
    // four by one wave).
    auto gam_rows = [&](int z) __attribute__((always_inline)) {
      float p = z == 3 ? 1.f : wave_prefix_product(l > 16 * (z + 1) ? gl : 1.f);
#pragma unroll 8
      for (int r = 16 * z + 15; r >= 16 * z; --r) {
        const float gr =
            r + 1 < kN ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), r + 1)) : 1.f;
        p = r < l ? p * gr : p;
        G[r * kGP + l] = r < l ? p : (r == l ? 1.f : 0.f);
      }
      return p;
    };
    float pre = 0.f;  // Gam(-1, l] = g_0 Gam(0, l]
    if (act) {
      if (!SPLIT) {
        (void)gam_rows(3);
        (void)gam_rows(2);
        (void)gam_rows(1);
      } else if (qw > 0) {
        (void)gam_rows(qw);
      }
      if (r0) {
        pre = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), 0)) * gam_rows(0);
        vb[l] = bl;
      }
    }
    if (SPLIT) __syncthreads();

    // the M (Mq) record, its blocks split between the four waves; suf is
    // read before Bm replaces Gam above the diagonal
    float suf = 0.f;  // Gam(l, n-1]
    if (act && r0) suf = l < n ? G[l * kGP + n - 1] : 0.f;
    if (act) {
      if (!bwd) {
        // M[t][s] = Gam(s,t] QK[t][s] beta_s, s <= t, in fragment order
        auto m_el = [&](int t, int s) __attribute__((always_inline)) {
          return s <= t ? G[s * kGP + t] * QK[qk_at(t, s)] * vb[s] : 0.f;
        };
        if (pieces) {
          pieces_quarter(rec + kBrM, l, m_el, std::false_type{});
        } else {
#pragma unroll 2
          for (int bx = SPLIT ? 4 * qw : 0; bx < (SPLIT ? 4 * qw + 4 : 16); ++bx) {
            const int t = 16 * (bx >> 2) + lr;
            f4 m4;
#pragma unroll
            for (int e = 0; e < 4; ++e) m4[e] = m_el(t, rstep(4 * (bx & 3) + e, lq));
            *reinterpret_cast<f4*>(rec + kPrM + (bx * 64 + l) * 4) = m4;
          }
        }
      } else {
        // Mq[t][s] = Gam(t,s] QK[s][t], s >= t, in fragment order
        auto m_el = [&](int t, int s) __attribute__((always_inline)) {
          return s >= t ? G[t * kGP + s] * QK[qk_at(s, t)] : 0.f;
        };
        if (pieces) {
          pieces_quarter(rec + kBbM, l, m_el, std::true_type{});
        } else {
#pragma unroll 2
          for (int bx = SPLIT ? 4 * qw : 0; bx < (SPLIT ? 4 * qw + 4 : 16); ++bx) {
            const int t = 16 * (bx >> 2) + lr;
            f4 m4;
#pragma unroll
            for (int e = 0; e < 4; ++e) m4[e] = m_el(t, rstep(4 * (bx & 3) + e, lq));
            *reinterpret_cast<f4*>(rec + kPbM + (bx * 64 + l) * 4) = m4;
          }
        }
      }
    }
    if (SPLIT) __syncthreads();

    // A (Bm) in place, its rows t split between the four waves of the head
    // (SPLIT: rows 16 q .. 16 q + 15 by quarter q), then its inverse by the
    // first wave
    auto build_a = [&](int ta, int tb) __attribute__((always_inline)) {
      if (!bwd) {
        // A[t][r] = Gam(r,t] KK[t][r] beta_r below the diagonal (lane l <-> r):
        // all of the lane's operands loaded first, then the stores
        float av[kN];
#pragma unroll
        for (int t = ta; t < tb; ++t)
          av[t] = t > 0 ? G[l * kGP + t] * QK[l * kNP + t] * bl : 0.f;  // KK[l][t], l < t
#pragma unroll
        for (int t = ta; t < tb; ++t)
          if (l < t) G[t * kGP + l] = av[t];
      } else {
        // Bm[t][s] = Gam(t,s] beta_s KK[s][t], s > t, in place of Gam above the
        // diagonal (lane l <-> s)
        float bv[kN];  // the lane's operands first, then the updates
#pragma unroll
        for (int t = ta; t < tb; ++t)
          bv[t] = t < kN - 1 ? bl * QK[t * kNP + l] * G[t * kGP + l] : 0.f;  // KK[t][l], t < l
#pragma unroll
        for (int t = ta; t < tb; ++t)
          if (l > t) G[t * kGP + l] = bv[t];
      }
    };
    if (act) {
      if (!SPLIT) build_a(0, kN);
      else if (qw == 0) build_a(0, 16);
      else if (qw == 1) build_a(16, 32);
      else if (qw == 2) build_a(32, 48);
      else build_a(48, kN);
    }
    if (SPLIT) __syncthreads();
    // T = (I + A)^-1 (Tb = (I + Bm)^-1) in place of A (Bm): the diagonal
    // blocks and the block rows by the first wave, the six L blocks (SPLIT)
    // over the head's four waves
    if (!SPLIT) {
      if (act) {
        if (!bwd) invert_unit_triangular<false>(G, l);
        else invert_unit_triangular<true>(G, l);
      }
    } else {
      if (act && r0) {
        if (!bwd) invert_unit_triangular<false, 1>(G, l);
        else invert_unit_triangular<true, 1>(G, l);
      }
      __syncthreads();
      if (act) {
        if (!bwd) invert_unit_triangular<false, 2>(G, l, qw, 4);
        else invert_unit_triangular<true, 2>(G, l, qw, 4);
      }
      __syncthreads();
      if (act && r0) {
        if (!bwd) invert_unit_triangular<false, 3>(G, l);
        else invert_unit_triangular<true, 3>(G, l);
      }
    }
    if (SPLIT) __syncthreads();

    // the T (Tb) record, its blocks split between the four waves, and the
    // step vectors by the first
    if (act) {
      auto t_el = [&](int t, int s) __attribute__((always_inline)) { return G[t * kGP + s]; };
      if (!bwd) {
        if (pieces) {
          pieces_quarter(rec + kBrT, l, t_el, std::false_type{});
        } else {
          store_frags(G, kGP, rec + kPrT, l, SPLIT ? 4 * qw : 0, SPLIT ? 4 * qw + 4 : 16);
        }
        if (r0) {
          rec[(pieces ? kBrGam : kPrGam) + l] = pre;
          rec[(pieces ? kBrKs : kPrKs) + l] = bl * suf;
          if (l == n - 1) rec[pieces ? kBrGend : kPrGend] = pre;
        }
      } else {
        if (pieces) {
          pieces_quarter(rec + kBbT, l, t_el, std::true_type{});
        } else {
          store_frags(G, kGP, rec + kPbT, l, SPLIT ? 4 * qw : 0, SPLIT ? 4 * qw + 4 : 16);
        }
        if (r0) {
          rec[(pieces ? kBbSuf : kPbSuf) + l] = suf;
          rec[(pieces ? kBbPre : kPbPre) + l] = pre;
          rec[(pieces ? kBbBeta : kPbBeta) + l] = bl;
        }
      }
    }
    // (the next head's Gam is written only after every wave has passed the
    // barrier that follows its own Gam rows, which comes after these reads)
    if (SPLIT) __syncthreads();
  }
}

// --------------------------------------------------------------- sweeps ---
// grid (ceil(Dv / 32), Hv, B): state rows i0 .. i0 + 31 of one value head,
// eight waves (two per SIMD).  In a chunk, wave w owns one 16 x 16 tile
// (steps 16 (w % 4) .., rows 16 (w / 4) ..) of the step-by-row products, and
// the state tiles (rows 16 (w % 2) .., Dk columns 16 (JW (w / 2) + nj) ..)
// of the state update.

// The sweeps' workgroup (row slice, value head, batch row) in an XCD-aware
// order.  Workgroups go to the 8 XCDs round-robin by linear id; numbering
// them so that consecutive ids share an XCD puts the row slices of a value
// head (one prep record) and the value heads of a kv head (one k, q) in one
// XCD's L2.  Any order is correct; this one only saves cache traffic.
struct SweepBlock {
  int x, h, b;
};

// Step tile tb (steps 16 tb ..) and row tile nt of wave w in the bf16-product
// sweeps: a SIMD's two waves (w, w + 4) take tiles 0 or 1 and 2 or 3, one
// with a zero k-step in the triangular products and one without, so that
// the SIMDs carry equal work.
__device__ __forceinline__ int sweep_tb(int w) { return w < 4 ? w >> 1 : 2 + ((w - 4) >> 1); }
__device__ __forceinline__ SweepBlock sweep_block() {
  const int nx = gridDim.x, ny = gridDim.y;
  const int total = nx * ny * gridDim.z;
  const int lin = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
  const int id = total % 8 == 0 ? (lin % 8) * (total / 8) + lin / 8 : lin;
  return SweepBlock{id % nx, (id / nx) % ny, id / (nx * ny)};
}

// The tiles a forward workgroup runs, from the batch index of its grid slot:
// every tile from S0 normally; with a.seg > 0 (a replay from the save
// buffer) segment s of batch row b, tiles s * seg .. from slot s.  s0 is the
// (batch row, value head, slot) index of the starting state in units of one
// [Dv][Dk] matrix, before the value head is added (see FwdSweepArgs).
struct TileRange {
  int b, c0, c1;
  int64_t s0;
};
__device__ __forceinline__ TileRange tile_range(const FwdSweepArgs& a, int z, int h) {
  TileRange r{z, 0, a.nch, 0};
  int s = 0;
  if (a.seg > 0) {
    const int nseg = (a.nch + a.seg - 1) / a.seg;
    r.b = z / nseg;
    s = z - r.b * nseg;
    r.c0 = s * a.seg;
    r.c1 = min(r.c0 + a.seg, a.nch);
  }
  r.s0 = ((int64_t)r.b * a.Hv + h) * a.s0_stride + s;
  return r;
}
// Save-buffer slot of the state before tile c, or -1 if it is not saved.
__device__ __forceinline__ int ckpt_slot(const FwdSweepArgs& a, int c) {
  return c % a.ck_every == 0 ? c / a.ck_every : -1;
}

// The k, q rows of a chunk: fetched into registers a chunk ahead (raw bits,
// masked where deposited), then deposited into the natural-layout LDS stages
// [kN][KLD] with zero padding columns.
template <typename TIn, int JT, bool VEC, int NTH = kSwThreads>
struct KQPrefetch {
  static constexpr int DKP = 16 * JT, KLD = DKP + 4;
  static constexpr int NQT = kN * DKP / 4;  // 4-column quads of one chunk
  static constexpr int NQ = NQT / NTH;
  static_assert(NQT % NTH == 0 && 4 * NQ <= 64, "quads per thread");
  uint64_t pm = 0;
  Quad<TIn, VEC> pk[NQ], pq[NQ];
  int tid;

  // quad u of this thread: step qt(u), columns qj(u) .. qj(u) + 3 (recomputed
  // where used rather than held in registers)
  __device__ __forceinline__ int qt(int u) const { return (tid + NTH * u) / (DKP / 4); }
  __device__ __forceinline__ int qj(int u) const { return 4 * ((tid + NTH * u) % (DKP / 4)); }
  __device__ __forceinline__ void init(int t) { tid = t; }
  // rows t0 .. t0 + n - 1; base = element (t0, kv head, 0); kst = row stride
  __device__ __forceinline__ void fetch(const TIn* __restrict__ k, const TIn* __restrict__ q,
                                        int64_t base, int n, int kst, int Dk) {
    uint64_t m = 0;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int t = qt(u), j = qj(u);
      const bool ok = j < Dk && t < n;
      const int o = ok ? t * kst + j : 0;
      pk[u].load(k + base, o, ok, Dk - j);
      pq[u].load(q + base, o, ok, Dk - j);
      m |= (uint64_t)Quad<TIn, VEC>::mask(ok, Dk - j) << (4 * u);
    }
    pm = m;
  }
  __device__ __forceinline__ void deposit(float* kl, float* ql) const {
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const uint32_t mu = (uint32_t)(pm >> (4 * u)) & 15u;
      const int o = qt(u) * KLD + qj(u);
      *reinterpret_cast<f4*>(kl + o) = pk[u].get(mu);
      *reinterpret_cast<f4*>(ql + o) = pq[u].get(mu);
    }
  }
};

template <int JT>
struct SL {
  static constexpr int DKP = 16 * JT;
  static constexpr int KLD = DKP + 4;
  static constexpr int KL = 0, QL = kN * KLD;   // k, q stages [kN][KLD]
  static constexpr int SK = 2 * kN * KLD;       // state k-interleaved [DKP/4][kDS][4]
  static constexpr int B0 = SK + kDS * DKP;     // three [kN][kUBS] stages
  static constexpr int B1 = B0 + kN * kUBS;
  static constexpr int B2 = B1 + kN * kUBS;
  static constexpr int SIZE = B2 + kN * kUBS;
  static_assert(SIZE * 4 <= 160 * 1024, "LDS");
};

// P[16 steps of tile tw][16 rows of slice 16 nt] = [K or Q rows] State^T:
// k-steps over Dk in groups of G, the LDS operands of a group read while
// the products of the previous group issue (two register slots; the
// scheduling barriers keep that order).  NACC accumulators per product
// alternate over the groups.
template <int DKP, int KLD, int G, int NM, int NACC>
__device__ __forceinline__ void state_products(const float* const (&ap)[NM], const float* sp,
                                               f4 (&acc)[NM][NACC]) {
  constexpr int NG = DKP / 4 / G;
  static_assert(NG % NACC == 0, "groups per accumulator");
  float av[2][NM][G], bs[2][G];
  auto rd = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < G; ++x) {
#pragma unroll
      for (int m = 0; m < NM; ++m) av[g & 1][m][x] = ap[m][4 * (G * g + x)];
      bs[g & 1][x] = sp[(G * g + x) * kDS * 4];
    }
  };
  rd(0);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g + 1 < NG) rd(g + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < G; ++x)
#pragma unroll
      for (int m = 0; m < NM; ++m)
        acc[m][g % NACC] = mfma(av[g & 1][m][x], bs[g & 1][x], acc[m][g % NACC]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Sacc[nj] += sum over the 64 steps of A[i][t] B[t][j] for the state tiles
// of a wave: A[i][t] = ab[t kUBS + i] (a [kN][kUBS] stage, i = 16 mt + lr),
// B[t][j] = bb[t KLD + j] (a [kN][KLD] stage, j = 16 (jg + nj) + lr).
// Steps rstep(ks, lq) in groups of four, read a group ahead.
template <int JW, int KLD>
__device__ __forceinline__ void update_products(const float* ab, const float* bb, int lq,
                                                f4 (&Sacc)[JW]) {
  const float* ep = ab + 4 * lq * kUBS;
  const float* kb = bb + 4 * lq * KLD;
  float ae[2][4], bk[2][4][JW];
  auto rd = [&](int g) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      ae[g & 1][x] = ep[(16 * g + x) * kUBS];
#pragma unroll
      for (int nj = 0; nj < JW; ++nj) bk[g & 1][x][nj] = kb[(16 * g + x) * KLD + 16 * nj];
    }
  };
  rd(0);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g + 1 < 4) rd(g + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int nj = 0; nj < JW; ++nj) Sacc[nj] = mfma(ae[g & 1][x], bk[g & 1][x][nj], Sacc[nj]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The state tiles of a wave (tile nj, register u <-> row 16 mt + 4 lq + u,
// column 16 (jg + nj) + lr) into the k-interleaved LDS copy [DKP/4][kDS][4]:
// element (i, j) at ((j / 4) kDS + i) 4 + j % 4.
template <int JW>
__device__ __forceinline__ void tiles_to_lds(float* sk, const f4 (&acc)[JW], int mt, int jg,
                                             int lq, int lr) {
  float* p = sk + ((4 * jg + (lr >> 2)) * kDS + 16 * mt + 4 * lq) * 4 + (lr & 3);
#pragma unroll
  for (int nj = 0; nj < JW; ++nj)
#pragma unroll
    for (int u = 0; u < 4; ++u) p[(4 * nj * kDS + u) * 4] = acc[nj][u];
}

// The slice in the LDS copy to rows i0 .. i0 + 31 of a [Dv][Dk] matrix in
// HBM, a 4-column group per thread and pass (one 16-byte store where Dk % 4
// == 0); rows vary fastest across the lanes, which keeps the LDS reads
// conflict-free.
template <int JT, bool VEC>
__device__ __forceinline__ void lds_to_matrix(const float* sk, float* __restrict__ dst, int i0,
                                              int Dv, int Dk, int tid) {
  constexpr int NQ4 = kDS * 4 * JT;  // 4-column groups of the slice
  static_assert(NQ4 % kSwThreads == 0, "passes");
#pragma unroll
  for (int x = 0; x < NQ4 / kSwThreads; ++x) {
    const int e = tid + kSwThreads * x;
    const int i = e % kDS, j = 4 * (e / kDS);
    if (i0 + i >= Dv || j >= Dk) continue;
    const f4 val = *reinterpret_cast<const f4*>(sk + (e / kDS * kDS + i) * 4);
    float* o = dst + (int64_t)(i0 + i) * Dk + j;
    if (VEC) {
      *reinterpret_cast<f4*>(o) = val;
    } else {
#pragma unroll
      for (int y = 0; y < 4; ++y)
        if (j + y < Dk) o[y] = val[y];
    }
  }
}

// ------------------------------------------------------- forward sweep ----
template <typename TIn, int JT, bool VEC>
__global__ __launch_bounds__(kSwThreads, 1) void fwd_chunked_kernel(FwdChunkedArgs A) {
  using L = SL<JT>;
  constexpr int DKP = L::DKP, KLD = L::KLD;
  constexpr int JW = JT / 4;  // Dk tiles per wave in the state update
  static_assert(JT % 4 == 0, "four waves of update tiles cover the Dk tiles");
  constexpr int UB = L::B0, EB = L::B1, ES = L::B2;  // U, E, diag(ks) E
  extern __shared__ __align__(16) float sm[];
  const FwdSweepArgs& a = A.s;
  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ v = static_cast<const TIn*>(a.v);
  TIn* __restrict__ y = static_cast<TIn*>(a.y);
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const SweepBlock wb = sweep_block();
  const TileRange tr = tile_range(a, wb.b, wb.h);
  const int i0 = wb.x * kDS, h = wb.h, b = tr.b;
  const int hk = h / (Hv / Hk);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 15, lq = l >> 4;
  const int tb = w & 3, nt = w >> 2;         // step-by-row tile
  const int mt = w & 1, jg = JW * (w >> 1);  // state update tiles
  const int tw = 16 * tb;
  const int64_t bh = (int64_t)b * Hv + h;
  const int64_t mat = (int64_t)Dv * Dk;
  // step strides of k, q and of v, y (the host bounds 64 steps of either to
  // fit an int)
  const int kst = Hk * Dk, vst = Hv * Dv;
  auto kq_base = [&](int c) { return ((int64_t)b * T + c * a.L) * kst + (int64_t)hk * Dk; };

  KQPrefetch<TIn, JT, VEC> kq;
  kq.init(tid);

  // state tiles in the accumulator layout of the update: tile nj, register u
  // <-> row i = 16 mt + 4 lq + u, column j = 16 (jg + nj) + lr
  f4 Sacc[JW];
#pragma unroll
  for (int nj = 0; nj < JW; ++nj)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 16 * mt + 4 * lq + u, j = 16 * (jg + nj) + lr;
      const bool ok = a.S0 != nullptr && i0 + i < Dv && j < Dk;
      Sacc[nj][u] = ok ? a.S0[ok ? tr.s0 * mat + (int64_t)(i0 + i) * Dk + j : 0] : 0.f;
    }
  tiles_to_lds<JW>(sm + L::SK, Sacc, mt, jg, lq, lr);
  kq.fetch(k, q, kq_base(tr.c0), min(a.L, T - tr.c0 * a.L), kst, Dk);

  // v, y of this wave's tile: step tw + 4 lq + u, row i0 + 16 nt + lr
  for (int c = tr.c0; c < tr.c1; ++c) {
    // lane indices re-derived in each chunk from an opaque copy of the
    // thread id: the compiler then recomputes the cheap per-lane addresses
    // instead of holding dozens of them in registers across the loop
    int tl = tid;
    asm volatile("" : "+v"(tl));
    kq.tid = tl;
    const int l = tl & 63, lr = l & 15, lq = l >> 4;
    const int ti = 16 * nt + lr;
    const bool iok = i0 + ti < Dv;
    const int t0 = c * a.L;
    const int n = min(a.L, T - t0);
    const float* __restrict__ rec = A.prep + (bh * a.nch + c) * kChunkPrepStride;
    const int64_t vbase = ((int64_t)b * T + t0) * vst + (int64_t)h * Dv + i0;
    kq.deposit(sm + L::KL, sm + L::QL);
    // this chunk's operands, issued before the next chunk's k, q so that
    // waiting for them never waits for those; held as loaded, masked at use
    float tf[16], mf[16], gam[4], ksc[4];
    TIn vr[4];
    uint32_t vm = 0;
    load_frags(rec + kPrT, tb, l, tf);
    {
      const f4 g4 = *reinterpret_cast<const f4*>(rec + kPrGam + tw + 4 * lq);
      const f4 k4 = *reinterpret_cast<const f4*>(rec + kPrKs + tw + 4 * lq);
#pragma unroll
      for (int u = 0; u < 4; ++u) gam[u] = g4[u], ksc[u] = k4[u];
    }
    const float gend = rec[kPrGend];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = tw + 4 * lq + u;
      const bool ok = iok && t < n;
      vr[u] = v[vbase + (ok ? t * vst + ti : 0)];
      vm |= (uint32_t)ok << u;
    }
    {  // unconditional (a branch around loads makes every later wait a full one)
      const int cn = min(c + 1, tr.c1 - 1);
      kq.fetch(k, q, kq_base(cn), min(a.L, T - cn * a.L), kst, Dk);
    }
    __syncthreads();
    // checkpoint: the state before this chunk, from its LDS copy
    const int slot = ckpt_slot(a, c);
    if (a.Sck != nullptr && slot >= 0)
      lds_to_matrix<JT, VEC>(sm + L::SK, a.Sck + (bh * a.nslot + slot) * mat, i0, Dv, Dk, tid);

    // X = [K; Q] S0^T on this wave's tile
    f4 X[2][1];
    X[0][0] = X[1][0] = f4{0.f, 0.f, 0.f, 0.f};
    {
      // (fp32 k, q prefetch registers leave room for groups of two)
      constexpr int G = sizeof(TIn) == 2 && VEC ? 4 : 2;
      const float* const ap[2] = {sm + L::KL + (tw + lr) * KLD + lq,
                                  sm + L::QL + (tw + lr) * KLD + lq};
      state_products<DKP, KLD, G, 2, 1>(ap, sm + L::SK + ((16 * nt + lr) << 2) + lq, X);
    }
    // M is first used after two more barriers; loading it here keeps its
    // registers free during the state products
    load_frags(rec + kPrM, tb, l, mf);
    // U = V - diag(gam) X_K
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float vu = ((vm >> u) & 1) ? to_f32(vr[u]) : 0.f;
      sm[UB + (tw + 4 * lq + u) * kUBS + ti] = vu - gam[u] * X[0][0][u];
    }
    __syncthreads();

    // E = T U
    f4 E = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) E = mfma(tf[ks], sm[UB + rstep(ks, lq) * kUBS + ti], E);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = tw + 4 * lq + u;
      sm[EB + t * kUBS + ti] = E[u];
      sm[ES + t * kUBS + ti] = ksc[u] * E[u];
      if (a.E != nullptr && iok && t < n) a.E[vbase + t * vst + ti] = E[u];
    }
    __syncthreads();

    // Y = diag(gam) X_Q + M E
    {
      f4 Yv;
#pragma unroll
      for (int u = 0; u < 4; ++u) Yv[u] = gam[u] * X[1][0][u];
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) Yv = mfma(mf[ks], sm[EB + rstep(ks, lq) * kUBS + ti], Yv);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = tw + 4 * lq + u;
        if (y != nullptr && iok && t < n) st(y, vbase + t * vst + ti, Yv[u]);
      }
    }

    // S_end = gend S0 + E^T diag(ks) K
#pragma unroll
    for (int nj = 0; nj < JW; ++nj) Sacc[nj] *= gend;
    update_products<JW, KLD>(sm + ES + 16 * mt + lr, sm + L::KL + 16 * jg + lr, lq, Sacc);
    __syncthreads();  // stage reads done before it is rewritten
    tiles_to_lds<JW>(sm + L::SK, Sacc, mt, jg, lq, lr);
  }
  if (a.ST != nullptr) {
#pragma unroll
    for (int nj = 0; nj < JW; ++nj)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 16 * mt + 4 * lq + u, j = 16 * (jg + nj) + lr;
        if (i0 + i < Dv && j < Dk) a.ST[bh * mat + (int64_t)(i0 + i) * Dk + j] = Sacc[nj][u];
      }
  }
}

// ------------------------------------------- bf16 operand tiles in LDS ----
// Operands whose reduction index is the step t or the column j reach the
// bf16 MFMA through transposing LDS reads (lds_read_tr16) from tiles stored
// as they are produced: k (and q) row-major [t][j] as loaded, state or
// gradient pieces j-major [j][i] from the accumulator layout (four
// consecutive rows i per lane).  Both are written in 8-byte blocks whose
// place inside the row is XOR-swizzled, so that the blocks one instruction
// writes or reads fall on distinct banks (64 banks of 4 bytes, a half-wave
// per cycle).
//
// k, q row stride: an odd multiple of 128 bytes, so rows of opposite parity
// use opposite halves of the banks (the swizzle of tile_swz then spreads a
// transposing read over all of them).
constexpr int kq_row_stride(int dkp) { return dkp % 128 == 0 ? dkp + 64 : dkp; }
// block c (of 8) of piece row j (kDS = 32 columns) is stored at block c ^ p_swz(j)
__device__ __forceinline__ int p_swz(int j) { return (j >> 1) & 6; }

// B operand from a swizzled j-major piece [j][kDS]: B[j][i] for rows
// j = k0 .. k0 + 31 and columns i = n0 .. n0 + 15
__device__ __forceinline__ uint4 piece_operand(const uint16_t* piece, int k0, int n0, int lr,
                                               int lq) {
  const int jl = k0 + 8 * lq + (lr >> 2), jh = jl + 4;
  const int cb = (n0 >> 2) + (lr & 3);
  const uint2 lo = lds_read_tr16(piece + jl * kDS + 4 * (cb ^ p_swz(jl)));
  const uint2 hi = lds_read_tr16(piece + jh * kDS + 4 * (cb ^ p_swz(jh)));
  return uint4{lo.x, lo.y, hi.x, hi.y};
}

// bf16 k, q rows of a chunk in 8-element groups (Dk a multiple of 8), a
// chunk ahead: one 16-byte load per group, and 16-byte LDS stores into the
// row-major tiles
template <int JT, int NTH = kSwThreads>
struct KQPrefetch8 {
  static constexpr int DKP = 16 * JT;
  static constexpr int NGT = kN * DKP / 8;  // 8-column groups of one chunk
  static constexpr int NG = NGT / NTH;
  static_assert(NGT % NTH == 0 && NG <= 32, "groups per thread");
  uint32_t pm = 0;
  uint4 pk[NG], pq[NG];
  int tid;
  // group u of this thread: step qt(u), columns qj(u) .. qj(u) + 7
  __device__ __forceinline__ int qt(int u) const { return (tid + NTH * u) / (DKP / 8); }
  __device__ __forceinline__ int qj(int u) const { return 8 * ((tid + NTH * u) % (DKP / 8)); }
  __device__ __forceinline__ void init(int t) { tid = t; }
  // rows t0 .. t0 + n - 1; base = element (t0, kv head, 0); kst = row stride
  __device__ __forceinline__ void fetch(const bf16* __restrict__ k, const bf16* __restrict__ q,
                                        int64_t base, int n, int kst, int Dk) {
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < NG; ++u) {
      const int t = qt(u), j = qj(u);
      const bool ok = j < Dk && t < n;
      int64_t o = ok ? base + (int64_t)t * kst + j : 0;
      asm volatile("" : "+v"(o));  // keeps the select (no branch around the loads)
      pk[u] = *reinterpret_cast<const uint4*>(k + o);
      pq[u] = *reinterpret_cast<const uint4*>(q + o);
      m |= (uint32_t)ok << u;
    }
    pm = m;
  }
};

// The row-major k (and q) tile of a chunk from the groups fetched a chunk
// ago (zero where the mask says so)
template <int KRS, int JT>
__device__ __forceinline__ void deposit_rows(const KQPrefetch8<JT>& kq, uint16_t* kr,
                                             uint16_t* qr) {
#pragma unroll
  for (int u = 0; u < KQPrefetch8<JT>::NG; ++u) {
    const bool ok = (kq.pm >> u) & 1u;
    const int t = kq.qt(u), c = kq.qj(u) >> 3;
    // 4-element blocks 2c, 2c + 1 stay adjacent under the swizzle
    const int o = t * KRS + 4 * ((2 * c) ^ tile_swz(t));
    uint4 rk = kq.pk[u];
    rk.x = ok ? rk.x : 0u;  // component selects (a vector select goes through memory)
    rk.y = ok ? rk.y : 0u;
    rk.z = ok ? rk.z : 0u;
    rk.w = ok ? rk.w : 0u;
    *reinterpret_cast<uint4*>(kr + o) = rk;
    if (qr != nullptr) {
      uint4 rq = kq.pq[u];
      rq.x = ok ? rq.x : 0u;
      rq.y = ok ? rq.y : 0u;
      rq.z = ok ? rq.z : 0u;
      rq.w = ok ? rq.w : 0u;
      *reinterpret_cast<uint4*>(qr + o) = rq;
    }
  }
}

// -------------------------------------------- forward sweep, bf16 inputs ----
// The same sweep for bf16 k, q (Dk a multiple of 8), with the two products
// that have k or q as an operand on bf16 MFMA (v_mfma_f32_16x16x32_bf16,
// 16 times the fp32 MFMA rate): [K; Q] S^T and the update E^T diag(ks) K.
// Their other operand (the state, diag(ks) E) is fp32 and is split exactly
// into three bf16 pieces (split3_quad), so each product is three bf16 MFMAs whose
// products are exact and whose sums are fp32: the accuracy of the fp32 path.
// T U and M E, both operands fp32 (T, M from the prep record as bf16
// pieces), take the six piece products (mfma_pieces6).
//
// LDS: k row-major [kN][KRS] and the state pieces j-major [3][DKP][kDS]
// (both swizzled, read through lds_read_tr16), and the U, E and diag(ks) E
// pieces [3][kDS][KTS] (row i, column t: 16-byte operand reads of 16 rows
// at one column group, the row stride 16 bytes modulo 32, so distinct
// banks).  The k and q operands of [K; Q] S^T (16 steps x Dk per wave) come
// straight from HBM as 16-byte fragments, fetched a chunk ahead.
template <int JT>
struct SLB {
  static constexpr int DKP = 16 * JT;
  static constexpr int KRS = kq_row_stride(DKP);  // bf16 row stride of k
  static constexpr int KTS = kN + 8;              // bf16 row stride of the step pieces
  static constexpr int PS = kDS * KTS;            // bf16 stride of one step piece
  static constexpr int KR = 0;                    // float offsets below
  static constexpr int QR = KR + kN * KRS / 2;
  static constexpr int SP = QR + kN * KRS / 2;
  // Dk above 192: the E and diag(ks) E pieces overlay the q tile, which X =
  // [K; Q] S^T reads before the barrier after which they are written, and
  // which the next chunk's deposit rewrites only after the barrier that
  // follows their last reads
  static constexpr bool QALIAS = JT > kMaxJT;
  static constexpr int EP = QALIAS ? QR : SP + 3 * DKP * kDS / 2;  // diag(ks) E pieces
  static constexpr int UP = QALIAS ? SP + 3 * DKP * kDS / 2 : EP + 3 * PS / 2;  // U pieces
  static constexpr int EQ = QALIAS ? EP + 3 * PS / 2 : UP + 3 * PS / 2;          // E pieces
  static constexpr int SIZE = QALIAS ? UP + 3 * PS / 2 : EQ + 3 * PS / 2;
  static_assert((2 * KRS) % 256 == 128 && (2 * KTS) % 32 == 16, "row strides");
  static_assert(DKP % 64 == 0, "16 blocks per swizzle group");
  static_assert(QR % 4 == 0 && SP % 4 == 0 && EP % 4 == 0 && UP % 4 == 0 && EQ % 4 == 0,
                "16-byte aligned regions");
  static_assert(!QALIAS || EQ + 3 * PS / 2 <= SP, "E pieces inside the q tile");
  static_assert(SIZE * 4 <= 160 * 1024, "LDS");
};

// kDS = 32 state rows per workgroup, eight waves.  GEN: the general tile
// range and save slots (a segment replay, a save every few tiles, a strided
// S0, no y or residuals); without it every tile runs from S0 and saves its
// state and residuals, which leaves the chunk loop fewer live scalars.
template <int JT, bool SAVE, bool GEN>
__global__ __launch_bounds__(kSwThreads, 1) void fwd_chunked_bf16_kernel(FwdChunkedArgs A) {
  using L = SLB<JT>;
  constexpr int PS = L::PS;
  constexpr int DKP = L::DKP, KRS = L::KRS, KTS = L::KTS;
  constexpr int NKS = DKP / 32;  // k-steps of 32 over Dk
  constexpr int JW = JT / 4;
  static_assert(JT % 4 == 0, "four waves of update tiles cover the Dk tiles");
  extern __shared__ __align__(16) float sm[];
  uint16_t* const kr = reinterpret_cast<uint16_t*>(sm + L::KR);
  uint16_t* const qr = reinterpret_cast<uint16_t*>(sm + L::QR);
  uint16_t* const sp = reinterpret_cast<uint16_t*>(sm + L::SP);
  uint16_t* const ep = reinterpret_cast<uint16_t*>(sm + L::EP);
  uint16_t* const up = reinterpret_cast<uint16_t*>(sm + L::UP);
  uint16_t* const eq = reinterpret_cast<uint16_t*>(sm + L::EQ);
  const FwdSweepArgs& a = A.s;
  const bf16* __restrict__ q = static_cast<const bf16*>(a.q);
  const bf16* __restrict__ k = static_cast<const bf16*>(a.k);
  const bf16* __restrict__ v = static_cast<const bf16*>(a.v);
  bf16* __restrict__ y = static_cast<bf16*>(a.y);
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const SweepBlock wb = sweep_block();
  const TileRange tr = GEN ? tile_range(a, wb.b, wb.h)
                           : TileRange{wb.b, 0, a.nch, (int64_t)wb.b * a.Hv + wb.h};
  const int nslot = GEN ? a.nslot : a.nch;
  auto slot_of = [&](int c) { return GEN ? ckpt_slot(a, c) : c; };
  const int i0 = wb.x * kDS, h = wb.h, b = tr.b;
  const int hk = h / (Hv / Hk);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = sweep_tb(w), nt = w & 1;
  // T, M are lower triangular: k-step 1 of step tiles 0, 1 is zero
  const int zk = tb < 2 ? 1 : -1;
  const int mt = w & 1, jg = JW * (w >> 1);
  const int tw = 16 * tb;
  const int64_t bh = (int64_t)b * Hv + h;
  const int64_t mat = (int64_t)Dv * Dk;
  const int kst = Hk * Dk, vst = Hv * Dv;
  auto kq_base = [&](int c) { return ((int64_t)b * T + c * a.L) * kst + (int64_t)hk * Dk; };
  auto chunk_len = [&](int c) { return min(a.L, T - c * a.L); };

  // k, q rows of a chunk (for the row-major tiles), a chunk ahead
  KQPrefetch8<JT> kq;
  kq.init(tid);
  // this wave's T pieces, the step factors and v of a chunk, a chunk ahead;
  // v as four bf16 of step tw + 4 lq + (l % 4), rows 16 nt + 4 (lr / 4) ..
  // (one 8-byte load; a quad transpose gives the lane its row at steps
  // tw + 4 lq + u)
  struct ChunkIn {
    uint4 tp[2][3];
    f4 g4, k4;
    float gend;
    uint2 v2;
    bool vok;
  };
  auto fetch_in = [&](int c, int l, ChunkIn& x) __attribute__((always_inline)) {
    const int lr = l & 15, lq = l >> 4;
    const float* __restrict__ rec = A.prep + (bh * a.nch + c) * kChunkPrepStride;
    pieces_from_record(rec + kBrT, tb, l, zk, x.tp);
    x.g4 = *reinterpret_cast<const f4*>(rec + kBrGam + tw + 4 * lq);
    x.k4 = *reinterpret_cast<const f4*>(rec + kBrKs + tw + 4 * lq);
    x.gend = rec[kBrGend];
    const int t = tw + 4 * lq + (lr & 3), r4 = 16 * nt + 4 * (lr >> 2);
    const bool ok = t < chunk_len(c) && i0 + r4 < Dv;
    int64_t o = ok ? ((int64_t)b * T + c * a.L + t) * vst + (int64_t)h * Dv + i0 + r4 : 0;
    asm volatile("" : "+v"(o));  // keeps the select (no branch around the load)
    x.v2 = *reinterpret_cast<const uint2*>(v + o);
    x.vok = ok;
  };
  ChunkIn nx;
  f4 Sacc[JW];
  {
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
#pragma unroll
    for (int nj = 0; nj < JW; ++nj)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 16 * mt + 4 * lq + u, j = 16 * (jg + nj) + lr;
        const bool ok = a.S0 != nullptr && i0 + i < Dv && j < Dk;
        Sacc[nj][u] = ok ? a.S0[ok ? tr.s0 * mat + (int64_t)(i0 + i) * Dk + j : 0] : 0.f;
      }
    kq.fetch(k, q, kq_base(tr.c0), chunk_len(tr.c0), kst, Dk);
    fetch_in(tr.c0, l, nx);
  }
  // the state tiles into the three j-major bf16 pieces (and checkpoint
  // `slot`, or the sink when slot < 0; out-of-range lanes store to the sink
  // too)
  auto put_state = [&](int slot, int lr, int lq, float* sink) __attribute__((always_inline)) {
    float* __restrict__ ck = SAVE ? a.Sck + (bh * nslot + (slot >= 0 ? slot : 0)) * mat : nullptr;
    asm volatile("" : "+v"(slot));  // a per-lane select below, not a branch
#pragma unroll
    for (int nj = 0; nj < JW; ++nj) {
      const int j = 16 * (jg + nj) + lr;
      uint2 p0, p1, p2;
      split3_quad(Sacc[nj], p0, p1, p2);
      if (SAVE) {
        // after a transpose across each lane quad, lane 4a + b holds row
        // 16 mt + 4 lq + b, columns 16 (jg + nj) + 4a .. +3: one 16-byte store
        // (read once, by the reverse pass: streamed past the caches that
        // hold the k, q and record lines the workgroups share)
        const f4 rowv = quad_transpose(Sacc[nj], lr);
        const int i = 16 * mt + 4 * lq + (lr & 3), jq = 16 * (jg + nj) + 4 * (lr >> 2);
        const bool ok = slot >= 0 && i0 + i < Dv && jq < Dk;
        __builtin_nontemporal_store(
            rowv, reinterpret_cast<f4*>(ok ? ck + (int64_t)(i0 + i) * Dk + jq : sink));
      }
      const int o = j * kDS + 4 * ((4 * mt + lq) ^ p_swz(j));
      *reinterpret_cast<uint2*>(sp + 0 * DKP * kDS + o) = p0;
      *reinterpret_cast<uint2*>(sp + 1 * DKP * kDS + o) = p1;
      *reinterpret_cast<uint2*>(sp + 2 * DKP * kDS + o) = p2;
    }
  };
  {
    int tl = tid;
    asm volatile("" : "+v"(tl));
    put_state(slot_of(tr.c0), tl & 15, (tl & 63) >> 4, A.prep + kPrSink);
  }
  for (int c = tr.c0; c < tr.c1; ++c) {
    int tl = tid;
    asm volatile("" : "+v"(tl));
    kq.tid = tl;
    const int l = tl & 63, lr = l & 15, lq = l >> 4;
    const int ti = 16 * nt + lr;
    const int t0 = c * a.L;
    const int n = chunk_len(c);
    const float* __restrict__ rec = A.prep + (bh * a.nch + c) * kChunkPrepStride;
    float* const sink16 = A.prep + (bh * a.nch + c) * kChunkPrepStride + kPrSink;  // 16-byte aligned
    const int64_t vbase = ((int64_t)b * T + t0) * vst + (int64_t)h * Dv + i0;
    deposit_rows<KRS>(kq, kr, qr);
    uint4 mp[2][3];  // M pieces of this wave's step tile
    const ChunkIn cur = nx;
    const uint4(&tp)[2][3] = cur.tp;  // T pieces
    float gam[4], ksc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) gam[u] = cur.g4[u], ksc[u] = cur.k4[u];
    const float gend = cur.gend;
    // the next chunk's loads: waves 0-3 here, waves 4-7 (the other wave of
    // each SIMD) after X, so that one wave's MFMAs run while the other
    // issues
    const int cn = min(c + 1, tr.c1 - 1);
    if (w < 4) {
      kq.fetch(k, q, kq_base(cn), chunk_len(cn), kst, Dk);
      fetch_in(cn, l, nx);
    }
    __syncthreads();

    // X = [K; Q] S0^T: three bf16 pieces of S, one accumulator per piece
    f4 XK, XQ;
    {
      f4 xk[3], xq[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) xk[p] = xq[p] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        // rows tw + l % 16 of the k, q tiles, columns 32 ks + 8 (l / 16) ..:
        // 4-element blocks 2c, 2c + 1 stay adjacent under the swizzle
        const int t = tw + lr, o = t * KRS + 4 * ((2 * (4 * ks + lq)) ^ tile_swz(t));
        const uint4 ak = *reinterpret_cast<const uint4*>(kr + o);
        const uint4 aq = *reinterpret_cast<const uint4*>(qr + o);
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          const uint4 bs = piece_operand(sp + p * DKP * kDS, 32 * ks, 16 * nt, lr, lq);
          xk[p] = mfma_bf16(ak, bs, xk[p]);
          xq[p] = mfma_bf16(aq, bs, xq[p]);
        }
      }
      XK = (xk[0] + xk[1]) + xk[2];
      XQ = (xq[0] + xq[1]) + xq[2];
    }
    // this chunk's M pieces before the next chunk's loads (loads complete in
    // order: waiting for mp then waits for nothing issued after it)
    pieces_from_record(rec + kBrM, tb, l, zk, mp);
    if (w >= 4) {
      kq.fetch(k, q, kq_base(cn), chunk_len(cn), kst, Dk);
      fetch_in(cn, l, nx);
    }
    // step pieces [i][t]: this lane's rows t = tw + 4 lq .. +3 of column ti
    const int so = ti * KTS + tw + 4 * lq;
    auto put_steps = [&](uint16_t* dst, f4 v) __attribute__((always_inline)) {
      uint2 p0, p1, p2;
      split3_quad(v, p0, p1, p2);
      *reinterpret_cast<uint2*>(dst + so) = p0;
      *reinterpret_cast<uint2*>(dst + PS + so) = p1;
      *reinterpret_cast<uint2*>(dst + 2 * PS + so) = p2;
    };
    // B operand piece p of k-step ks from step pieces: rows t = 32 ks +
    // 8 (l / 16) .., column ti
    auto step_piece = [&](const uint16_t* src, int ks, int p) __attribute__((always_inline)) {
      return *reinterpret_cast<const uint4*>(src + p * PS + ti * KTS + 32 * ks + 8 * lq);
    };
    // U = V - diag(gam) X_K
    {
      f4 v4 = {__uint_as_float(cur.v2.x << 16), __uint_as_float(cur.v2.x & 0xffff0000u),
               __uint_as_float(cur.v2.y << 16), __uint_as_float(cur.v2.y & 0xffff0000u)};
#pragma unroll
      for (int u = 0; u < 4; ++u) v4[u] = cur.vok ? v4[u] : 0.f;
      v4 = quad_transpose(v4, lr);  // steps tw + 4 lq + u of row ti (exact moves)
      f4 uv;
#pragma unroll
      for (int u = 0; u < 4; ++u) uv[u] = v4[u] - gam[u] * XK[u];
      put_steps(up, uv);
    }
    __syncthreads();

    // E = T U; E and diag(ks) E as three bf16 pieces each (row i, column t)
    {
      const f4 E = mfma_pieces6(
          tp, [&](int ks, int p) { return step_piece(up, ks, p); }, zk, f4{0.f, 0.f, 0.f, 0.f});
      f4 ke;
#pragma unroll
      for (int u = 0; u < 4; ++u) ke[u] = ksc[u] * E[u];
      if (SAVE) {
        // after a transpose across each lane quad, lane 4a + b holds step
        // tw + 4 lq + b, rows 16 nt + 4a .. +3: one 16-byte store (read once,
        // by the reverse pass: non-temporal)
        const f4 er = quad_transpose(E, lr);
        const int t = tw + 4 * lq + (lr & 3), r4 = 16 * nt + 4 * (lr >> 2);
        const bool ok = (!GEN || a.E != nullptr) && t < n && i0 + r4 < Dv;
        __builtin_nontemporal_store(
            er, reinterpret_cast<f4*>(ok ? a.E + vbase + (int64_t)t * vst + r4 : sink16));
      }
      put_steps(eq, E);
      put_steps(ep, ke);
    }
    __syncthreads();

    // Y = diag(gam) X_Q + M E
    {
      f4 Yv;
#pragma unroll
      for (int u = 0; u < 4; ++u) Yv[u] = gam[u] * XQ[u];
      Yv = mfma_pieces6(mp, [&](int ks, int p) { return step_piece(eq, ks, p); }, zk, Yv);
      {
        // as E: one 8-byte store of four bf16 rows per lane
        const f4 yr = quad_transpose(Yv, lr);
        const int t = tw + 4 * lq + (lr & 3), r4 = 16 * nt + 4 * (lr >> 2);
        const bool ok = (!GEN || y != nullptr) && t < n && i0 + r4 < Dv;
        const uint2 yb = {cvt_pk_bf16(yr[0], yr[1]), cvt_pk_bf16(yr[2], yr[3])};
        __builtin_nontemporal_store((uint64_t)yb.x | ((uint64_t)yb.y << 32),
                                    ok ? reinterpret_cast<uint64_t*>(y + vbase + (int64_t)t * vst + r4)
                                       : reinterpret_cast<uint64_t*>(sink16));
      }
    }

    // S_end = gend S0 + (diag(ks) E)^T K on bf16 MFMA: A = the E pieces (row
    // i = 16 mt + l % 16), B = k (rows t, columns 16 (jg + nj) ..)
#pragma unroll
    for (int nj = 0; nj < JW; ++nj) Sacc[nj] *= gend;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 ae[3];
#pragma unroll
      for (int p = 0; p < 3; ++p)
        ae[p] = *reinterpret_cast<const uint4*>(ep + p * PS + (16 * mt + lr) * KTS + 32 * ks +
                                                8 * lq);
#pragma unroll
      for (int nj = 0; nj < JW; ++nj) {
        const uint4 bk = tile_operand<KRS>(kr, 32 * ks, 16 * (jg + nj), lr, lq);
#pragma unroll
        for (int p = 0; p < 3; ++p) Sacc[nj] = mfma_bf16(ae[p], bk, Sacc[nj]);
      }
    }
    __syncthreads();  // stage reads done before it is rewritten
    put_state(c + 1 < tr.c1 ? slot_of(c + 1) : -1, lr, lq, sink16);
  }
  if (a.ST != nullptr) {
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
#pragma unroll
    for (int nj = 0; nj < JW; ++nj)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 16 * mt + 4 * lq + u, j = 16 * (jg + nj) + lr;
        if (i0 + i < Dv && j < Dk) a.ST[bh * mat + (int64_t)(i0 + i) * Dk + j] = Sacc[nj][u];
      }
  }
}

// ------------------------------------------------------- reverse sweep ----
template <typename TIn, int JT, bool VEC>
__global__ __launch_bounds__(kSwThreads, 1) void bwd_chunked_kernel(BwdChunkedArgs A) {
  using L = SL<JT>;
  constexpr int DKP = L::DKP, KLD = L::KLD;
  constexpr int JW = JT / 4;
  static_assert(JT % 4 == 0, "four waves of update tiles cover the Dk tiles");
  // dy, then -diag(beta pre) C (dy is dead once U is formed); U; diag(pre) dy
  constexpr int DB = L::B0, UB = L::B1, DP = L::B2;
  extern __shared__ __align__(16) float sm[];
  const BwdSweepArgs& a = A.s;
  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ dy = static_cast<const TIn*>(a.dy);
  TIn* __restrict__ dv = static_cast<TIn*>(a.dv);
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const SweepBlock wb = sweep_block();
  const int i0 = wb.x * kDS, h = wb.h, b = wb.b;
  const int hk = h / (Hv / Hk);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 15, lq = l >> 4;
  const int tb = w & 3, nt = w >> 2;
  const int mt = w & 1, jg = JW * (w >> 1);
  const int tw = 16 * tb;
  const int64_t bh = (int64_t)b * Hv + h;
  const int64_t mat = (int64_t)Dv * Dk;
  const int kst = Hk * Dk, vst = Hv * Dv;
  auto kq_base = [&](int c) { return ((int64_t)b * T + c * a.L) * kst + (int64_t)hk * Dk; };
  auto v_base = [&](int c) { return ((int64_t)b * T + c * a.L) * vst + (int64_t)h * Dv + i0; };

  KQPrefetch<TIn, JT, VEC> kq;
  kq.init(tid);
  // dy of this wave's tile (step tw + 4 lq + u, row i0 + ti), a chunk ahead
  TIn dr[4];
  uint32_t dm = 0;
  auto fetch_dy = [&](int c, int lq, int ti, bool iok) __attribute__((always_inline)) {
    const int n = min(a.L, T - c * a.L);
    const int64_t base = v_base(c);
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = tw + 4 * lq + u;
      const bool ok = iok && t < n;
      dr[u] = dy[base + (ok ? t * vst + ti : 0)];
      m |= (uint32_t)ok << u;
    }
    dm = m;
  };

  // gradient tiles, same layout as the forward state tiles
  f4 Hacc[JW];
#pragma unroll
  for (int nj = 0; nj < JW; ++nj)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 16 * mt + 4 * lq + u, j = 16 * (jg + nj) + lr;
      const bool ok = a.dST != nullptr && i0 + i < Dv && j < Dk;
      Hacc[nj][u] = ok ? a.dST[ok ? bh * mat + (int64_t)(i0 + i) * Dk + j : 0] : 0.f;
    }
  const int cl = a.nch - 1;
  tiles_to_lds<JW>(sm + L::SK, Hacc, mt, jg, lq, lr);
  kq.fetch(k, q, kq_base(cl), min(a.L, T - cl * a.L), kst, Dk);
  fetch_dy(cl, lq, 16 * nt + lr, i0 + 16 * nt + lr < Dv);

  for (int c = cl; c >= 0; --c) {
    // lane indices re-derived in each chunk from an opaque copy of the
    // thread id: the compiler then recomputes the cheap per-lane addresses
    // instead of holding dozens of them in registers across the loop
    int tl = tid;
    asm volatile("" : "+v"(tl));
    kq.tid = tl;
    const int l = tl & 63, lr = l & 15, lq = l >> 4;
    const int ti = 16 * nt + lr;
    const bool iok = i0 + ti < Dv;
    const int t0 = c * a.L;
    const int n = min(a.L, T - t0);
    const float* __restrict__ rec = A.prep + (bh * a.nch + c) * kChunkPrepStride;
    const int64_t vbase = v_base(c);
    kq.deposit(sm + L::KL, sm + L::QL);
    float dyv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      dyv[u] = ((dm >> u) & 1) ? to_f32(dr[u]) : 0.f;
      sm[DB + (tw + 4 * lq + u) * kUBS + ti] = dyv[u];
    }
    float tf[16], mf[16], suf[4], pre[4], bet[4];
    load_frags(rec + kPbT, tb, l, tf);
    load_frags(rec + kPbM, tb, l, mf);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      suf[u] = rec[kPbSuf + tw + 4 * lq + u];  // (four consecutive floats each)
      pre[u] = rec[kPbPre + tw + 4 * lq + u];
      bet[u] = rec[kPbBeta + tw + 4 * lq + u];
    }
    const float pend = rec[kPbPre + n - 1];
    {
      const int cn = max(c - 1, 0);
      kq.fetch(k, q, kq_base(cn), min(a.L, T - cn * a.L), kst, Dk);
      fetch_dy(cn, lq, ti, iok);
    }
    __syncthreads();
    // slot c: the gradient after this chunk (dS_T for the last), from its LDS copy
    lds_to_matrix<JT, VEC>(sm + L::SK, a.Hck + (bh * a.nch + c) * mat, i0, Dv, Dk, tid);

    // X = K Hend^T on this wave's tile (two accumulators over the k-steps)
    f4 X[1][2];
    X[0][0] = X[0][1] = f4{0.f, 0.f, 0.f, 0.f};
    {
      constexpr int G = sizeof(TIn) == 2 && VEC ? 4 : 2;
      const float* const ap[1] = {sm + L::KL + (tw + lr) * KLD + lq};
      state_products<DKP, KLD, G, 1, 2>(ap, sm + L::SK + ((16 * nt + lr) << 2) + lq, X);
    }
    // U = diag(suf) X + Mq DY; the stage of diag(pre) DY for the update
    {
      f4 U;
#pragma unroll
      for (int u = 0; u < 4; ++u) U[u] = suf[u] * (X[0][0][u] + X[0][1][u]);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) U = mfma(mf[ks], sm[DB + rstep(ks, lq) * kUBS + ti], U);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = tw + 4 * lq + u;
        sm[UB + t * kUBS + ti] = U[u];
        sm[DP + t * kUBS + ti] = pre[u] * dyv[u];
      }
    }
    __syncthreads();

    // C = Tb U; dv = diag(beta) C; the stage of -diag(beta pre) C
    {
      f4 Cv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) Cv = mfma(tf[ks], sm[UB + rstep(ks, lq) * kUBS + ti], Cv);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = tw + 4 * lq + u;
        sm[DB + t * kUBS + ti] = -(bet[u] * pre[u]) * Cv[u];
        if (iok && t < n) {
          a.C[vbase + t * vst + ti] = Cv[u];
          st(dv, vbase + t * vst + ti, bet[u] * Cv[u]);
        }
      }
    }
    __syncthreads();

    // H_start = pre_{n-1} Hend + DY^T diag(pre) Q - C^T diag(beta pre) K
#pragma unroll
    for (int nj = 0; nj < JW; ++nj) Hacc[nj] *= pend;
    update_products<JW, KLD>(sm + DP + 16 * mt + lr, sm + L::QL + 16 * jg + lr, lq, Hacc);
    update_products<JW, KLD>(sm + DB + 16 * mt + lr, sm + L::KL + 16 * jg + lr, lq, Hacc);
    __syncthreads();  // stage reads done before it is rewritten
    tiles_to_lds<JW>(sm + L::SK, Hacc, mt, jg, lq, lr);
  }
  if (a.dS0 != nullptr) {
#pragma unroll
    for (int nj = 0; nj < JW; ++nj)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 16 * mt + 4 * lq + u, j = 16 * (jg + nj) + lr;
        if (i0 + i < Dv && j < Dk) a.dS0[bh * mat + (int64_t)(i0 + i) * Dk + j] = Hacc[nj][u];
      }
  }
}

// -------------------------------------------- reverse sweep, bf16 inputs ----
// The same reverse sweep for bf16 k, q, dy (Dk a multiple of 8), with the
// products that have k or q as an operand on bf16 MFMA, the fp32 operand
// split exactly into three bf16 pieces (as in fwd_chunked_bf16_kernel):
// K H^T, and the update DY^T diag(pre) Q - C^T diag(beta pre) K; Mq DY
// (Mq pieces against bf16 dy) and Tb U (six piece products) from the prep
// record's bf16 pieces.  k, q row-major and the gradient pieces j-major,
// read through lds_read_tr16 (the tiles above); dy, U and the diag(pre) DY
// and -diag(beta pre) C pieces [i][t] as the step pieces of the forward
// sweep.
template <int JT>
struct SLR {
  static constexpr int DKP = 16 * JT;
  static constexpr int KRS = kq_row_stride(DKP);  // bf16 row stride of k, q
  static constexpr int KTS = kN + 8;              // bf16 row stride of the step pieces
  static constexpr int PS = kDS * KTS;            // bf16 stride of one step piece
  static constexpr int KR = 0;                    // float offsets below
  static constexpr int QR = KR + kN * KRS / 2;
  static constexpr int HT = QR + kN * KRS / 2;        // gradient pieces [3][DKP][kDS]
  static constexpr int DPP = HT + 3 * DKP * kDS / 2;  // diag(pre) DY pieces [3][kDS][KTS]
  // Dk above 192: the -diag(beta pre) C pieces overlay the gradient pieces,
  // which X = K Hend^T reads before the barrier after which they are
  // written, and which are rewritten only after the barrier that follows
  // their last reads
  static constexpr bool HALIAS = JT > kMaxJT;
  static constexpr int CPP = HALIAS ? HT : DPP + 3 * PS / 2;  // -diag(beta pre) C pieces
  static constexpr int DYT = HALIAS ? DPP + 3 * PS / 2 : CPP + 3 * PS / 2;  // dy bf16 [kDS][KTS]
  static constexpr int UP = DYT + PS / 2;             // U pieces [3][kDS][KTS]
  static constexpr int SIZE = UP + 3 * PS / 2;
  static_assert((2 * KRS) % 256 == 128, "k, q row stride");
  static_assert((2 * KTS) % 32 == 16, "step-piece row stride");
  static_assert(DKP % 64 == 0, "16 blocks per swizzle group");
  static_assert(QR % 4 == 0 && HT % 4 == 0 && DPP % 4 == 0 && CPP % 4 == 0 && DYT % 4 == 0 &&
                    UP % 4 == 0,
                "alignment");
  static_assert(!HALIAS || 3 * PS <= 3 * DKP * kDS, "C pieces inside the gradient pieces");
  static_assert(SIZE * 4 <= 160 * 1024, "LDS");
};

template <int JT>
__global__ __launch_bounds__(kSwThreads, 1) void bwd_chunked_bf16_kernel(BwdChunkedArgs A) {
  using L = SLR<JT>;
  constexpr int DKP = L::DKP, KRS = L::KRS, KTS = L::KTS, PS = L::PS;
  constexpr int NKS = DKP / 32;
  constexpr int JW = JT / 4;
  static_assert(JT % 4 == 0, "four waves of update tiles cover the Dk tiles");
  extern __shared__ __align__(16) float sm[];
  uint16_t* const kr = reinterpret_cast<uint16_t*>(sm + L::KR);
  uint16_t* const qr = reinterpret_cast<uint16_t*>(sm + L::QR);
  uint16_t* const ht = reinterpret_cast<uint16_t*>(sm + L::HT);
  uint16_t* const dpp = reinterpret_cast<uint16_t*>(sm + L::DPP);
  uint16_t* const cpp = reinterpret_cast<uint16_t*>(sm + L::CPP);
  uint16_t* const dyt = reinterpret_cast<uint16_t*>(sm + L::DYT);
  uint16_t* const up = reinterpret_cast<uint16_t*>(sm + L::UP);
  const BwdSweepArgs& a = A.s;
  const bf16* __restrict__ q = static_cast<const bf16*>(a.q);
  const bf16* __restrict__ k = static_cast<const bf16*>(a.k);
  const bf16* __restrict__ dy = static_cast<const bf16*>(a.dy);
  bf16* __restrict__ dv = static_cast<bf16*>(a.dv);
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const SweepBlock wb = sweep_block();
  const int i0 = wb.x * kDS, h = wb.h, b = wb.b;
  const int hk = h / (Hv / Hk);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tb = sweep_tb(w), nt = w & 1;
  // Tb, Mq are upper triangular: k-step 0 of step tiles 2, 3 is zero
  const int zk = tb >= 2 ? 0 : -1;
  const int mt = w & 1, jg = JW * (w >> 1);
  const int tw = 16 * tb;
  const int64_t bh = (int64_t)b * Hv + h;
  const int64_t mat = (int64_t)Dv * Dk;
  const int kst = Hk * Dk, vst = Hv * Dv;
  auto kq_base = [&](int c) { return ((int64_t)b * T + c * a.L) * kst + (int64_t)hk * Dk; };
  auto v_base = [&](int c) { return ((int64_t)b * T + c * a.L) * vst + (int64_t)h * Dv + i0; };
  auto chunk_len = [&](int c) { return min(a.L, T - c * a.L); };

  KQPrefetch8<JT> kq;
  kq.init(tid);
  // dy of this wave's tile, a chunk ahead: four bf16 of step
  // tw + 4 lq + (l % 4), rows 16 nt + 4 (lr / 4) .. (one 8-byte load; a quad
  // transpose gives the lane its row ti at steps tw + 4 lq + u)
  uint2 dq2;
  bool dok = false;
  auto fetch_dy = [&](int c, int lq, int lr) __attribute__((always_inline)) {
    const int t = tw + 4 * lq + (lr & 3), r4 = 16 * nt + 4 * (lr >> 2);
    const bool ok = t < chunk_len(c) && i0 + r4 < Dv;
    int64_t o = ok ? v_base(c) + (int64_t)t * vst + r4 : 0;
    asm volatile("" : "+v"(o));  // keeps the select (no branch around the load)
    dq2 = *reinterpret_cast<const uint2*>(dy + o);
    dok = ok;
  };

  // this wave's Mq pieces and the step factors of a chunk, a chunk ahead
  struct ChunkIn {
    uint4 mp[2][3];
    f4 s4, p4, b4;
    float pend;
  };
  auto fetch_in = [&](int c, int l, ChunkIn& x) __attribute__((always_inline)) {
    const int lq = l >> 4;
    const float* __restrict__ rec = A.prep + (bh * a.nch + c) * kChunkPrepStride;
    pieces_from_record(rec + kBbM, tb, l, zk, x.mp);
    x.s4 = *reinterpret_cast<const f4*>(rec + kBbSuf + tw + 4 * lq);
    x.p4 = *reinterpret_cast<const f4*>(rec + kBbPre + tw + 4 * lq);
    x.b4 = *reinterpret_cast<const f4*>(rec + kBbBeta + tw + 4 * lq);
    x.pend = rec[kBbPre + chunk_len(c) - 1];
  };
  ChunkIn nx;

  f4 Hacc[JW];
  const int cl = a.nch - 1;
  {
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
#pragma unroll
    for (int nj = 0; nj < JW; ++nj)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 16 * mt + 4 * lq + u, j = 16 * (jg + nj) + lr;
        const bool ok = a.dST != nullptr && i0 + i < Dv && j < Dk;
        Hacc[nj][u] = ok ? a.dST[ok ? bh * mat + (int64_t)(i0 + i) * Dk + j : 0] : 0.f;
      }
    kq.fetch(k, q, kq_base(cl), chunk_len(cl), kst, Dk);
    fetch_dy(cl, lq, lr);
    fetch_in(cl, l, nx);
  }
  // gradient tiles into the three j-major bf16 pieces and into checkpoint
  // slot `slot` (slot < 0: the sink; out-of-range lanes store to the sink too)
  auto put_grad = [&](int slot, int lr, int lq, float* sink16) __attribute__((always_inline)) {
    float* __restrict__ hc = a.Hck + (bh * a.nch + (slot >= 0 ? slot : 0)) * mat;
    asm volatile("" : "+v"(slot));  // a per-lane select below, not a branch
#pragma unroll
    for (int nj = 0; nj < JW; ++nj) {
      const int j = 16 * (jg + nj) + lr;
      uint2 p0, p1, p2;
      split3_quad(Hacc[nj], p0, p1, p2);
      {
        // after a transpose across each lane quad, lane 4a + b holds row
        // 16 mt + 4 lq + b, columns 16 (jg + nj) + 4a .. +3: one 16-byte store
        // (read once, by the chunk-parallel pass: streamed past the caches)
        const f4 rowv = quad_transpose(Hacc[nj], lr);
        const int i = 16 * mt + 4 * lq + (lr & 3), jq = 16 * (jg + nj) + 4 * (lr >> 2);
        const bool ok = slot >= 0 && i0 + i < Dv && jq < Dk;
        __builtin_nontemporal_store(
            rowv, reinterpret_cast<f4*>(ok ? hc + (int64_t)(i0 + i) * Dk + jq : sink16));
      }
      const int o = j * kDS + 4 * ((4 * mt + lq) ^ p_swz(j));
      *reinterpret_cast<uint2*>(ht + 0 * DKP * kDS + o) = p0;
      *reinterpret_cast<uint2*>(ht + 1 * DKP * kDS + o) = p1;
      *reinterpret_cast<uint2*>(ht + 2 * DKP * kDS + o) = p2;
    }
  };
  {
    int tl = tid;
    asm volatile("" : "+v"(tl));
    put_grad(cl, tl & 15, (tl & 63) >> 4, A.sink);
  }

  for (int c = cl; c >= 0; --c) {
    int tl = tid;
    asm volatile("" : "+v"(tl));
    kq.tid = tl;
    const int l = tl & 63, lr = l & 15, lq = l >> 4;
    const int ti = 16 * nt + lr;
    const int n = chunk_len(c);
    const float* __restrict__ rec = A.prep + (bh * a.nch + c) * kChunkPrepStride;
    float* const sink16 = A.sink + (bh * a.nch + c) * 64;  // 16-byte aligned
    const int64_t vbase = v_base(c);
    deposit_rows<KRS>(kq, kr, qr);
    // step pieces [i][t]: this lane's rows t = tw + 4 lq .. +3 of column ti
    const int so = ti * KTS + tw + 4 * lq;
    auto put_steps = [&](uint16_t* dst, f4 v) __attribute__((always_inline)) {
      uint2 p0, p1, p2;
      split3_quad(v, p0, p1, p2);
      *reinterpret_cast<uint2*>(dst + so) = p0;
      *reinterpret_cast<uint2*>(dst + PS + so) = p1;
      *reinterpret_cast<uint2*>(dst + 2 * PS + so) = p2;
    };
    // B operand piece p of k-step ks from step pieces: rows t = 32 ks +
    // 8 (l / 16) .., column ti
    auto step_piece = [&](const uint16_t* src, int ks, int p) __attribute__((always_inline)) {
      return *reinterpret_cast<const uint4*>(src + p * PS + ti * KTS + 32 * ks + 8 * lq);
    };
    float dyv[4];
    {
      f4 d4 = {__uint_as_float(dq2.x << 16), __uint_as_float(dq2.x & 0xffff0000u),
               __uint_as_float(dq2.y << 16), __uint_as_float(dq2.y & 0xffff0000u)};
#pragma unroll
      for (int u = 0; u < 4; ++u) d4[u] = dok ? d4[u] : 0.f;
      d4 = quad_transpose(d4, lr);  // steps tw + 4 lq + u of row ti (exact moves)
      uint32_t db[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dyv[u] = d4[u];
        db[u] = __float_as_uint(d4[u]) >> 16;
      }
      *reinterpret_cast<uint2*>(dyt + so) = uint2{db[0] | (db[1] << 16), db[2] | (db[3] << 16)};
    }
    uint4 tp[2][3];  // Tb pieces of this wave's step tile
    const ChunkIn cur = nx;
    const uint4(&mp)[2][3] = cur.mp;  // Mq pieces
    float suf[4], pre[4], bet[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) suf[u] = cur.s4[u], pre[u] = cur.p4[u], bet[u] = cur.b4[u];
    const float pend = cur.pend;
    // the next chunk's loads: waves 0-3 here, waves 4-7 (the other wave of
    // each SIMD) after X, so that one wave's MFMAs run while the other
    // issues
    const int cn = max(c - 1, 0);
    if (w < 4) {
      kq.fetch(k, q, kq_base(cn), chunk_len(cn), kst, Dk);
      fetch_dy(cn, lq, lr);
      fetch_in(cn, l, nx);
    }
    __syncthreads();

    // X = K Hend^T: three bf16 pieces of H, one accumulator per piece
    f4 X;
    {
      f4 x3[3];
#pragma unroll
      for (int p = 0; p < 3; ++p) x3[p] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        // row tw + l % 16 of the k tile, columns 32 ks + 8 (l / 16) ..
        const int t = tw + lr;
        const uint4 ak =
            *reinterpret_cast<const uint4*>(kr + t * KRS + 4 * ((2 * (4 * ks + lq)) ^ tile_swz(t)));
#pragma unroll
        for (int p = 0; p < 3; ++p)
          x3[p] = mfma_bf16(ak, piece_operand(ht + p * DKP * kDS, 32 * ks, 16 * nt, lr, lq), x3[p]);
      }
      X = (x3[0] + x3[1]) + x3[2];
    }
    // this chunk's Tb pieces (first used by C = Tb U) before the next
    // chunk's loads (loads complete in order: waiting for tp then waits for
    // nothing issued after it)
    pieces_from_record(rec + kBbT, tb, l, zk, tp);
    if (w >= 4) {
      kq.fetch(k, q, kq_base(cn), chunk_len(cn), kst, Dk);
      fetch_dy(cn, lq, lr);
      fetch_in(cn, l, nx);
    }
    // U = diag(suf) X + Mq DY; diag(pre) DY as three bf16 pieces [i][t]
    {
      f4 U;
#pragma unroll
      for (int u = 0; u < 4; ++u) U[u] = suf[u] * X[u];
      // Mq DY: dy is bf16, so the three Mq pieces give the exact products
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if (ks == zk) continue;
        const uint4 bd = step_piece(dyt, ks, 0);
#pragma unroll
        for (int p = 0; p < 3; ++p) U = mfma_bf16(mp[ks][p], bd, U);
      }
      put_steps(up, U);
      f4 pd;
#pragma unroll
      for (int u = 0; u < 4; ++u) pd[u] = pre[u] * dyv[u];
      put_steps(dpp, pd);
    }
    __syncthreads();

    // C = Tb U; dv = diag(beta) C; -diag(beta pre) C as three bf16 pieces
    {
      const f4 Cv = mfma_pieces6(
          tp, [&](int ks, int p) { return step_piece(up, ks, p); }, zk, f4{0.f, 0.f, 0.f, 0.f});
      f4 pc, dvv;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pc[u] = -(bet[u] * pre[u]) * Cv[u];
        dvv[u] = bet[u] * Cv[u];
      }
      // after a transpose across each lane quad, lane 4a + b holds step
      // tw + 4 lq + b, rows 16 nt + 4a .. +3: one 16-byte C store (read once,
      // by the chunk-parallel pass: non-temporal) and one 8-byte dv store
      {
        const f4 cr = quad_transpose(Cv, lr), dr4 = quad_transpose(dvv, lr);
        const int t = tw + 4 * lq + (lr & 3), r4 = 16 * nt + 4 * (lr >> 2);
        const bool ok = t < n && i0 + r4 < Dv;
        const int64_t o = vbase + (int64_t)t * vst + r4;
        __builtin_nontemporal_store(cr, reinterpret_cast<f4*>(ok ? a.C + o : sink16));
        const uint2 dvb = {cvt_pk_bf16(dr4[0], dr4[1]), cvt_pk_bf16(dr4[2], dr4[3])};
        __builtin_nontemporal_store((uint64_t)dvb.x | ((uint64_t)dvb.y << 32),
                                    ok ? reinterpret_cast<uint64_t*>(dv + o)
                                       : reinterpret_cast<uint64_t*>(sink16));
      }
      put_steps(cpp, pc);
    }
    // H_start = pre_{n-1} Hend + (diag(pre) DY)^T Q + (-diag(beta pre) C)^T K.
    // The first two terms do not depend on C: formed here, beside the C
    // phase (the diag(pre) DY pieces are in place since the last barrier).
    auto h_update = [&](const uint16_t* steps, const uint16_t* rows)
                        __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 as[3];
#pragma unroll
        for (int p = 0; p < 3; ++p)
          as[p] = *reinterpret_cast<const uint4*>(steps + (p * kDS + 16 * mt + lr) * KTS +
                                                  32 * ks + 8 * lq);
#pragma unroll
        for (int nj = 0; nj < JW; ++nj) {
          const uint4 br = tile_operand<KRS>(rows, 32 * ks, 16 * (jg + nj), lr, lq);
#pragma unroll
          for (int p = 0; p < 3; ++p) Hacc[nj] = mfma_bf16(as[p], br, Hacc[nj]);
        }
      }
    };
#pragma unroll
    for (int nj = 0; nj < JW; ++nj) Hacc[nj] *= pend;
    h_update(dpp, qr);
    __syncthreads();
    h_update(cpp, kr);
    __syncthreads();  // stage reads done before it is rewritten
    put_grad(c - 1, lr, lq, sink16);
  }
  if (a.dS0 != nullptr) {
    const int l = tid & 63, lr = l & 15, lq = l >> 4;
#pragma unroll
    for (int nj = 0; nj < JW; ++nj)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 16 * mt + 4 * lq + u, j = 16 * (jg + nj) + lr;
        if (i0 + i < Dv && j < Dk) a.dS0[bh * mat + (int64_t)(i0 + i) * Dk + j] = Hacc[nj][u];
      }
  }
}

// ------------------------------------------------------------ launches ----
template <typename Kern, typename... Args>
hipError_t launch(Kern kern, dim3 grid, int threads, size_t lds, hipStream_t s,
                  const Args&... args) {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  hipLaunchKernelGGL(kern, grid, dim3(threads), lds, s, args...);
  const hipError_t e = hipGetLastError();
  note_launch(s);
  return e;
}

// The records of MODE (forward records to prep_f, reverse to prep_b).
template <typename TIn, int MODE>
hipError_t launch_prep(ChunkedSweepShape sh, float* prep_f, float* prep_b, hipStream_t s) {
  // per-head matrices: one per value head of a round (four waves share it),
  // or one per wave with both record sets
  constexpr int NG = MODE == kPrepBoth ? 8 : 2;
  // one workgroup per pair of a kv head's value heads (each one round, the
  // Gram matrices formed per pair) when all of them fit on the device at
  // once (three per CU), else one per kv head (the rounds one after another)
  const int npair = (sh.Hv / sh.Hk + 1) / 2;
  const int64_t pairs = (int64_t)sh.nch * sh.Hk * npair * sh.B;
  sh.pair_grid = MODE != kPrepBoth && npair > 1 && pairs <= 3 * device_cu_count();
  const dim3 grid(sh.nch, sh.pair_grid ? sh.Hk * npair : sh.Hk, sh.B);
  const size_t lds = sizeof(float) * PL<NG>::SIZE;
  if (sh.Dk % 4 == 0)
    return launch(prep_kernel<TIn, MODE, true>, grid, kPrepThreads, lds, s, sh, prep_f, prep_b);
  return launch(prep_kernel<TIn, MODE, false>, grid, kPrepThreads, lds, s, sh, prep_f, prep_b);
}

// The bf16-product sweep of JT 16-column Dk tiles.
template <int JT, bool BWD, typename Args>
hipError_t launch_bf16_sweep(const Args& A, dim3 grid, hipStream_t s) {
  if constexpr (BWD) {
    return launch(bwd_chunked_bf16_kernel<JT>, grid, kSwThreads, sizeof(float) * SLR<JT>::SIZE,
                  s, A);
  } else {
    const size_t lb = sizeof(float) * SLB<JT>::SIZE;
    const FwdSweepArgs& f = A.s;
    const bool gen = f.seg > 0 || f.ck_every != 1 || f.s0_stride != 1 || f.nslot != f.nch ||
                     f.y == nullptr || (f.Sck != nullptr && f.E == nullptr);
    if (f.Sck != nullptr)
      return gen ? launch(fwd_chunked_bf16_kernel<JT, true, true>, grid, kSwThreads, lb, s, A)
                 : launch(fwd_chunked_bf16_kernel<JT, true, false>, grid, kSwThreads, lb, s, A);
    return gen ? launch(fwd_chunked_bf16_kernel<JT, false, true>, grid, kSwThreads, lb, s, A)
               : launch(fwd_chunked_bf16_kernel<JT, false, false>, grid, kSwThreads, lb, s, A);
  }
}

template <typename TIn, bool BWD, typename Args>
hipError_t launch_sweep(const Args& A, int Dk, int Dv, int Hv, int B, hipStream_t s) {
  const dim3 grid((Dv + kDS - 1) / kDS, Hv, B);
  const int jt = (Dk + 15) / 16;
  const bool vec = Dk % 4 == 0;  // 4-element groups of a row start on a 4-element boundary
  // bf16 k, q in 8-element groups (and 4-element row blocks of the value
  // rows): the bf16-product kernels
  constexpr bool kBf16 = std::is_same<TIn, gdr::bf16>::value;
  const bool pieces = kBf16 && vec && bf16_products(true, Dk, Dv);
  auto go = [&](auto jtc, auto vc) {
    constexpr int JT = decltype(jtc)::value;
    constexpr bool V = decltype(vc)::value;
    if constexpr (kBf16 && V)
      if (pieces) return launch_bf16_sweep<JT, BWD>(A, grid, s);
    const size_t lds = sizeof(float) * SL<JT>::SIZE;
    if constexpr (BWD)
      return launch(bwd_chunked_kernel<TIn, JT, V>, grid, kSwThreads, lds, s, A);
    else
      return launch(fwd_chunked_kernel<TIn, JT, V>, grid, kSwThreads, lds, s, A);
  };
  using I4 = std::integral_constant<int, 4>;
  using I8 = std::integral_constant<int, 8>;
  using I12 = std::integral_constant<int, 12>;
  if (jt > kMaxJT) {
    // Dk above 192: the bf16-product kernels alone
    if (pieces && jt <= kMaxJTB) return launch_bf16_sweep<kMaxJTB, BWD>(A, grid, s);
    return hipErrorInvalidValue;
  }
  if (vec) {
    if (jt <= 4) return go(I4{}, std::true_type{});
    if (jt <= 8) return go(I8{}, std::true_type{});
    return go(I12{}, std::true_type{});
  }
  if (jt <= 4) return go(I4{}, std::false_type{});
  if (jt <= 8) return go(I8{}, std::false_type{});
  return go(I12{}, std::false_type{});
}

template <typename Args>
ChunkedSweepShape shape_of(const Args& a) {
  ChunkedSweepShape sh{};
  sh.B = a.B;
  sh.T = a.T;
  sh.Hk = a.Hk;
  sh.Hv = a.Hv;
  sh.Dk = a.Dk;
  sh.Dv = a.Dv;
  sh.L = a.L;
  sh.nch = a.nch;
  sh.log_g = a.log_g;
  sh.mask = a.mask;
  sh.q = a.q;
  sh.k = a.k;
  sh.g = a.g;
  sh.beta = a.beta;
  return sh;
}

template <typename TIn>
hipError_t fwd_go(const FwdChunkedArgs& A, hipStream_t s) {
  const hipError_t e =
      A.prep_b != nullptr
          ? launch_prep<TIn, kPrepBoth>(shape_of(A.s), A.prep, A.prep_b, s)
          : launch_prep<TIn, kPrepFwd>(shape_of(A.s), A.prep, nullptr, s);
  if (e != hipSuccess) return e;
  // a segment replay runs every (batch row, segment) pair side by side
  const int zb = A.s.seg > 0 ? A.s.B * ((A.s.nch + A.s.seg - 1) / A.s.seg) : A.s.B;
  return launch_sweep<TIn, false>(A, A.s.Dk, A.s.Dv, A.s.Hv, zb, s);
}

template <typename TIn>
hipError_t bwd_go(const BwdChunkedArgs& A, hipStream_t s) {
  if (A.own_prep) {
    const hipError_t e = launch_prep<TIn, kPrepBwd>(shape_of(A.s), nullptr,
                                                    const_cast<float*>(A.prep), s);
    if (e != hipSuccess) return e;
  }
  return launch_sweep<TIn, true>(A, A.s.Dk, A.s.Dv, A.s.Hv, A.s.B, s);
}

}  // namespace

bool chunked_sweep_ok(int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv, int64_t L, int64_t T,
                      bool bf16) {
  // the sweep kernels index 64 steps of k, q, v, y with int offsets
  const int64_t lim = int64_t(1) << 31;
  // Dk up to 192 on every form, up to 256 on the bf16-product sweeps
  const bool dk_ok = Dk <= 16 * kMaxJT ||
                     (Dk <= 16 * kMaxJTB && bf16_products(bf16, (int)Dk, (int)Dv));
  return dk_ok && L >= 16 && L <= kN && T >= L && kN * Hk * Dk < lim && kN * Hv * Dv < lim;
}

int64_t chunked_prep_floats(int64_t B, int64_t Hv, int64_t nch) {
  return B * Hv * nch * kChunkPrepStride;
}

hipError_t launch_fwd_chunked(const FwdChunkedArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? fwd_go<gdr::bf16>(a, s) : fwd_go<float>(a, s);
}

hipError_t launch_bwd_chunked(const BwdChunkedArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? bwd_go<gdr::bf16>(a, s) : bwd_go<float>(a, s);
}

}  // namespace gdr
