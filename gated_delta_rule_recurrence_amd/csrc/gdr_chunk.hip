// Chunk-parallel part of the gated delta rule VJP on gfx950: dq, dk, dg, dbeta.
//
// The two sweeps leave, per chunk of n <= 64 steps (t0 .. t0+n-1, local index
// t = 0..n-1) and per value head:
//   S0 = the state before the chunk (forward checkpoint),
//   H1 = dL/dS after the chunk (reverse-sweep checkpoint),
//   e_t, c_t (per row): the forward residual and G_t k_t,
// and with delta_t = beta_t e_t, dv_t = beta_t c_t every state inside the
// chunk is an explicit sum of these pieces (unrolling the two recurrences):
//   S_t = Gam(start,t] S0 + sum_{r<=t} Gam(r,t] delta_r k_r^T
//   H_t = Gam(t,end] H1 + sum_{s>t} Gam(t,s] (dy_s q_s^T - dv_s k_s^T)
// where Gam(a,b] is the product of g over the steps a+1..b, always formed as a
// running product (no ratio of cumulative decays and no division by g, which
// is what keeps dg accurate under strong decay, cf. mlx issue #4614).
// Substituting into the per-step VJP (dq_t = S_t^T dy_t,
// dk_t = G_t^T delta_t - g_t S_{t-1}^T dv_t, dg_t = <dA_t, S_{t-1}>,
// dbeta_t = e_t . c_t) turns every sum over Dv into a contraction over the
// chunk:
//   P1 = S0^T DY, P2' = S0^T C, P3' = H1^T E          [Dk x n]
//   Phi'[t][r] = dy_t . e_r,  Psi'[t][r] = c_t . e_r  [n x n]
//   QK[s][r] = q_s . k_r,     KK[s][r] = k_s . k_r    [n x n]
// followed by O(n^2) work per head and the products dq += K Wq,
// dk += Q W1 - K W2 with [n x n] weight matrices summed over the heads.
//
// Mapping: one workgroup of 256 threads (4 waves, one per SIMD, so each wave
// may hold 512 registers) per (batch row, kv head, chunk).  It loops over the
// Hv/Hk value heads of the kv head in ascending order and accumulates dq, dk
// in registers, so the GQA sum has a fixed order and needs no atomics.  Wave
// w owns the chunk steps 16w .. 16w+15: the [Dk x 16] slices of P1, P2', P3',
// dq, dk (all Dk tiles) and the rows 16w.. of Phi', Psi', QK, KK.  Every
// contraction runs on fp32 MFMA (v_mfma_f32_16x16x4_f32; bf16 inputs are
// widened as they are staged) with the accumulator layout "lane l, register
// v: row 16 i + 4 (l / 16) + v,
// column 16 j + l % 16" of a 16 x 16 tile (i, j).  The Dv contractions P and
// the Gram matrices share one pass over Dv: the dy/c fragments of a wave are
// at once the B operands of P and the A operands of Phi', Psi'.  MFMA
// operands are staged in LDS "k-interleaved" ([k / 4][m][k % 4]) so that a
// fragment (lane l <-> m = l % 16, k = l / 16) is 64 consecutive floats,
// kKB = 32 Dv rows (eight k-steps) per block, with the next block fetched
// into registers while the current one is multiplied.
//
// bf16 inputs whose Dk and Dv are multiples of 8 with 48 < Dk <= 256 take the
// eight-wave form of this computation instead, with every contraction on bf16
// MFMA (chunk_bf16_kernel, gdr_chunk_bf16.hip); this file keeps fp32 inputs
// and the other bf16 shapes.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;
constexpr int kN = 64;       // max chunk length
constexpr int kNP = kN + 4;  // padded row stride of [kN][kN] LDS matrices
constexpr int kKB = 32;      // Dv rows per staged block of the Dv pass
constexpr int kSB = 16;      // chunk steps per staged block of the final products

template <int JT>
struct CL {  // LDS layout, offsets in floats
  static constexpr int DKP = 16 * JT;
  // The Dv pass covers JPW column tiles of Dk at a time (NJP passes), which
  // bounds the live P1, P2', P3' accumulators to 3 JPW tiles per wave.
  static constexpr int JPW = JT < 4 ? JT : 4;
  static constexpr int NJP = JT / JPW;
  static constexpr int PC = 16 * JPW;  // Dk columns of one pass
  // Dv block stage: S0, H1 row-major [kKB][PCP] (rows padded so that the
  // four rows of an MFMA fragment fall in disjoint banks); DY, C, E
  // k-interleaved [kKB/4][kN][4]
  static constexpr int PCP = PC == 16 ? 48 : PC + 16;
  static constexpr int ST_S = 0, ST_H = kKB * PCP, ST_Y = 2 * kKB * PCP,
                       ST_C = ST_Y + kKB * kN, ST_E = ST_C + kKB * kN;
  static constexpr int STAGE = ST_E + kKB * kN;
  // per-head M [kN][kNP] and the Phi', Psi' accumulators of every lane
  // ([8][kThreads] f4, in lane order), after the Dv pass (alias the stage)
  static constexpr int MZ = 0, GRD = (MZ + kN * kNP + 3) & ~3;
  static constexpr int HEAD = GRD + 8 * kThreads * 4;
  // q, k stage of the QK/KK pass: [16][kN][4] each (64 Dk columns)
  static constexpr int QS = 0, KS = 64 * kN, QKST = 2 * 64 * kN;
  // k, q stage of the final products: [kSB/4][DKP][4] each
  static constexpr int FK = 0, FQ = kSB * DKP, FINAL = 2 * kSB * DKP;
  static constexpr int A_SZ0 = STAGE > HEAD ? STAGE : HEAD;
  static constexpr int A_SZ1 = A_SZ0 > QKST ? A_SZ0 : QKST;
  static constexpr int A_SZ = A_SZ1 > FINAL ? A_SZ1 : FINAL;
  // per-head vectors
  static constexpr int VEC = A_SZ;
  static constexpr int V_G = VEC, V_B = VEC + kN, V_PRE = VEC + 2 * kN,
                       V_PREX = VEC + 3 * kN, V_SUF = VEC + 4 * kN,
                       V_CHI = VEC + 5 * kN, V_PSI = VEC + 6 * kN,
                       V_A = VEC + 7 * kN, V_SCR = VEC + 8 * kN;  // kThreads
  // persistent per workgroup: QK, KK, the head sums W1 (lower triangle
  // with the diagonal; Wq = W1^T) and -W2 (strict lower triangle; W2 is
  // symmetric), and the decay products GM of the current value head
  // [kN][kNP]
  static_assert(V_SCR % 4 == 0, "16-byte reads of the partials");
  static constexpr int QK = V_SCR + kThreads, KK = QK + kN * kNP,
                       W1 = KK + kN * kNP, W2 = W1 + kN * kNP, GM = W2 + kN * kNP;
  static constexpr int SIZE = GM + kN * kNP;
  static_assert(SIZE * 4 <= 160 * 1024, "LDS budget of one workgroup");
  static_assert(JT % JPW == 0, "whole passes");
};

// Four consecutive elements p[o .. o+3] as fp32; elements at or beyond `lim`
// (and all four when !ok) read as 0.  VEC: o is a multiple of 4 and the
// four are either all below lim or all at/above it, so one vector load does.
template <bool VEC, typename T>
__device__ __forceinline__ f4 ld4(const T* __restrict__ p, int64_t o, bool ok,
                                  int lim) {
  f4 r = {0.f, 0.f, 0.f, 0.f};
  if constexpr (VEC) {
    if constexpr (sizeof(T) == 4) {
      const float4 x = *reinterpret_cast<const float4*>(p + (ok ? o : 0));
      r = f4{x.x, x.y, x.z, x.w};
    } else {
      const uint2 x = *reinterpret_cast<const uint2*>(p + (ok ? o : 0));
      r = f4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u),
             __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xffff0000u)};
    }
    if (!ok) r = f4{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const bool good = ok && x < lim;
      const T v = p[good ? o + x : 0];  // never an address past the row
      r[x] = good ? to_f32(v) : 0.f;
    }
  }
  return r;
}

template <typename TIn, int JT, bool VEC>
__global__ __launch_bounds__(kThreads, 1) void chunk_kernel(ChunkArgs a) {
  using L = CL<JT>;
  constexpr int DKP = L::DKP;
  constexpr int JPW = L::JPW, NJP = L::NJP, PC = L::PC;
  constexpr int PCP = L::PCP;
  constexpr int NSQ = kKB * PC / 4;  // 4-column quads of a pass's S0 slice
  constexpr int SQT = (NSQ + kThreads - 1) / kThreads;  // per thread
  constexpr int NFB = (kSB / 4) * (DKP / 4);  // 4x4 blocks of a k, q step block
  static_assert(SQT <= 4 && NFB <= kThreads, "staging shares per thread");
  extern __shared__ __align__(16) float sm[];

  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ g = static_cast<const TIn*>(a.g);
  const TIn* __restrict__ beta = static_cast<const TIn*>(a.beta);
  const TIn* __restrict__ dy = static_cast<const TIn*>(a.dy);

  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const int jc = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int rep = Hv / Hk;
  const int t0 = jc * a.L;
  const int n = min(a.L, T - t0);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l = tid & 63;
  const int lr = l & 15, lq = l >> 4;
  const int tw = 16 * w;  // first chunk step of this wave's tiles
  const int64_t mat = (int64_t)Dv * Dk;

  auto qk_index = [&](int t, int j) __attribute__((always_inline)) -> int64_t {
    return ((int64_t)(b * (int64_t)T + t0 + t) * Hk + hk) * Dk + j;
  };

  f4 dQ[JT], dK[JT];
#pragma unroll
  for (int u = 0; u < JT; ++u) dQ[u] = dK[u] = f4{0.f, 0.f, 0.f, 0.f};

  // staging roles: thread tid moves the quads tid + 256 u (row qd / (PC/4),
  // columns 4 (qd % (PC/4))..) of a pass's S0 and H1 slices, and two quads
  // (step ts, rows 4 iq.. and 4 iq + 16..) of dy, e and c.
  const int ts = tid >> 2, iq = tid & 3;
  // final products: thread tid < NFB moves the 4x4 block (steps 4 fb..,
  // columns 4 fj..) of k and q
  const int fb = tid / (DKP / 4), fj = tid % (DKP / 4);
  const bool f_role = tid < NFB;

  // ---- the block stream of the Dv passes ---------------------------------
  // Blocks are numbered over the whole workgroup, gb = (hh NJP + jp) nbk +
  // blk, with nbk (blocks per pass) rounded up to even; a block past Dv reads
  // as zeros.  Two register slots carry blocks gb and gb + 1 while block gb -
  // 1 is multiplied out of LDS, so every load has two MFMA phases to land,
  // and the first blocks of the next pass or value head are in flight while
  // the current one finishes.
  const int nbk = (((Dv + kKB - 1) / kKB) + 1) & ~1;
  const int nblk_all = rep * NJP * nbk;
  const int64_t tstride = (int64_t)Hv * Dv;
  struct Slot {
    Quad<float, VEC> s[SQT], h[SQT], e[2], c[2];
    Quad<TIn, VEC> y[2];
    uint32_t ms;  // validity: 4 bits per S0/H1 quad, then 4 per dy/e/c quad
  };
  Slot RA, RB;
  float hs = 0.f;  // partial <H1, S0> of the current value head
  auto fetch = [&](Slot& R, int gbi) __attribute__((always_inline)) {
    const int hb = gbi / (NJP * nbk);
    const int rem = gbi - hb * (NJP * nbk);
    const int jp = rem / nbk;
    const int i0 = (rem - jp * nbk) * kKB;
    const int64_t bh = (int64_t)b * Hv + hk * rep + hb;
    const float* __restrict__ S0 = a.Sck + (bh * a.nch + jc) * mat;
    const float* __restrict__ H1 = a.Hck + (bh * a.nch + jc) * mat;
    const int64_t rowbase = ((int64_t)b * T + t0) * tstride + (bh - (int64_t)b * Hv) * Dv;
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < SQT; ++u) {
      const int qd = tid + kThreads * u;
      const int i = i0 + qd / (PC / 4), j = PC * jp + 4 * (qd % (PC / 4));
      const bool ok = qd < NSQ && i < Dv && j < Dk;
      const int64_t o = (int64_t)i * Dk + j;
      R.s[u].load(S0, o, ok, Dk - j);
      R.h[u].load(H1, o, ok, Dk - j);
      m |= Quad<float, VEC>::mask(ok, Dk - j) << (4 * u);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = i0 + 4 * iq + 16 * u;
      const bool ok = ts < n && i < Dv;
      const int64_t o = rowbase + ts * tstride + i;
      R.y[u].load(dy, o, ok, Dv - i);
      R.e[u].load(a.E, o, ok, Dv - i);
      R.c[u].load(a.C, o, ok, Dv - i);
      m |= Quad<float, VEC>::mask(ok, Dv - i) << (16 + 4 * u);
    }
    R.ms = m;
  };
  // a block's S0, H1 slices and dy, E, C rows to the stage
  auto deposit = [&](const Slot& R) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < SQT; ++u) {
      const int qd = tid + kThreads * u;
      if (qd < NSQ) {
        const uint32_t mu = (R.ms >> (4 * u)) & 15u;
        const int o = (qd / (PC / 4)) * PCP + 4 * (qd % (PC / 4));
        *reinterpret_cast<f4*>(sm + L::ST_S + o) = R.s[u].get(mu);
        *reinterpret_cast<f4*>(sm + L::ST_H + o) = R.h[u].get(mu);
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t mu = (R.ms >> (16 + 4 * u)) & 15u;
      const int o = ((iq + 4 * u) * kN + ts) << 2;
      *reinterpret_cast<f4*>(sm + L::ST_Y + o) = R.y[u].get(mu);
      *reinterpret_cast<f4*>(sm + L::ST_E + o) = R.e[u].get(mu);
      *reinterpret_cast<f4*>(sm + L::ST_C + o) = R.c[u].get(mu);
    }
  };
  // g, beta of step tid (threads tid < kN), a value head ahead; an identity
  // step (mask byte 0) has g = 1, beta = 0
  const bool gb_ok = tid < n;
  const bool gb_skip = gb_ok && skipped(a.mask, b, T, t0 + tid);
  auto gb_index = [&](int hh) {
    return (int64_t)(b * (int64_t)T + t0 + (gb_ok ? tid : 0)) * Hv + hk * rep + hh;
  };
  // ---- QK and KK for the kv head (shared by all its value heads) ----------
  {
    f4 acc[8];  // QK tiles (w, 0..3), KK tiles (w, 0..3)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = f4{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < Dk; j0 += 64) {
      // 64 steps x 64 columns of q and k: 4 quads of 4 columns per thread
      f4 rq[4], rk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int qi = tid + kThreads * u;
        const int s = qi >> 4, j = j0 + 4 * (qi & 15);
        const bool ok = s < n && j < Dk;
        rq[u] = ld4<VEC>(q, qk_index(ok ? s : 0, ok ? j : 0), ok, Dk - j);
        rk[u] = ld4<VEC>(k, qk_index(ok ? s : 0, ok ? j : 0), ok, Dk - j);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int qi = tid + kThreads * u;
        const int s = qi >> 4, jq = qi & 15;
        *reinterpret_cast<f4*>(sm + L::QS + (jq * kN + s) * 4) = rq[u];
        *reinterpret_cast<f4*>(sm + L::KS + (jq * kN + s) * 4) = rk[u];
      }
      __syncthreads();
#pragma unroll 2
      for (int ks = 0; ks < 16; ++ks) {
        const int fw = ((ks * kN + tw + lr) << 2) + lq;
        const float aq = sm[L::QS + fw], ak = sm[L::KS + fw];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const float bk = sm[L::KS + ((ks * kN + 16 * tb + lr) << 2) + lq];
          acc[tb] = mfma(aq, bk, acc[tb]);
          acc[4 + tb] = mfma(ak, bk, acc[4 + tb]);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int o = (tw + 4 * lq + v) * kNP + 16 * tb + lr;
        sm[L::QK + o] = acc[tb][v];
        sm[L::KK + o] = acc[4 + tb][v];
      }
#pragma unroll
    for (int x = 0; x < 16; ++x) {  // running sums over the value heads
      const int e = tid + kThreads * x;
      const int o = (e >> 6) * kNP + (e & 63);
      sm[L::W1 + o] = 0.f;
      sm[L::W2 + o] = 0.f;
    }
  }

  TIn g_nx = g[gb_index(0)], b_nx = beta[gb_index(0)];
  fetch(RA, 0);
  fetch(RB, 1);

  for (int hh = 0; hh < rep; ++hh) {
    // per-head vectors: g, beta and the running decay products
    if (tid < kN) {
      sm[L::V_G + tid] = !gb_ok ? 0.f : gb_skip ? 1.f : decay_of(to_f32(g_nx), a.log_g);
      sm[L::V_B + tid] = gb_ok && !gb_skip ? to_f32(b_nx) : 0.f;
    }
    {
      const int hn = hh + 1 < rep ? hh + 1 : hh;  // (unconditional: clamped)
      g_nx = g[gb_index(hn)];
      b_nx = beta[gb_index(hn)];
    }
    const int h = hk * rep + hh;
    __syncthreads();
    if (w == 3) {  // decay products along the chunk, one step per lane
      // pre[t] = Gam(start, t], prex[t] = Gam(start, t-1], suf[t] = Gam(t, end]
      const float gi = l < n ? sm[L::V_G + l] : 1.f;
      const float ge = (l >= 1 && l <= n) ? sm[L::V_G + l - 1] : 1.f;
      const float gs = (l >= 1 && l < n) ? sm[L::V_G + n - l] : 1.f;  // lane l <-> t = n-1-l
      sm[L::V_PRE + l] = wave_prefix_product(gi);
      sm[L::V_PREX + l] = wave_prefix_product(ge);
      const float sf = wave_prefix_product(gs);
      if (l < n) sm[L::V_SUF + n - 1 - l] = sf;
    }
    // Gam(r, t] for r, t in the chunk: row r is read after the Dv passes
    {  // rows r = 16 w .. 16 w + 15 of Gam(r, t] (lane l <-> t = l): the
       // wave's last row by a product scan, the others up from it as running
       // products, Gam(r, t] = g_{r+1} Gam(r+1, t] (1 where t <= r)
      const float gl = l < n ? sm[L::V_G + l] : 1.f;
      const int rl = tw + 15;
      float y = wave_prefix_product(l > rl ? gl : 1.f);
      sm[L::GM + rl * kNP + l] = l == rl ? 1.f : ((l > rl && l < n) ? y : 0.f);
#pragma unroll 5
      for (int i = 14; i >= 0; --i) {
        const int r = tw + i;
        const float gr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), r + 1));
        y = l > r ? gr * y : 1.f;
        sm[L::GM + r * kNP + l] = l == r ? 1.f : ((l > r && l < n) ? y : 0.f);
      }
    }

    // ---- passes over Dv: P1, P2', P3' (JPW column tiles per pass) and, in
    // the first pass, Phi', Psi' (MFMA) --------------------------------------
    hs = 0.f;
    float cp = 0.f, pp = 0.f;  // partial chi, psi of step tw + lr
    const int tl = tw + lr;    // the step this lane accumulates
    f4 GR[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) GR[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jp = 0; jp < NJP; ++jp) {
      f4 P1[JPW], P2[JPW], P3[JPW];
#pragma unroll
      for (int u = 0; u < JPW; ++u) P1[u] = P2[u] = P3[u] = f4{0.f, 0.f, 0.f, 0.f};
      // One staged block: kKB / 4 MFMA k-steps.  The operands of k-step
      // ks + 1 are read from LDS while the MFMAs of k-step ks issue.
      auto multiply = [&]() __attribute__((always_inline)) {
        constexpr int KS = kKB / 4;
        const bool gram = jp == 0;  // Phi', Psi' ride along in the first pass
        float by[2], bc[2], bw[2], be[2][4], as[2][JPW], ah[2][JPW];
        auto rd = [&](int ks, int x) __attribute__((always_inline)) {
          const int fw = ((ks * kN + tw + lr) << 2) + lq;
          by[x] = sm[L::ST_Y + fw];
          bc[x] = sm[L::ST_C + fw];
          bw[x] = sm[L::ST_E + fw];
          if (gram) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
              be[x][tb] = sm[L::ST_E + ((ks * kN + 16 * tb + lr) << 2) + lq];
          }
#pragma unroll
          for (int jt = 0; jt < JPW; ++jt) {
            const int fa = (4 * ks + lq) * PCP + 16 * jt + lr;
            as[x][jt] = sm[L::ST_S + fa];
            ah[x][jt] = sm[L::ST_H + fa];
          }
        };
        auto mm = [&](int x) __attribute__((always_inline)) {
#pragma unroll
          for (int jt = 0; jt < JPW; ++jt) {
            P1[jt] = mfma(as[x][jt], by[x], P1[jt]);
            P2[jt] = mfma(as[x][jt], bc[x], P2[jt]);
            P3[jt] = mfma(ah[x][jt], bw[x], P3[jt]);
            // the fragments of one wave cover the slice once: <H1, S0>
            if (w == 0) hs = fmaf(as[x][jt], ah[x][jt], hs);
          }
          if (gram) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
              GR[tb] = mfma(by[x], be[x][tb], GR[tb]);
              GR[4 + tb] = mfma(bc[x], be[x][tb], GR[4 + tb]);
            }
          }
        };
        static_assert(KS % 2 == 0, "k-steps in pairs");
        rd(0, 0);
#pragma unroll 1
        for (int ks = 0; ks < KS; ks += 2) {
          rd(ks + 1, 1);
          mm(0);
          if (ks + 2 < KS) rd(ks + 2, 0);
          mm(1);
        }
      };
      // q, k of this lane's step for the pass's chi/psi, loaded before the
      // pass's block loads so that waiting for them never waits for those
      Quad<TIn, VEC> qq[JPW], kq[JPW];
      uint32_t qkm = 0;
#pragma unroll
      for (int jt = 0; jt < JPW; ++jt) {
        const int j = 16 * (JPW * jp + jt) + 4 * lq;
        const bool ok = tl < n && j < Dk;
        const int64_t o = qk_index(ok ? tl : 0, ok ? j : 0);
        qq[jt].load(q, o, ok, Dk - j);
        kq[jt].load(k, o, ok, Dk - j);
        qkm |= Quad<TIn, VEC>::mask(ok, Dk - j) << (4 * jt);
      }
      const int gbase = (hh * NJP + jp) * nbk;
      // nbk >= 2: a do-while keeps the loads in flight identical on every
      // path out of the loop (the waits for qq/kq then skip the ring's loads)
      int blk = 0;
      do {
        const int gb = gbase + blk;
        __syncthreads();  // the stage is no longer read
        deposit(RA);
        __syncthreads();
        // unconditional (clamped) refills: every path has the same loads in
        // flight, so the wait before a deposit covers only that slot
        fetch(RA, min(gb + 2, nblk_all - 1));
        multiply();
        __syncthreads();
        deposit(RB);
        __syncthreads();
        fetch(RB, min(gb + 3, nblk_all - 1));
        multiply();
        blk += 2;
      } while (blk < nbk);

      // chi, psi and the P terms of dq, dk (accumulator layout: the lane
      // holds step tl and the rows 16 (JPW jp + jt) + 4 lq + v)
      if (tl < n) {
        const float bt = sm[L::V_B + tl];
        const float pre = sm[L::V_PRE + tl], suf = sm[L::V_SUF + tl];
#pragma unroll
        for (int jt = 0; jt < JPW; ++jt) {
          const int J = JPW * jp + jt;
          const f4 qv = qq[jt].get((qkm >> (4 * jt)) & 15u);
          const f4 kv = kq[jt].get((qkm >> (4 * jt)) & 15u);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p2 = bt * P2[jt][v], p3 = bt * P3[jt][v];
            cp = fmaf(P1[jt][v], qv[v], cp);
            cp = fmaf(-p2, kv[v], cp);
            pp = fmaf(p3, kv[v], pp);
            dQ[J][v] = fmaf(pre, P1[jt][v], dQ[J][v]);
            dK[J][v] = fmaf(suf, p3, dK[J][v]);
            dK[J][v] = fmaf(-pre, p2, dK[J][v]);
          }
        }
      }
    }
    // the four lanes of a step (lq = 0..3) hold disjoint row sets
    cp += __shfl_xor(cp, 16);
    cp += __shfl_xor(cp, 32);
    pp += __shfl_xor(pp, 16);
    pp += __shfl_xor(pp, 32);
    if (lq == 0) {
      sm[L::V_CHI + tl] = tl < n ? cp : 0.f;
      sm[L::V_PSI + tl] = tl < n ? pp : 0.f;
    }
    __syncthreads();  // the stage is free: the O(n^2) arrays alias it

    // ---- per-head O(n^2) stage -------------------------------------------
    sm[L::V_SCR + tid] = hs;
    f4* const grd = reinterpret_cast<f4*>(sm + L::GRD);
#pragma unroll
    for (int u = 0; u < 8; ++u) grd[u * kThreads + tid] = GR[u];
    __syncthreads();
    if (w == 0) {  // phi0 = <H1, S0> from the 256 partials, in a fixed order
      const f4 x4 = *reinterpret_cast<const f4*>(sm + L::V_SCR + 4 * l);
      const float x = rowsum16((x4[0] + x4[1]) + (x4[2] + x4[3]));
      const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
      const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
      const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
      const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
      if (l == 0) sm[L::V_SCR + 1] = (r0 + r1) + (r2 + r3);
    }

    // Running weight matrices, M and dbeta, from the Phi', Psi' accumulators
    // as each lane left them: register v of tile tb holds entry (t, r),
    // t = tw + 4 lq + v, r = 16 tb + lr.  The arrays are disjoint LDS regions:
    // restrict-qualified pointers let the loads of later entries issue ahead
    // of the stores of earlier ones.
    {
      const float* __restrict__ vB = sm + L::V_B;
      const float* __restrict__ pGM = sm + L::GM;
      const float* __restrict__ pQK = sm + L::QK;
      const float* __restrict__ pKK = sm + L::KK;
      float* __restrict__ pW1 = sm + L::W1;
      float* __restrict__ pW2 = sm + L::W2;
      float* __restrict__ pMZ = sm + L::MZ;
      float bt[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) bt[v] = vB[tw + 4 * lq + v];
#pragma unroll 2
      for (int tb = 0; tb < 4; ++tb) {
        const int r = 16 * tb + lr;
        const float br = vB[r];
        const f4 phi4 = grd[tb * kThreads + tid], psi4 = grd[(4 + tb) * kThreads + tid];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = tw + 4 * lq + v;
          const bool in = t < n && r < n;
          const int o = t * kNP + r;
          const float phi = phi4[v], psi = psi4[v];
          const float gam = pGM[r * kNP + t];  // Gam(r,t] (r <= t)
          const float qk = pQK[o], kk = pKK[o], w1 = pW1[o], w2 = pW2[o];
          // W1[t][r] = Gam(r,t] beta_r Phi'[t][r]            (t >= r)
          // (Wq[s][t] = Gam(s,t] beta_s Phi'[t][s], s <= t, is W1[t][s])
          if (in && t >= r) pW1[o] = fmaf(gam * br, phi, w1);
          // -W2[t][r] = -Gam(r,t] beta_t beta_r Psi'[t][r]    (t > r)
          if (in && t > r) pW2[o] = fmaf(-gam * (bt[v] * br), psi, w2);
          // M[t][r] = Phi[t][r] QK[t][r] - Psi[t][r] KK[t][r] (0 outside the
          // chunk: M is multiplied over all 64 rows)
          pMZ[o] = in ? (br * phi) * qk - ((bt[v] * br) * psi) * kk : 0.f;
        }
      }
      // dbeta_t = Psi'[t][t]: tile tb = w, lanes lr = 4 lq + v
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        if (tb != w) continue;
        const int v = lr & 3, t = tw + lr;
        const float d = sm[L::GRD + ((4 + tb) * kThreads + tid) * 4 + v];
        if ((lr >> 2) == lq && t < n)  // g and beta do not enter an identity step
          st(static_cast<TIn*>(a.dbeta), (int64_t)(b * (int64_t)T + t0 + t) * Hv + h,
             skipped(a.mask, b, T, t0 + t) ? 0.f : d);
      }
    }

    __syncthreads();
    // dg.  With A_t = sum_{s>=t} Gam(t,s] chi_s + Gam(t,end] phi0 and
    // B_t[r] = sum_{s>=t} Gam(t,s] M[s][r] + Gam(t,end] psi_r:
    //   dg_t = prex[t] A_t + sum_{r<t} Gam(r,t-1] B_t[r].
    // Gam(t,s] for s >= t is row t of GM (0 below the diagonal), so the sums
    // over s are the product GM [M | chi] (MFMA; chi rides in column 0 of a
    // fifth tile), and the sum over r is a 16-lane row reduction.
    {
      f4 Bt[5];
#pragma unroll
      for (int u = 0; u < 5; ++u) Bt[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const int sk = 4 * ks + lq;
        const float ga = sm[L::GM + (tw + lr) * kNP + sk];  // A[t][s]
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
          Bt[tb] = mfma(ga, sm[L::MZ + sk * kNP + 16 * tb + lr], Bt[tb]);
        const float cb = lr == 0 ? sm[L::V_CHI + sk] : 0.f;
        Bt[4] = mfma(ga, cb, Bt[4]);
      }
      const float phi0 = sm[L::V_SCR + 1];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = tw + 4 * lq + v;
        const float gend = n > 0 ? sm[L::GM + t * kNP + n - 1] : 0.f;  // Gam(t,end]
        float acc = 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const int r = 16 * tb + lr;
          const float bv = fmaf(gend, sm[L::V_PSI + r], Bt[tb][v]);
          const float gr = r < t ? sm[L::GM + r * kNP + t - 1] : 0.f;  // Gam(r,t-1]
          acc = fmaf(gr, bv, acc);
        }
        acc = rowsum16(acc);
        if (lr == 0 && t < n) {
          const float At = fmaf(gend, phi0, Bt[4][v]);
          const float dgt = fmaf(sm[L::V_PREX + t], At, acc);
          // with log-decay input: dL/dlg_t = g_t dL/dg_t
          st(static_cast<TIn*>(a.dg), (int64_t)(b * (int64_t)T + t0 + t) * Hv + h,
             skipped(a.mask, b, T, t0 + t) ? 0.f : a.log_g ? sm[L::V_G + t] * dgt : dgt);
        }
      }
    }
    __syncthreads();
  }

  // ---- dq += K Wq;  dk += Q W1 - K W2 (MFMA over the chunk steps) --------
  // Wq = W1^T; W1 is held on and below the diagonal, -W2 below it (W2 is
  // symmetric with a zero diagonal, which reads back as the zero the array
  // was cleared to)
  auto wq_at = [&](int s, int t) __attribute__((always_inline)) {
    return sm[L::W1 + t * kNP + s];
  };
  auto w1_at = [&](int s, int t) __attribute__((always_inline)) {
    return sm[L::W1 + s * kNP + t];
  };
  auto w2_at = [&](int s, int t) __attribute__((always_inline)) {
    return sm[L::W2 + (s > t ? s * kNP + t : t * kNP + s)];
  };
  for (int s0 = 0; s0 < n; s0 += kSB) {
    if (f_role) {
      f4 rk[4], rq[4];
      const int j = 4 * fj;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int s = s0 + 4 * fb + x;
        const bool ok = s < n && j < Dk;
        rk[x] = ld4<VEC>(k, qk_index(ok ? s : 0, ok ? j : 0), ok, Dk - j);
        rq[x] = ld4<VEC>(q, qk_index(ok ? s : 0, ok ? j : 0), ok, Dk - j);
      }
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int o = ((fb * DKP + 4 * fj + y) << 2);
        *reinterpret_cast<f4*>(sm + L::FK + o) = f4{rk[0][y], rk[1][y], rk[2][y], rk[3][y]};
        *reinterpret_cast<f4*>(sm + L::FQ + o) = f4{rq[0][y], rq[1][y], rq[2][y], rq[3][y]};
      }
    }
    __syncthreads();
#pragma unroll 2
    for (int ks = 0; ks < kSB / 4; ++ks) {
      const int sb = s0 + 4 * ks + lq, tc = tw + lr;  // B: rows s, columns t
      const float wq = wq_at(sb, tc), w1 = w1_at(sb, tc), w2 = w2_at(sb, tc);
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        const int fa = ((ks * DKP + 16 * jt + lr) << 2) + lq;
        const float ak = sm[L::FK + fa], aq = sm[L::FQ + fa];
        dQ[jt] = mfma(ak, wq, dQ[jt]);
        dK[jt] = mfma(aq, w1, dK[jt]);
        dK[jt] = mfma(ak, w2, dK[jt]);
      }
    }
    __syncthreads();
  }
  {
    const int t = tw + lr;
    if (t < n) {
#pragma unroll
      for (int jt = 0; jt < JT; ++jt) {
        if constexpr (VEC) {
          // columns 16 jt + 4 lq .. +3 of step t: one 4-element store each
          const int j = 16 * jt + 4 * lq;
          if (j < Dk) {
            if constexpr (std::is_same<TIn, bf16>::value) {
              *reinterpret_cast<uint2*>(static_cast<bf16*>(a.dq) + qk_index(t, j)) =
                  uint2{cvt_pk_bf16(dQ[jt][0], dQ[jt][1]), cvt_pk_bf16(dQ[jt][2], dQ[jt][3])};
              *reinterpret_cast<uint2*>(static_cast<bf16*>(a.dk) + qk_index(t, j)) =
                  uint2{cvt_pk_bf16(dK[jt][0], dK[jt][1]), cvt_pk_bf16(dK[jt][2], dK[jt][3])};
            } else {
              *reinterpret_cast<f4*>(static_cast<float*>(a.dq) + qk_index(t, j)) = dQ[jt];
              *reinterpret_cast<f4*>(static_cast<float*>(a.dk) + qk_index(t, j)) = dK[jt];
            }
          }
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int j = 16 * jt + 4 * lq + v;
            if (j < Dk) {
              st(static_cast<TIn*>(a.dq), qk_index(t, j), dQ[jt][v]);
              st(static_cast<TIn*>(a.dk), qk_index(t, j), dK[jt][v]);
            }
          }
        }
      }
    }
  }
}

template <typename TIn, int JT, bool VEC>
hipError_t chunk_launch(const ChunkArgs& a, hipStream_t s) {
  const size_t lds = sizeof(float) * CL<JT>::SIZE;
  auto kern = chunk_kernel<TIn, JT, VEC>;
  // Opt in to more than 64 KiB of dynamic LDS; a failure here surfaces as a
  // launch error below.
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
  dim3 grid(a.nch, a.Hk, a.B);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a);
  const hipError_t e = hipGetLastError();
  note_launch(s);
  return e;
}

template <typename TIn, bool VEC>
hipError_t chunk_dispatch_jt(const ChunkArgs& a, hipStream_t s) {
  const int jt = (a.Dk + 15) / 16;
  if (jt <= 1) return chunk_launch<TIn, 1, VEC>(a, s);
  if (jt <= 2) return chunk_launch<TIn, 2, VEC>(a, s);
  if (jt <= 4) return chunk_launch<TIn, 4, VEC>(a, s);
  if (jt <= 8) return chunk_launch<TIn, 8, VEC>(a, s);
  if (jt <= 12) return chunk_launch<TIn, 12, VEC>(a, s);
  if (jt <= 16) return chunk_launch<TIn, 16, VEC>(a, s);
  return hipErrorInvalidValue;
}

// Vector staging needs every 4-element group of a k/q row (Dk) and of a
// dy/e/c row (Dv) to start on a 4-element boundary.
template <typename TIn>
hipError_t chunk_dispatch(const ChunkArgs& a, hipStream_t s) {
  if (a.Dk % 4 == 0 && a.Dv % 4 == 0) return chunk_dispatch_jt<TIn, true>(a, s);
  return chunk_dispatch_jt<TIn, false>(a, s);
}

}  // namespace

hipError_t launch_bwd_chunk(const ChunkArgs& a, bool bf16, hipStream_t s) {
  if (bf16 && chunk_bf16_ok(a)) return launch_chunk_bf16(a, s);
  return bf16 ? chunk_dispatch<gdr::bf16>(a, s) : chunk_dispatch<float>(a, s);
}

}  // namespace gdr
