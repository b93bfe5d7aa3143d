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
// Mapping: one workgroup of 512 threads (8 waves) per (batch row, kv head,
// chunk).  It loops over the Hv/Hk value heads of the kv head in ascending
// order and accumulates dq, dk in registers, so the GQA sum has a fixed order
// and needs no atomics.  The contractions over Dv and the final products run
// on fp32 MFMA (v_mfma_f32_16x16x4_f32): the [Dk x n] plane is cut into
// 16 x 16 tiles (jt, tt) handed to the waves in jt-major order, each tile
// holding P1, P2', P3', dq and dk in the MFMA accumulator layout (lane l,
// register v: row 16 jt + 4 (l / 16) + v, column 16 tt + l % 16).  MFMA
// operands are staged in LDS "k-interleaved" ([k / 4][m][k % 4]) so that a
// fragment (lane l <-> m = l % 16, k = l / 16) is 64 consecutive floats.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kN = 64;       // max chunk length
constexpr int kNP = kN + 1;  // padded row stride of [kN][kN] LDS matrices
constexpr int kKB = 8;       // Dv rows per staged block (2 MFMA k-steps)

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int JT>
struct CL {  // LDS layout, offsets in floats
  static constexpr int DKP = 16 * JT;
  static constexpr int G = 4 * JT;  // j-groups of 4 rows (chi/psi partials)
  // Phase A stage: S0, H1 [kKB/4][DKP][4]; DY, C, E [kKB/4][kN][4]
  static constexpr int ST_S = 0, ST_H = kKB * DKP, ST_Y = 2 * kKB * DKP,
                       ST_C = ST_Y + kKB * kN, ST_E = ST_C + kKB * kN;
  static constexpr int STAGE = ST_E + kKB * kN;
  // per-head O(n^2) arrays.  Phi'/Psi' alias the stage (written after the
  // last Gram block); the chi/psi partials alias Gam/M (consumed before
  // those are formed).
  static constexpr int PHI = 0, PSI = PHI + kN * kNP, GM = PSI + kN * kNP,
                       MZ = GM + kN * kNP, VEC = MZ + kN * kNP;
  static constexpr int RED = GM;
  static_assert(2 * G * kNP <= 2 * kN * kNP, "chi/psi partials fit Gam/M");
  static_assert(STAGE <= GM, "stage stays clear of the chi/psi partials");
  static constexpr int V_G = VEC, V_B = VEC + kN, V_PRE = VEC + 2 * kN,
                       V_PREX = VEC + 3 * kN, V_SUF = VEC + 4 * kN,
                       V_CHI = VEC + 5 * kN, V_PSI = VEC + 6 * kN,
                       V_A = VEC + 7 * kN, V_SCR = VEC + 8 * kN;  // 512 floats
  static constexpr int HEAD = V_SCR + kThreads;
  // final products: K, Q blocks [kKB/4][DKP][4]
  static constexpr int FK = 0, FQ = FK + kKB * DKP;
  static constexpr int FINAL = FQ + kKB * DKP;
  // QK/KK staging: q, k [kN][kNP] j-blocks of 64
  static constexpr int QKST = 2 * kN * kNP;
  static constexpr int A_SZ0 = STAGE > HEAD ? STAGE : HEAD;
  static constexpr int A_SZ1 = A_SZ0 > FINAL ? A_SZ0 : FINAL;
  static constexpr int A_SZ = A_SZ1 > QKST ? A_SZ1 : QKST;
  // persistent per workgroup: QK, KK and the head sums W1, -W2, Wq [kN][kNP]
  static constexpr int QK = A_SZ, KK = QK + kN * kNP, W1 = KK + kN * kNP,
                       W2 = W1 + kN * kNP, WQ = W2 + kN * kNP;
  static constexpr int SIZE = WQ + kN * kNP;
};

template <typename TIn, int JT>
__global__ __launch_bounds__(kThreads) void chunk_kernel(ChunkArgs a) {
  using L = CL<JT>;
  constexpr int DKP = L::DKP;
  constexpr int NPAIR = 4 * JT;                      // (jt, tt) tiles
  constexpr int NPW = (NPAIR + kWaves - 1) / kWaves;  // tiles per wave
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
  const int64_t mat = (int64_t)Dv * Dk;

  auto qk_index = [&](int t, int j) -> int64_t {
    return ((int64_t)(b * (int64_t)T + t0 + t) * Hk + hk) * Dk + j;
  };

  // tiles of this wave
  int pj[NPW], pt[NPW];
  bool pv[NPW];
#pragma unroll
  for (int u = 0; u < NPW; ++u) {
    const int pi = w * NPW + u;
    pv[u] = (NPAIR % kWaves == 0) || pi < NPAIR;  // constant when tiles divide evenly
    pj[u] = pv[u] ? (pi >> 2) : 0;
    pt[u] = pi & 3;
  }

  // ---- QK and KK for the kv head (shared by all its value heads) ----------
  {
    float qk8[8], kk8[8];
#pragma unroll
    for (int x = 0; x < 8; ++x) qk8[x] = kk8[x] = 0.f;
    float* sq = sm;
    float* sk = sm + kN * kNP;
    for (int j0 = 0; j0 < Dk; j0 += 64) {
      constexpr int U = (kN * 64) / kThreads;
      TIn rq[U], rk[U];
      uint32_t okm = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = tid + kThreads * u;
        const int s = idx >> 6, j = j0 + (idx & 63);
        const bool ok = s < n && j < Dk;
        const int64_t o = ok ? qk_index(s, j) : 0;
        rq[u] = q[o];
        rk[u] = k[o];
        okm |= (uint32_t)ok << u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = tid + kThreads * u;
        const int s = idx >> 6, jj = idx & 63;
        const bool ok = (okm >> u) & 1;
        sq[s * kNP + jj] = ok ? to_f32(rq[u]) : 0.f;
        sk[s * kNP + jj] = ok ? to_f32(rk[u]) : 0.f;
      }
      __syncthreads();
#pragma unroll 1
      for (int x = 0; x < 8; ++x) {
        const int e = tid + kThreads * x;
        const int s = e >> 6, r = e & 63;
        float aq = qk8[x], ak = kk8[x];
#pragma unroll 4
        for (int jj = 0; jj < 64; ++jj) {
          const float kr = sk[r * kNP + jj];
          aq = fmaf(sq[s * kNP + jj], kr, aq);
          ak = fmaf(sk[s * kNP + jj], kr, ak);
        }
        qk8[x] = aq;
        kk8[x] = ak;
      }
      __syncthreads();
    }
#pragma unroll
    for (int x = 0; x < 8; ++x) {
      const int e = tid + kThreads * x;
      const int o = (e >> 6) * kNP + (e & 63);
      sm[L::QK + o] = qk8[x];
      sm[L::KK + o] = kk8[x];
      sm[L::W1 + o] = 0.f;  // running sums over the value heads
      sm[L::W2 + o] = 0.f;
      sm[L::WQ + o] = 0.f;
    }
  }

  f4 dQ[NPW], dK[NPW];
#pragma unroll
  for (int u = 0; u < NPW; ++u) dQ[u] = dK[u] = f4{0.f, 0.f, 0.f, 0.f};

  for (int hh = 0; hh < rep; ++hh) {
    const int h = hk * rep + hh;
    const int64_t bh = (int64_t)b * Hv + h;
    const float* __restrict__ S0 = a.Sck + (bh * a.nch + jc) * mat;
    const float* __restrict__ H1 = a.Hck + (bh * a.nch + jc) * mat;
    const int64_t rowbase = ((int64_t)b * T + t0) * Hv * Dv + (int64_t)h * Dv;
    const int64_t tstride = (int64_t)Hv * Dv;
    const TIn* __restrict__ dyh = dy + rowbase;
    const float* __restrict__ Eh = a.E + rowbase;
    const float* __restrict__ Ch = a.C + rowbase;

    // per-head vectors: g, beta and the running decay products
    if (tid < kN) {
      const bool ok = tid < n;
      sm[L::V_G + tid] = ok ? ld(g, (int64_t)(b * (int64_t)T + t0 + tid) * Hv + h) : 0.f;
      sm[L::V_B + tid] = ok ? ld(beta, (int64_t)(b * (int64_t)T + t0 + tid) * Hv + h) : 0.f;
    }
    __syncthreads();
    if (tid == kThreads - 1) {
      float acc = 1.f;
      for (int t = 0; t < n; ++t) {
        sm[L::V_PREX + t] = acc;
        acc *= sm[L::V_G + t];
        sm[L::V_PRE + t] = acc;
      }
      acc = 1.f;
      for (int t = n - 1; t >= 0; --t) {
        sm[L::V_SUF + t] = acc;
        acc *= sm[L::V_G + t];
      }
    }

    // Dv blocks (kKB rows) of S0, H1 and of dy, e, c are fetched into
    // registers with unconditional loads from clamped offsets and deposited
    // k-interleaved in the stage.
    constexpr int US = (kKB * DKP + kThreads - 1) / kThreads;  // S0, H1 / thread
    constexpr int UX = (kKB * kN) / kThreads;                  // dy, e, c / thread
    float fs[US], fh[US], fe[UX], fc[UX];
    TIn fy[UX];
    uint32_t fok = 0;
    float hs = 0.f;  // partial <H1, S0>
    auto fetch_x = [&](int i0) {
#pragma unroll
      for (int u = 0; u < UX; ++u) {
        const int idx = tid + kThreads * u;
        const int ii = idx % kKB, t = idx / kKB, i = i0 + ii;  // rows fastest
        const bool ok = i < Dv && t < n;
        const int64_t o = ok ? t * tstride + i : 0;
        fy[u] = dyh[o];
        fe[u] = Eh[o];
        fc[u] = Ch[o];
        fok = (fok & ~(1u << (16 + u))) | ((uint32_t)ok << (16 + u));
      }
    };
    auto fetch_s = [&](int i0) {
#pragma unroll
      for (int u = 0; u < US; ++u) {
        const int idx = tid + kThreads * u;
        const int ii = idx / DKP, j = idx - ii * DKP, i = i0 + ii;
        const bool ok = idx < kKB * DKP && i < Dv && j < Dk;
        const int64_t o = ok ? (int64_t)i * Dk + j : 0;
        fs[u] = S0[o];
        fh[u] = H1[o];
        fok = (fok & ~(1u << u)) | ((uint32_t)ok << u);
      }
    };
    auto deposit_x = [&]() {
#pragma unroll
      for (int u = 0; u < UX; ++u) {
        const int idx = tid + kThreads * u;
        const int ii = idx % kKB, t = idx / kKB;
        const bool ok = (fok >> (16 + u)) & 1;
        const int o = ((ii >> 2) * kN + t) * 4 + (ii & 3);
        sm[L::ST_Y + o] = ok ? to_f32(fy[u]) : 0.f;
        sm[L::ST_E + o] = ok ? fe[u] : 0.f;
        sm[L::ST_C + o] = ok ? fc[u] : 0.f;
      }
    };
    auto deposit_s = [&]() {  // also accumulates <H1, S0>
#pragma unroll
      for (int u = 0; u < US; ++u) {
        const int idx = tid + kThreads * u;
        if (idx < kKB * DKP) {
          const int ii = idx / DKP, j = idx - ii * DKP;
          const bool ok = (fok >> u) & 1;
          const float sv = ok ? fs[u] : 0.f, hv = ok ? fh[u] : 0.f;
          const int o = ((ii >> 2) * DKP + j) * 4 + (ii & 3);
          sm[L::ST_S + o] = sv;
          sm[L::ST_H + o] = hv;
          hs = fmaf(sv, hv, hs);
        }
      }
    };

    // ---- P1 = S0^T DY, P2' = S0^T C, P3' = H1^T E  (MFMA over Dv) ---------
    f4 P1[NPW], P2[NPW], P3[NPW];
#pragma unroll
    for (int u = 0; u < NPW; ++u) P1[u] = P2[u] = P3[u] = f4{0.f, 0.f, 0.f, 0.f};
    fetch_s(0);
    fetch_x(0);
    deposit_s();
    deposit_x();
    __syncthreads();
    for (int i0 = 0; i0 < Dv; i0 += kKB) {
      const bool more = i0 + kKB < Dv;
      if (more) {
        fetch_s(i0 + kKB);
        fetch_x(i0 + kKB);
      }
#pragma unroll 1
      for (int ks = 0; ks < kKB / 4; ++ks) {
#pragma unroll
        for (int u = 0; u < NPW; ++u) {
          if (!pv[u]) continue;
          const int ja = ((ks * DKP + pj[u] * 16 + lr) << 2) + lq;
          const int tb = ((ks * kN + pt[u] * 16 + lr) << 2) + lq;
          const float as = sm[L::ST_S + ja], ah = sm[L::ST_H + ja];
          const float by = sm[L::ST_Y + tb], bc = sm[L::ST_C + tb],
                      be = sm[L::ST_E + tb];
          P1[u] = mfma(as, by, P1[u]);
          P2[u] = mfma(as, bc, P2[u]);
          P3[u] = mfma(ah, be, P3[u]);
        }
      }
      __syncthreads();
      if (more) {
        deposit_s();
        deposit_x();
        __syncthreads();
      }
    }

    // chi, psi partials and the P terms of dq, dk (accumulator layout)
#pragma unroll
    for (int u = 0; u < NPW; ++u) {
      if (!pv[u]) continue;
      const int t = pt[u] * 16 + lr;
      const int gidx = pj[u] * 4 + lq;
      float cp = 0.f, pp = 0.f;
      if (t < n) {
        const float bt = sm[L::V_B + t];
        const float pre = sm[L::V_PRE + t], suf = sm[L::V_SUF + t];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int j = pj[u] * 16 + 4 * lq + v;
          float qv = 0.f, kv = 0.f;
          if (j < Dk) {
            qv = ld(q, qk_index(t, j));
            kv = ld(k, qk_index(t, j));
          }
          const float p2 = bt * P2[u][v], p3 = bt * P3[u][v];
          cp = fmaf(P1[u][v], qv, cp);
          cp = fmaf(-p2, kv, cp);
          pp = fmaf(p3, kv, pp);
          dQ[u][v] = fmaf(pre, P1[u][v], dQ[u][v]);
          dK[u][v] = fmaf(suf, p3, dK[u][v]);
          dK[u][v] = fmaf(-pre, p2, dK[u][v]);
        }
      }
      sm[L::RED + gidx * kNP + t] = cp;
      sm[L::RED + L::G * kNP + gidx * kNP + t] = pp;
    }
    __syncthreads();
    if (tid < n) {
      float cs = 0.f, ps = 0.f;
      for (int x = 0; x < L::G; ++x) {
        cs += sm[L::RED + x * kNP + tid];
        ps += sm[L::RED + L::G * kNP + x * kNP + tid];
      }
      sm[L::V_CHI + tid] = cs;
      sm[L::V_PSI + tid] = ps;
    }

    // ---- Phi' = DY E^T, Psi' = C E^T  (MFMA over Dv) ----------------------
    f4 GR[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) GR[u] = f4{0.f, 0.f, 0.f, 0.f};
    fetch_x(0);
    deposit_x();
    __syncthreads();
    for (int i0 = 0; i0 < Dv; i0 += kKB) {
      const bool more = i0 + kKB < Dv;
      if (more) fetch_x(i0 + kKB);
#pragma unroll 1
      for (int ks = 0; ks < kKB / 4; ++ks) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int gi = w * 4 + u;  // Gram tile: kind, (ta, tb)
          const int ta = (gi >> 2) & 3, tb = gi & 3;
          const float av = sm[((gi >> 4) ? L::ST_C : L::ST_Y) +
                              (((ks * kN + ta * 16 + lr) << 2) + lq)];
          const float bv = sm[L::ST_E + (((ks * kN + tb * 16 + lr) << 2) + lq)];
          GR[u] = mfma(av, bv, GR[u]);
        }
      }
      __syncthreads();
      if (more) {
        deposit_x();
        __syncthreads();
      }
    }

    // ---- per-head O(n^2) stage -------------------------------------------
    float* sPhi = sm + L::PHI;  // Phi'[t][r]
    float* sPsi = sm + L::PSI;  // Psi'[t][r]
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gi = w * 4 + u;
      const int ta = (gi >> 2) & 3, tb = gi & 3;
      float* dst = (gi >> 4) ? sPsi : sPhi;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        dst[(ta * 16 + 4 * lq + v) * kNP + tb * 16 + lr] = GR[u][v];
    }
    sm[L::V_SCR + tid] = hs;
    __syncthreads();
    if (tid < 64) {  // <H1, S0>: 8 partials per thread, fixed order
      float x = 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u) x += sm[L::V_SCR + tid * 8 + u];
      sm[L::V_SCR + tid * 8] = x;
    }
    if (tid >= 64 && tid < 64 + kN) {  // row r of Gam(r, t]
      const int r = tid - 64;
      float acc = 1.f;
      for (int t = 0; t < kN; ++t) {
        float val = 0.f;
        if (t == r) {
          val = 1.f;
        } else if (t > r && t < n) {
          acc *= sm[L::V_G + t];
          val = acc;
        }
        sm[L::GM + r * kNP + t] = val;
      }
    }
    __syncthreads();
    if (tid == 0) {
      float x = 0.f;
      for (int u = 0; u < 64; ++u) x += sm[L::V_SCR + u * 8];
      sm[L::V_SCR + 1] = x;  // phi0 = <H1, S0>
    }
    if (tid < n)
      st(static_cast<TIn*>(a.dbeta), (int64_t)(b * (int64_t)T + t0 + tid) * Hv + h,
         sPsi[tid * kNP + tid]);

    // running weight matrices and M
#pragma unroll 1
    for (int x = 0; x < 8; ++x) {
      const int e = tid + kThreads * x;
      const int s = e >> 6, t = e & 63;  // entry (s, t)
      if (s < n && t < n) {
        const float bs = sm[L::V_B + s], bt = sm[L::V_B + t];
        const float phi_st = sPhi[s * kNP + t], phi_ts = sPhi[t * kNP + s];
        const float psi_st = sPsi[s * kNP + t], psi_ts = sPsi[t * kNP + s];
        const float gam_st = sm[L::GM + s * kNP + t];  // Gam(s,t], s <= t
        const float gam_ts = sm[L::GM + t * kNP + s];  // Gam(t,s], t <= s
        const int o = s * kNP + t;
        // Wq[s][t] = Gam(s,t] beta_s Phi'[t][s]            (s <= t)
        if (s <= t) sm[L::WQ + o] = fmaf(gam_st * bs, phi_ts, sm[L::WQ + o]);
        // W1[s][t] = Gam(t,s] beta_t Phi'[s][t]            (s >= t)
        if (s >= t) sm[L::W1 + o] = fmaf(gam_ts * bt, phi_st, sm[L::W1 + o]);
        // -W2[s][t]: W2 = Gam(t,s] Psi[s][t] (s > t), Gam(s,t] Psi[t][s] (s < t)
        if (s > t) sm[L::W2 + o] = fmaf(-gam_ts * (bs * bt), psi_st, sm[L::W2 + o]);
        if (s < t) sm[L::W2 + o] = fmaf(-gam_st * (bs * bt), psi_ts, sm[L::W2 + o]);
        // M[s][r=t] = Phi[s][r] QK[s][r] - Psi[s][r] KK[s][r]
        sm[L::MZ + o] = (bt * phi_st) * sm[L::QK + o] -
                        ((bs * bt) * psi_st) * sm[L::KK + o];
      }
    }

    __syncthreads();
    if (tid == kThreads - 1 && n > 0) {
      // A_t = sum_{s>=t} Gam(t,s] chi_s + Gam(t,end] phi0
      float acc = sm[L::V_CHI + n - 1] + sm[L::V_SCR + 1];
      sm[L::V_A + n - 1] = acc;
      for (int t = n - 1; t > 0; --t) {
        acc = fmaf(sm[L::V_G + t], acc, sm[L::V_CHI + t - 1]);
        sm[L::V_A + t - 1] = acc;
      }
    }
    if (tid < n) {
      // B_t[r] = sum_{s>=t} Gam(t,s] M[s][r] + Gam(t,end] psi_r, for t > r;
      // store Gam(r,t-1] B_t[r] in place of M[t][r].
      const int r = tid;
      float bacc = 0.f;
      for (int t = n - 1; t > r; --t) {
        const float mtr = sm[L::MZ + t * kNP + r];
        bacc = (t == n - 1) ? mtr + sm[L::V_PSI + r]
                            : fmaf(sm[L::V_G + t + 1], bacc, mtr);
        sm[L::MZ + t * kNP + r] = sm[L::GM + r * kNP + t - 1] * bacc;
      }
    }
    __syncthreads();
    if (tid < n) {
      const int t = tid;
      float dgv = sm[L::V_PREX + t] * sm[L::V_A + t];
      for (int r = 0; r < t; ++r) dgv += sm[L::MZ + t * kNP + r];
      st(static_cast<TIn*>(a.dg), (int64_t)(b * (int64_t)T + t0 + t) * Hv + h, dgv);
    }
    __syncthreads();
  }

  // ---- dq += K Wq;  dk += Q W1 - K W2 (MFMA over the chunk steps) --------
  for (int s0 = 0; s0 < n; s0 += kKB) {
    {
      constexpr int U = (kKB * DKP + kThreads - 1) / kThreads;
      TIn rk[U], rq[U];
      uint32_t okm = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = tid + kThreads * u;
        const int ss = idx / DKP, j = idx - ss * DKP, s = s0 + ss;
        const bool ok = idx < kKB * DKP && s < n && j < Dk;
        const int64_t o = ok ? qk_index(s, j) : 0;
        rk[u] = k[o];
        rq[u] = q[o];
        okm |= (uint32_t)ok << u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = tid + kThreads * u;
        if (idx < kKB * DKP) {
          const int ss = idx / DKP, j = idx - ss * DKP;
          const bool ok = (okm >> u) & 1;
          const int o = ((ss >> 2) * DKP + j) * 4 + (ss & 3);
          sm[L::FK + o] = ok ? to_f32(rk[u]) : 0.f;
          sm[L::FQ + o] = ok ? to_f32(rq[u]) : 0.f;
        }
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int ks = 0; ks < kKB / 4; ++ks) {
      const int srow = s0 + 4 * ks + lq;  // k index of this lane's B element
#pragma unroll
      for (int u = 0; u < NPW; ++u) {
        if (!pv[u]) continue;
        const int ja = ((ks * DKP + pj[u] * 16 + lr) << 2) + lq;
        const float ak = sm[L::FK + ja], aq = sm[L::FQ + ja];
        const int wb = srow * kNP + pt[u] * 16 + lr;
        dQ[u] = mfma(ak, sm[L::WQ + wb], dQ[u]);
        dK[u] = mfma(aq, sm[L::W1 + wb], dK[u]);
        dK[u] = mfma(ak, sm[L::W2 + wb], dK[u]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < NPW; ++u) {
    if (!pv[u]) continue;
    const int t = pt[u] * 16 + lr;
    if (t >= n) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = pj[u] * 16 + 4 * lq + v;
      if (j < Dk) {
        st(static_cast<TIn*>(a.dq), qk_index(t, j), dQ[u][v]);
        st(static_cast<TIn*>(a.dk), qk_index(t, j), dK[u][v]);
      }
    }
  }
}

template <typename TIn, int JT>
hipError_t chunk_launch(const ChunkArgs& a, hipStream_t s) {
  const size_t lds = sizeof(float) * CL<JT>::SIZE;
  auto kern = chunk_kernel<TIn, JT>;
  // Opt in to more than 64 KiB of dynamic LDS; a failure here surfaces as a
  // launch error below.
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
  dim3 grid(a.nch, a.Hk, a.B);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), lds, s, a);
  return hipGetLastError();
}

template <typename TIn>
hipError_t chunk_dispatch(const ChunkArgs& a, hipStream_t s) {
  const int jt = (a.Dk + 15) / 16;
  if (jt <= 1) return chunk_launch<TIn, 1>(a, s);
  if (jt <= 2) return chunk_launch<TIn, 2>(a, s);
  if (jt <= 4) return chunk_launch<TIn, 4>(a, s);
  if (jt <= 8) return chunk_launch<TIn, 8>(a, s);
  if (jt <= 12) return chunk_launch<TIn, 12>(a, s);
  if (jt <= 16) return chunk_launch<TIn, 16>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd_chunk(const ChunkArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? chunk_dispatch<gdr::bf16>(a, s) : chunk_dispatch<float>(a, s);
}

}  // namespace gdr
