// Chunk-parallel part of the gated delta rule VJP for bf16 inputs on gfx950:
// dq, dk, dg, dbeta of every chunk from the sweeps' checkpoints, with every
// contraction on bf16 MFMA over exact three-piece splits of the fp32
// operands.  The mathematics is that of chunk_kernel (gdr_chunk.hip): with
// S0, H1 the states around a chunk of n <= 64 steps and e_t, c_t its rows,
//   P1 = S0^T DY, P2' = S0^T C, P3' = H1^T E           [Dk x n]
//   Phi'[t][r] = dy_t . e_r,  Psi'[t][r] = c_t . e_r   [n x n]
// then O(n^2) work per value head and dq += K Wq, dk += Q W1 - K W2.
//
// Mapping: one workgroup of 512 threads (eight waves, two per SIMD, so that
// one wave's MFMAs run while the other waits for LDS or memory; at most 256
// registers each) per (batch row, kv head, chunk), looping over the value
// heads of the kv head in ascending order (the GQA sum in a fixed order, no
// atomics); on short sequences, per (batch row, group of the kv head's value
// heads, chunk), the groups' dq, dk terms summed afterwards (chunk_head_split).  Wave w owns the chunk steps 16 (w % 4) .. +15 and the half
// h = w / 4 of every 64-column group of Dk: its Dk tiles are 4 p + 2 h + {0, 1}
// (p = 0 .. Dk/64 - 1).  The two waves of a step tile split the Dv-pass
// products, the Gram matrices (by column tile), the weight-matrix update and
// the dg product.  Per Dv block of 32 rows, all 512 threads stage the S0, H1
// slices of the pass and the chunk's dy, C, E rows in LDS as bf16 pieces
// (each value split once), and every wave reads its MFMA operands from there.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kThreads = 512;
constexpr int kN = 64;       // max chunk length
constexpr int kNP = kN + 4;  // padded row stride of the [kN][kN] LDS matrices
constexpr int kKB = 32;      // Dv rows per block: one 16x16x32 k-step

constexpr int cmax(int x, int y) { return x > y ? x : y; }

template <int JT>
struct BL {  // LDS layout, offsets in floats
  static constexpr int DKP = 16 * JT;
  static constexpr int NJP = JT / 4;  // 64-column passes over Dk
  static constexpr int NT = JT / 2;   // Dk tiles per wave
  static constexpr int PC = 64;       // Dk columns of one pass
  // Dv block stage: S0, H1 slices as three bf16 pieces each [3][kKB][PC]
  // (swizzled tiles, rows i, read through lds_read_tr16); dy as one plane and
  // C, E as three, [kN][YS] each (rows t, columns i; the row stride of 80
  // bytes puts the 16-byte reads of 16 rows on distinct banks)
  static constexpr int YS = kKB + 8;
  static constexpr int SP = kKB * PC, YP = kN * YS;  // bf16 per plane
  static constexpr int BS_S = 0, BS_H = BS_S + 3 * SP / 2, BS_Y = BS_H + 3 * SP / 2,
                       BS_C = BS_Y + YP / 2, BS_E = BS_C + 3 * YP / 2;
  static constexpr int BSTAGE = BS_E + 3 * YP / 2;
  // per-head M^T as three bf16 pieces [3][kN][MS] and the Phi', Psi'
  // accumulators of every lane ([4][kThreads] f4, in lane order), after the
  // Dv passes (alias the block stage)
  static constexpr int MS = kN + 8;
  static constexpr int MZ = 0, GRD = (3 * kN * MS / 2 + 3) & ~3;
  static constexpr int HEAD = GRD + 4 * kThreads * 4;
  // q, k rows of the QK/KK pass as bf16 [kN][KGS]
  static constexpr int KGS = DKP + 8;
  static constexpr int BQ = 0, BK = kN * KGS / 2, QKST = kN * KGS;
  // final products: k, q rows as swizzled bf16 tiles [kN][KFS] (the row
  // stride an odd multiple of 128 bytes); a weight matrix as three bf16
  // pieces [3][kN][WS] in the QK, KK region (free after the value heads)
  static constexpr int KFS = DKP % 128 == 0 ? DKP + 64 : DKP;
  static constexpr int BFK = 0, BFQ = kN * KFS / 2, BFINAL = kN * KFS;
  static constexpr int WS = kN + 8;
  // Dk above 192 (WIDE): the QK/KK stage and the final k, q tiles overlay the
  // per-head vectors and GM too, which the first value head writes only after
  // the stage is released and the last one reads before the final products
  static constexpr bool WIDE = JT > 12;
  static constexpr int A_SZ = WIDE ? cmax(BSTAGE, HEAD)
                                   : cmax(cmax(BSTAGE, HEAD), cmax(QKST, BFINAL));
  // per-head vectors; chi, psi and the dg partials of the two column halves
  static constexpr int VEC = A_SZ;
  static constexpr int V_G = VEC, V_B = VEC + kN, V_PRE = VEC + 2 * kN,
                       V_PREX = VEC + 3 * kN, V_SUF = VEC + 4 * kN, V_CHI = VEC + 5 * kN,
                       V_PSI = VEC + 7 * kN, V_DG = VEC + 9 * kN, V_SCR = VEC + 11 * kN;
  // persistent: QK, KK, the head sums W1 (lower triangle with the diagonal;
  // Wq = W1^T) and -W2 (strict lower triangle; W2 is symmetric); and the
  // decay products GM of the current value head [kN][kNP] (after the
  // vectors when WIDE, else last)
  static constexpr int GM0 = V_SCR + kThreads;
  static constexpr int QK = WIDE ? GM0 + kN * kNP : GM0, KK = QK + kN * kNP, W1 = KK + kN * kNP,
                       W2 = W1 + kN * kNP, GM = WIDE ? GM0 : W2 + kN * kNP;
  static constexpr int SIZE = (WIDE ? W2 : GM) + kN * kNP;
  static_assert(JT % 4 == 0 && JT <= 16, "64-column passes, Dk <= 256");
  static_assert(!WIDE || (QKST <= QK && BFINAL <= QK), "overlays end before QK");
  static_assert((2 * YS) % 32 == 16 && (2 * MS) % 32 == 16 && (2 * KGS) % 32 == 16 &&
                    (2 * WS) % 32 == 16,
                "row strides: odd multiples of 16 bytes");
  static_assert(3 * kN * WS / 2 <= 2 * kN * kNP, "W pieces fit the QK, KK region");
  static_assert(V_SCR % 4 == 0 && V_CHI % 4 == 0, "16-byte reads of the partials");
  static_assert(SIZE * 4 <= 160 * 1024, "LDS budget of one workgroup");
};

__device__ __forceinline__ f4 six(const uint4 (&x)[3], const uint4 (&y)[3], f4 acc) {
  // the six piece products down to the order of fp32 rounding
  acc = mfma_bf16(x[0], y[0], acc);
  acc = mfma_bf16(x[0], y[1], acc);
  acc = mfma_bf16(x[1], y[0], acc);
  acc = mfma_bf16(x[0], y[2], acc);
  acc = mfma_bf16(x[2], y[0], acc);
  acc = mfma_bf16(x[1], y[1], acc);
  return acc;
}

__device__ __forceinline__ void pieces8(const f4& x0, const f4& x1, uint4 (&f)[3]) {
  uint2 a0, a1, a2, b0, b1, b2;
  split3_quad(x0, a0, a1, a2);
  split3_quad(x1, b0, b1, b2);
  f[0] = uint4{a0.x, a0.y, b0.x, b0.y};
  f[1] = uint4{a1.x, a1.y, b1.x, b1.y};
  f[2] = uint4{a2.x, a2.y, b2.x, b2.y};
}

// three bf16 pieces of four fp32 values to planes `stride` apart, as 8-byte
// blocks at element o
__device__ __forceinline__ void put3(uint16_t* dst, int stride, int o, f4 v) {
  uint2 p0, p1, p2;
  split3_quad(v, p0, p1, p2);
  *reinterpret_cast<uint2*>(dst + o) = p0;
  *reinterpret_cast<uint2*>(dst + stride + o) = p1;
  *reinterpret_cast<uint2*>(dst + 2 * stride + o) = p2;
}

template <int JT>
__global__ __launch_bounds__(kThreads, 1) void chunk_bf16_kernel(ChunkArgs a) {
  using L = BL<JT>;
  constexpr int DKP = L::DKP, NJP = L::NJP, NT = L::NT, PC = L::PC;
  extern __shared__ __align__(16) float sm[];

  const bf16* __restrict__ q = static_cast<const bf16*>(a.q);
  const bf16* __restrict__ k = static_cast<const bf16*>(a.k);
  const bf16* __restrict__ g = static_cast<const bf16*>(a.g);
  const bf16* __restrict__ beta = static_cast<const bf16*>(a.beta);
  const bf16* __restrict__ dy = static_cast<const bf16*>(a.dy);

  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const int rep = Hv / Hk;
  // all the value heads of kv head blockIdx.y, or (a.part) the group
  // blockIdx.y % ng of a.hpw of them, their dq, dk terms to a.part
  const bool split = a.part != nullptr;
  const int ng = split ? rep / a.hpw : 1;  // head groups per kv head
  const int jc = blockIdx.x, b = blockIdx.z;
  const int hk = (int)blockIdx.y / ng;
  const int grp = (int)blockIdx.y - hk * ng;
  const int nh = rep / ng;      // value heads of this workgroup
  const int h_lo = grp * nh;    // the first (of the kv head)
  const int t0 = jc * a.L;
  const int n = min(a.L, T - t0);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // lane indices (re-derived at the top of every value head)
  int l = tid & 63;
  int lr = l & 15, lq = l >> 4;
  const int hf = w >> 2;         // column half
  const int tw = 16 * (w & 3);   // first chunk step of this wave's tiles
  const int64_t mat = (int64_t)Dv * Dk;

  auto qk_index = [&](int t, int j) __attribute__((always_inline)) -> int64_t {
    return ((int64_t)(b * (int64_t)T + t0 + t) * Hk + hk) * Dk + j;
  };
  // Dk tile of the wave's slot u: pass u / 2, tile 2 hf + u % 2 of the pass
  auto jtile = [&](int u) __attribute__((always_inline)) {
    return 4 * (u >> 1) + 2 * hf + (u & 1);
  };

  f4 dQ[NT], dK[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) dQ[u] = dK[u] = f4{0.f, 0.f, 0.f, 0.f};

  // staging shares: the S0, H1 quad of row sr, columns 4 sc .. of a pass's
  // slice, and the dy, C, E quad of step ys, Dv rows 4 yq .. of a block.  The
  // 32 lanes of a half-wave take steps c, c + 4, c + 8, c + 12 (step_of): with
  // the 80-byte row stride of the step planes their 8-byte writes then cover
  // the 64 banks once (four consecutive steps would overlap on 12 banks).
  auto step_of = [](int x) __attribute__((always_inline)) {
    const int q = x >> 5;
    return 16 * (q >> 2) + (q & 3) + 4 * ((x >> 3) & 3);
  };
  int sr = tid >> 4, sc = tid & 15;
  int ys = step_of(tid), yq = tid & 7;

  // ---- the block stream of the Dv passes ---------------------------------
  // Blocks are numbered over the whole workgroup, gb = (hh NJP + jp) nbk +
  // blk, with nbk (blocks per pass) rounded up to even; a block past Dv reads
  // as zeros.  Two register slots carry blocks gb and gb + 1 while block
  // gb - 1 is multiplied out of LDS, so every load has two MFMA phases to
  // land, and the first blocks of the next pass or value head are in flight
  // while the current one finishes.
  const int nbk = (((Dv + kKB - 1) / kKB) + 1) & ~1;
  const int nblk_all = nh * NJP * nbk;
  const int64_t tstride = (int64_t)Hv * Dv;
  struct Slot {
    Quad<float, true> s, h, c, e;
    uint2 y;
    uint32_t ms;  // bit 0: the S0/H1 quad is inside the tensors; bit 1: the step quad
  };
  // S0, H1 slices are read once (each pass its own columns): non-temporal
  // loads keep them from displacing the dy, C, E rows that every pass of a
  // value head reads again
  auto ld_nt = [](const float* p, int64_t o, bool ok) __attribute__((always_inline)) {
    const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p + (ok ? o : 0)));
    return float4{x[0], x[1], x[2], x[3]};
  };
  Slot RA, RB;
  float hs = 0.f;  // partial <H1, S0> of the current value head
  auto fetch = [&](Slot& R, int gbi) __attribute__((always_inline)) {
    const int hb = gbi / (NJP * nbk);
    const int rem = gbi - hb * (NJP * nbk);
    const int jp = rem / nbk;
    const int i0 = (rem - jp * nbk) * kKB;
    const int hv = hk * rep + h_lo + hb;
    const int64_t bh = (int64_t)b * Hv + hv;
    uint32_t m;
    {
      const int i = i0 + sr, j = PC * jp + 4 * sc;
      const bool ok = i < Dv && j < Dk;  // Dk a multiple of 8: the quad is all in or all out
      const int64_t o = (bh * a.nch + jc) * mat + (int64_t)i * Dk + j;
      R.s.v = ld_nt(a.Sck, o, ok);
      R.h.v = ld_nt(a.Hck, o, ok);
      m = ok ? 1u : 0u;
    }
    {
      const int i = i0 + 4 * yq;
      const bool ok = ys < n && i < Dv;  // Dv a multiple of 8: likewise
      const int64_t o = ((int64_t)b * T + t0 + ys) * tstride + (int64_t)hv * Dv + i;
      R.c.load(a.C, o, ok, 4);
      R.e.load(a.E, o, ok, 4);
      int64_t oy = ok ? o : 0;
      asm volatile("" : "+v"(oy));  // keeps the select (no branch around the load)
      R.y = *reinterpret_cast<const uint2*>(dy + oy);
      m |= ok ? 2u : 0u;
    }
    R.ms = m;
  };
  // a block's S0, H1, dy, C, E to LDS as bf16 pieces
  auto deposit = [&](const Slot& R) __attribute__((always_inline)) {
    uint16_t* const bs = reinterpret_cast<uint16_t*>(sm + L::BS_S);
    uint16_t* const bh = reinterpret_cast<uint16_t*>(sm + L::BS_H);
    uint16_t* const by = reinterpret_cast<uint16_t*>(sm + L::BS_Y);
    uint16_t* const bc = reinterpret_cast<uint16_t*>(sm + L::BS_C);
    uint16_t* const be = reinterpret_cast<uint16_t*>(sm + L::BS_E);
    {
      const uint32_t mu = (R.ms & 1u) ? 15u : 0u;
      const f4 sv = R.s.get(mu), hv = R.h.get(mu);
      // every element of the slice passes one thread once: <H1, S0>
#pragma unroll
      for (int e = 0; e < 4; ++e) hs = fmaf(sv[e], hv[e], hs);
      const int o = sr * PC + 4 * (sc ^ tile_swz(sr));
      put3(bs, L::SP, o, sv);
      put3(bh, L::SP, o, hv);
    }
    {
      const bool ok = (R.ms >> 1) & 1u;
      const uint32_t mu = ok ? 15u : 0u;
      const int o = ys * L::YS + 4 * yq;
      put3(bc, L::YP, o, R.c.get(mu));
      put3(be, L::YP, o, R.e.get(mu));
      // component selects (a vector select goes through memory)
      *reinterpret_cast<uint2*>(by + o) = uint2{ok ? R.y.x : 0u, ok ? R.y.y : 0u};
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
    // q, k rows staged as bf16, products on bf16 MFMA (exact products)
    constexpr int NCH = DKP / 8;  // 16-byte chunks per row
    constexpr int NL = (kN * NCH + kThreads - 1) / kThreads;
    uint16_t* const sq = reinterpret_cast<uint16_t*>(sm + L::BQ);
    uint16_t* const sk = reinterpret_cast<uint16_t*>(sm + L::BK);
    uint4 rq[NL], rk[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int ci = tid + kThreads * u;
      const int s = ci / NCH, j = 8 * (ci % NCH);
      const bool ok = ci < kN * NCH && s < n && j < Dk;
      int64_t o = ok ? qk_index(s, j) : 0;
      asm volatile("" : "+v"(o));  // keeps the select (no branch around the loads)
      rq[u] = *reinterpret_cast<const uint4*>(q + o);
      rk[u] = *reinterpret_cast<const uint4*>(k + o);
    }
    // the first two blocks of the Dv passes, in flight during QK and KK
    // (issued after the q, k loads: waiting for those never waits for these)
    fetch(RA, 0);
    fetch(RB, 1);
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int ci = tid + kThreads * u;
      const int s = ci / NCH, j = 8 * (ci % NCH);
      const bool ok = ci < kN * NCH && s < n && j < Dk;
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
        *reinterpret_cast<uint4*>(sq + s * L::KGS + j) = xq;
        *reinterpret_cast<uint4*>(sk + s * L::KGS + j) = xk;
      }
    }
    __syncthreads();
    // QK, KK tiles (step tile of the wave, column tiles 2 hf, 2 hf + 1)
    f4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DKP / 32; ++ks) {
      const int o = (tw + lr) * L::KGS + 32 * ks + 8 * lq;
      const uint4 aq = *reinterpret_cast<const uint4*>(sq + o);
      const uint4 ak = *reinterpret_cast<const uint4*>(sk + o);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int tb = 2 * hf + x;
        const uint4 bk =
            *reinterpret_cast<const uint4*>(sk + (16 * tb + lr) * L::KGS + 32 * ks + 8 * lq);
        acc[x] = mfma_bf16(aq, bk, acc[x]);
        acc[2 + x] = mfma_bf16(ak, bk, acc[2 + x]);
      }
    }
    __syncthreads();  // the stage is reused below
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int o = (tw + 4 * lq + v) * kNP + 16 * (2 * hf + x) + lr;
        sm[L::QK + o] = acc[x][v];
        sm[L::KK + o] = acc[2 + x][v];
      }
#pragma unroll
    for (int x = 0; x < kN * kN / kThreads; ++x) {  // running sums over the value heads
      const int e = tid + kThreads * x;
      const int o = (e >> 6) * kNP + (e & 63);
      sm[L::W1 + o] = 0.f;
      sm[L::W2 + o] = 0.f;
    }
  }

  bf16 g_nx = g[gb_index(h_lo)], b_nx = beta[gb_index(h_lo)];

  for (int hh = h_lo; hh < h_lo + nh; ++hh) {
    {  // lane indices re-derived per head from an opaque copy of the thread
       // id, so that the compiler does not hoist per-lane addresses out of
       // the loop (and spill them)
      int t_ = tid;
      asm volatile("" : "+v"(t_));
      l = t_ & 63;
      lr = l & 15;
      lq = l >> 4;
      sr = t_ >> 4;
      sc = t_ & 15;
      ys = step_of(t_);
      yq = t_ & 7;
    }
    // per-head vectors: g, beta and the running decay products
    if (tid < kN) {
      sm[L::V_G + tid] = !gb_ok ? 0.f : gb_skip ? 1.f : decay_of(to_f32(g_nx), a.log_g);
      sm[L::V_B + tid] = gb_ok && !gb_skip ? to_f32(b_nx) : 0.f;
    }
    {
      const int hn = hh + 1 < h_lo + nh ? hh + 1 : hh;  // (unconditional: clamped)
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
    {  // rows r = 8 w .. 8 w + 7 of Gam(r, t] (lane l <-> t = l): the
       // wave's last row by a product scan, the others up from it as running
       // products, Gam(r, t] = g_{r+1} Gam(r+1, t] (1 where t <= r)
      const float gl = l < n ? sm[L::V_G + l] : 1.f;
      const int rl = 8 * w + 7;
      float y = wave_prefix_product(l > rl ? gl : 1.f);
      sm[L::GM + rl * kNP + l] = l == rl ? 1.f : ((l > rl && l < n) ? y : 0.f);
#pragma unroll
      for (int i = 6; i >= 0; --i) {
        const int r = 8 * w + i;
        const float gr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), r + 1));
        y = l > r ? gr * y : 1.f;
        sm[L::GM + r * kNP + l] = l == r ? 1.f : ((l > r && l < n) ? y : 0.f);
      }
    }

    // ---- passes over Dv: P1, P2', P3' (two column tiles per wave and pass)
    // and, in the first pass, Phi', Psi' (two column tiles) -----------------
    hs = 0.f;
    float cp = 0.f, pp = 0.f;  // partial chi, psi of step tw + lr (this half's columns)
    const int tl = tw + lr;    // the step this lane accumulates
    f4 GR[4];                  // Phi' tiles 2 hf, 2 hf + 1, then Psi' tiles
#pragma unroll
    for (int u = 0; u < 4; ++u) GR[u] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jp = 0; jp < NJP; ++jp) {
      f4 P1[2], P2[2], P3[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) P1[u] = P2[u] = P3[u] = f4{0.f, 0.f, 0.f, 0.f};
      // One staged block (one k-step of 32 Dv rows): the wave's dy, C, E
      // rows tw + l % 16, Dv rows 8 (l / 16) .. from the step planes
      auto multiply = [&]() __attribute__((always_inline)) {
        const uint16_t* const bs = reinterpret_cast<const uint16_t*>(sm + L::BS_S);
        const uint16_t* const bh = reinterpret_cast<const uint16_t*>(sm + L::BS_H);
        const uint16_t* const by = reinterpret_cast<const uint16_t*>(sm + L::BS_Y);
        const uint16_t* const bc = reinterpret_cast<const uint16_t*>(sm + L::BS_C);
        const uint16_t* const be = reinterpret_cast<const uint16_t*>(sm + L::BS_E);
        const int ro = (tw + lr) * L::YS + 8 * lq;
        const uint4 fy = *reinterpret_cast<const uint4*>(by + ro);
        uint4 fc[3], fe[3];
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          fc[p] = *reinterpret_cast<const uint4*>(bc + p * L::YP + ro);
          fe[p] = *reinterpret_cast<const uint4*>(be + p * L::YP + ro);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int n0 = 16 * (2 * hf + x);
          uint4 fs[3], fh[3];
#pragma unroll
          for (int p = 0; p < 3; ++p) {
            fs[p] = tile_operand<PC>(bs + p * L::SP, 0, n0, lr, lq);
            fh[p] = tile_operand<PC>(bh + p * L::SP, 0, n0, lr, lq);
          }
          // P1 = S0^T DY; P2' = S0^T C; P3' = H1^T E
#pragma unroll
          for (int p = 0; p < 3; ++p) P1[x] = mfma_bf16(fs[p], fy, P1[x]);
          P2[x] = six(fs, fc, P2[x]);
          P3[x] = six(fh, fe, P3[x]);
        }
        if (jp == 0) {  // Phi'[t][r] = dy_t . e_r, Psi'[t][r] = c_t . e_r
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int rr = (16 * (2 * hf + x) + lr) * L::YS + 8 * lq;
            uint4 ge[3];
#pragma unroll
            for (int p = 0; p < 3; ++p) ge[p] = *reinterpret_cast<const uint4*>(be + p * L::YP + rr);
#pragma unroll
            for (int p = 0; p < 3; ++p) GR[x] = mfma_bf16(fy, ge[p], GR[x]);
            GR[2 + x] = six(fc, ge, GR[2 + x]);
          }
        }
      };
      // q, k of this lane's step for the pass's chi/psi, loaded before the
      // pass's block loads so that waiting for them never waits for those
      Quad<bf16, true> qq[2], kq[2];
      uint32_t qkm = 0;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int j = 16 * (4 * jp + 2 * hf + x) + 4 * lq;
        const bool ok = tl < n && j < Dk;
        const int64_t o = qk_index(ok ? tl : 0, ok ? j : 0);
        qq[x].load(q, o, ok, 4);
        kq[x].load(k, o, ok, 4);
        qkm |= Quad<bf16, true>::mask(ok, 4) << (4 * x);
      }
      const int gbase = ((hh - h_lo) * NJP + jp) * nbk;
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
      // holds step tl and the rows 16 J + 4 lq + v of Dk tile J)
      if (tl < n) {
        const float bt = sm[L::V_B + tl];
        const float pre = sm[L::V_PRE + tl], suf = sm[L::V_SUF + tl];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int u = 2 * jp + x;
          const f4 qv = qq[x].get((qkm >> (4 * x)) & 15u);
          const f4 kv = kq[x].get((qkm >> (4 * x)) & 15u);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p2 = bt * P2[x][v], p3 = bt * P3[x][v];
            cp = fmaf(P1[x][v], qv[v], cp);
            cp = fmaf(-p2, kv[v], cp);
            pp = fmaf(p3, kv[v], pp);
            dQ[u][v] = fmaf(pre, P1[x][v], dQ[u][v]);
            dK[u][v] = fmaf(suf, p3, dK[u][v]);
            dK[u][v] = fmaf(-pre, p2, dK[u][v]);
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
      sm[L::V_CHI + kN * hf + tl] = tl < n ? cp : 0.f;
      sm[L::V_PSI + kN * hf + tl] = tl < n ? pp : 0.f;
    }
    __syncthreads();  // the stage is free: the O(n^2) arrays alias it

    // ---- per-head O(n^2) stage -------------------------------------------
    sm[L::V_SCR + tid] = hs;
    f4* const grd = reinterpret_cast<f4*>(sm + L::GRD);
#pragma unroll
    for (int u = 0; u < 4; ++u) grd[u * kThreads + tid] = GR[u];
    __syncthreads();
    if (w == 0) {  // phi0 = <H1, S0> from the 512 partials, in a fixed order
      const f4 x0 = *reinterpret_cast<const f4*>(sm + L::V_SCR + 8 * l);
      const f4 x1 = *reinterpret_cast<const f4*>(sm + L::V_SCR + 8 * l + 4);
      const float x = rowsum16(((x0[0] + x0[1]) + (x0[2] + x0[3])) +
                               ((x1[0] + x1[1]) + (x1[2] + x1[3])));
      const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
      const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
      const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
      const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
      if (l == 0) sm[L::V_SCR + 1] = (r0 + r1) + (r2 + r3);
    }

    // Running weight matrices, M and dbeta, from the Phi', Psi' accumulators
    // as each lane left them: register v of tile x holds entry (t, r),
    // t = tw + 4 lq + v, r = 16 (2 hf + x) + lr.  The arrays are disjoint LDS
    // regions: restrict-qualified pointers let the loads of later entries
    // issue ahead of the stores of earlier ones.
    {
      const float* __restrict__ vB = sm + L::V_B;
      const float* __restrict__ pGM = sm + L::GM;
      const float* __restrict__ pQK = sm + L::QK;
      const float* __restrict__ pKK = sm + L::KK;
      float* __restrict__ pW1 = sm + L::W1;
      float* __restrict__ pW2 = sm + L::W2;
      uint16_t* __restrict__ mt = reinterpret_cast<uint16_t*>(sm + L::MZ);
      float bt[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) bt[v] = vB[tw + 4 * lq + v];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int r = 16 * (2 * hf + x) + lr;
        const float br = vB[r];
        const f4 phi4 = grd[x * kThreads + tid], psi4 = grd[(2 + x) * kThreads + tid];
        f4 m4;  // M[t][r] of this lane's four steps t
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
          m4[v] = in ? (br * phi) * qk - ((bt[v] * br) * psi) * kk : 0.f;
        }
        // M^T pieces: row r, steps tw + 4 lq .. +3
        uint2 p0, p1, p2;
        split3_quad(m4, p0, p1, p2);
        const int om = r * L::MS + tw + 4 * lq;
        *reinterpret_cast<uint2*>(mt + om) = p0;
        *reinterpret_cast<uint2*>(mt + kN * L::MS + om) = p1;
        *reinterpret_cast<uint2*>(mt + 2 * kN * L::MS + om) = p2;
      }
      // dbeta_t = Psi'[t][t]: column tile x = (w % 4) - 2 hf of the wave
      // whose half holds the diagonal tile, lanes lr = 4 lq + v
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        if (2 * hf + x != (w & 3)) continue;
        const int v = lr & 3, t = tw + lr;
        const float d = sm[L::GRD + ((2 + x) * kThreads + tid) * 4 + v];
        if ((lr >> 2) == lq && t < n)  // g and beta do not enter an identity step
          st(static_cast<bf16*>(a.dbeta), (int64_t)(b * (int64_t)T + t0 + t) * Hv + h,
             skipped(a.mask, b, T, t0 + t) ? 0.f : d);
      }
    }

    __syncthreads();
    // dg.  With A_t = sum_{s>=t} Gam(t,s] chi_s + Gam(t,end] phi0 and
    // B_t[r] = sum_{s>=t} Gam(t,s] M[s][r] + Gam(t,end] psi_r:
    //   dg_t = prex[t] A_t + sum_{r<t} Gam(r,t-1] B_t[r].
    // Gam(t,s] for s >= t is row t of GM (0 below the diagonal), so the sums
    // over s are the product GM [M | chi] (bf16 MFMA, both operands as three
    // pieces; chi rides in column 0 of a third tile of the first half), and
    // the sum over r is a 16-lane row reduction over each half's two column
    // tiles; the halves meet in LDS.
    {
      f4 Bt[3];
#pragma unroll
      for (int u = 0; u < 3; ++u) Bt[u] = f4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* const mt = reinterpret_cast<const uint16_t*>(sm + L::MZ);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // A = GM rows tw + l % 16, s = 32 ks + 8 (l / 16) ..; B = M^T pieces
        // (row r = 16 tb + l % 16)
        const int s0 = 32 * ks + 8 * lq;
        const float* const gr = sm + L::GM + (tw + lr) * kNP + s0;
        uint4 ga[3];
        pieces8(*reinterpret_cast<const f4*>(gr), *reinterpret_cast<const f4*>(gr + 4), ga);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          uint4 bm[3];
#pragma unroll
          for (int p = 0; p < 3; ++p)
            bm[p] = *reinterpret_cast<const uint4*>(mt + p * kN * L::MS +
                                                    (16 * (2 * hf + x) + lr) * L::MS + s0);
          Bt[x] = six(ga, bm, Bt[x]);
        }
        if (hf == 0) {
          const float m0 = lr == 0 ? 1.f : 0.f;
          const float* const ch = sm + L::V_CHI + s0;
          const f4 c0 = (*reinterpret_cast<const f4*>(ch) +
                         *reinterpret_cast<const f4*>(ch + kN)) * m0;
          const f4 c1 = (*reinterpret_cast<const f4*>(ch + 4) +
                         *reinterpret_cast<const f4*>(ch + kN + 4)) * m0;
          uint4 bc[3];
          pieces8(c0, c1, bc);
          Bt[2] = six(ga, bc, Bt[2]);
        }
      }
      const float phi0 = sm[L::V_SCR + 1];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = tw + 4 * lq + v;
        const float gend = n > 0 ? sm[L::GM + t * kNP + n - 1] : 0.f;  // Gam(t,end]
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int r = 16 * (2 * hf + x) + lr;
          const float psi = sm[L::V_PSI + r] + sm[L::V_PSI + kN + r];
          const float bv = fmaf(gend, psi, Bt[x][v]);
          const float gr = r < t ? sm[L::GM + r * kNP + t - 1] : 0.f;  // Gam(r,t-1]
          acc = fmaf(gr, bv, acc);
        }
        acc = rowsum16(acc);
        if (lr == 0) {
          // the first half adds prex[t] A_t
          const float At = fmaf(gend, phi0, Bt[2][v]);
          sm[L::V_DG + kN * hf + t] = hf == 0 ? fmaf(sm[L::V_PREX + t], At, acc) : acc;
        }
      }
    }
    __syncthreads();
    if (tid < n) {
      const int t = tid;
      const float dgt = sm[L::V_DG + t] + sm[L::V_DG + kN + t];
      // with log-decay input: dL/dlg_t = g_t dL/dg_t
      st(static_cast<bf16*>(a.dg), (int64_t)(b * (int64_t)T + t0 + t) * Hv + h,
         skipped(a.mask, b, T, t0 + t) ? 0.f : a.log_g ? sm[L::V_G + t] * dgt : dgt);
    }
    __syncthreads();
  }

  // ---- dq += K Wq;  dk += Q W1 - K W2 (MFMA over the chunk steps) --------
  // Wq = W1^T; W1 is held on and below the diagonal, -W2 below it (W2 is
  // symmetric with a zero diagonal, which reads back as the zero the array
  // was cleared to).  k, q (bf16) as swizzled tiles, read as A operands
  // (A[j][s] = k_s[j]) through lds_read_tr16; each W as three bf16 pieces
  // W^T [t][s] in the (then free) QK, KK region, one W at a time.
  auto wq_at = [&](int s, int t) __attribute__((always_inline)) {
    return sm[L::W1 + t * kNP + s];
  };
  auto w1_at = [&](int s, int t) __attribute__((always_inline)) {
    return sm[L::W1 + s * kNP + t];
  };
  auto w2_at = [&](int s, int t) __attribute__((always_inline)) {
    return sm[L::W2 + (s > t ? s * kNP + t : t * kNP + s)];
  };
  {
    constexpr int KFS = L::KFS, WS = L::WS;
    constexpr int NCH = DKP / 8;
    constexpr int NL = (kN * NCH + kThreads - 1) / kThreads;
    uint16_t* const fk = reinterpret_cast<uint16_t*>(sm + L::BFK);
    uint16_t* const fq = reinterpret_cast<uint16_t*>(sm + L::BFQ);
    uint16_t* const wp = reinterpret_cast<uint16_t*>(sm + L::QK);
    {
      uint4 rq[NL], rk[NL];
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int ci = tid + kThreads * u;
        const int s = ci / NCH, j = 8 * (ci % NCH);
        const bool ok = ci < kN * NCH && s < n && j < Dk;
        int64_t o = ok ? qk_index(s, j) : 0;
        asm volatile("" : "+v"(o));  // keeps the select (no branch around the loads)
        rq[u] = *reinterpret_cast<const uint4*>(q + o);
        rk[u] = *reinterpret_cast<const uint4*>(k + o);
      }
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int ci = tid + kThreads * u;
        const int s = ci / NCH, c = ci % NCH;
        const bool ok = ci < kN * NCH && s < n && 8 * c < Dk;
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
          // 4-element blocks 2c, 2c + 1 stay adjacent under the swizzle
          const int o = s * KFS + 4 * ((2 * c) ^ tile_swz(s));
          *reinterpret_cast<uint4*>(fk + o) = xk;
          *reinterpret_cast<uint4*>(fq + o) = xq;
        }
      }
    }
    // acc[u] += A^T W over the chunk steps for the wave's Dk tiles,
    // W[s][t] = wget(s, t)
    auto wpass = [&](auto wget, const uint16_t* at, f4(&acc)[NT]) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < kN * kN / 4 / kThreads; ++x) {  // W[s..s+3][t] -> pieces of row t
        const int e = tid + kThreads * x;
        const int t = e & 63, s = 4 * (e >> 6);
        f4 wv;
#pragma unroll
        for (int y = 0; y < 4; ++y) wv[y] = wget(s + y, t);
        uint2 p0, p1, p2;
        split3_quad(wv, p0, p1, p2);
        const int o = t * WS + s;
        *reinterpret_cast<uint2*>(wp + o) = p0;
        *reinterpret_cast<uint2*>(wp + kN * WS + o) = p1;
        *reinterpret_cast<uint2*>(wp + 2 * kN * WS + o) = p2;
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 bw[3];
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
          bw[pc] = *reinterpret_cast<const uint4*>(wp + pc * kN * WS + (tw + lr) * WS + 32 * ks +
                                                   8 * lq);
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          const uint4 af = tile_operand<KFS>(at, 32 * ks, 16 * jtile(u), lr, lq);
#pragma unroll
          for (int pc = 0; pc < 3; ++pc) acc[u] = mfma_bf16(af, bw[pc], acc[u]);
        }
      }
      __syncthreads();  // the pieces are rewritten by the next pass
    };
    wpass(wq_at, fk, dQ);
    wpass(w1_at, fq, dK);
    wpass(w2_at, fk, dK);  // -W2
  }
  {
    // columns 16 J + 4 lq .. +3 of step t: one 4-element store each (bf16,
    // or the head's fp32 terms)
    const int t = tw + lr;
    const int64_t nqk = (int64_t)a.B * T * Hk * Dk;
    float* const pq = split ? a.part + (int64_t)grp * nqk : nullptr;
    float* const pk = split ? a.part + (int64_t)(ng + grp) * nqk : nullptr;
    if (t < n) {
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int j = 16 * jtile(u) + 4 * lq;
        if (j < Dk) {
          const int64_t o = qk_index(t, j);
          if (split) {
            *reinterpret_cast<f4*>(pq + o) = dQ[u];
            *reinterpret_cast<f4*>(pk + o) = dK[u];
          } else {
            *reinterpret_cast<uint2*>(static_cast<bf16*>(a.dq) + o) =
                uint2{cvt_pk_bf16(dQ[u][0], dQ[u][1]), cvt_pk_bf16(dQ[u][2], dQ[u][3])};
            *reinterpret_cast<uint2*>(static_cast<bf16*>(a.dk) + o) =
                uint2{cvt_pk_bf16(dK[u][0], dK[u][1]), cvt_pk_bf16(dK[u][2], dK[u][3])};
          }
        }
      }
    }
  }
}

// dq, dk = the sum of the ng head groups' terms (a.part), in ascending group
// order, to bf16: thread i takes four consecutive elements of dq (i < n4) or
// of dk.
__global__ __launch_bounds__(256) void head_sum_kernel(const float* __restrict__ part, int ng,
                                                       int64_t n4, bf16* __restrict__ dq,
                                                       bf16* __restrict__ dk) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * n4) return;
  const bool second = i >= n4;
  const int64_t e = 4 * (second ? i - n4 : i);
  const float* __restrict__ p = part + (second ? (int64_t)ng * 4 * n4 : 0) + e;
  f4 acc = *reinterpret_cast<const f4*>(p);
  for (int r = 1; r < ng; ++r) acc += *reinterpret_cast<const f4*>(p + (int64_t)r * 4 * n4);
  *reinterpret_cast<uint2*>((second ? dk : dq) + e) =
      uint2{cvt_pk_bf16(acc[0], acc[1]), cvt_pk_bf16(acc[2], acc[3])};
}

template <int JT>
hipError_t launch_jt(const ChunkArgs& a, hipStream_t s) {
  const size_t lds = sizeof(float) * BL<JT>::SIZE;
  auto kern = chunk_bf16_kernel<JT>;
  // Opt in to more than 64 KiB of dynamic LDS; a failure here surfaces as a
  // launch error below.
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  const int ng = a.part != nullptr ? a.Hv / a.Hk / a.hpw : 1;  // head groups per kv head
  hipLaunchKernelGGL(kern, dim3(a.nch, a.Hk * ng, a.B), dim3(kThreads), lds, s, a);
  hipError_t e = hipGetLastError();
  note_launch(s);
  if (e != hipSuccess || a.part == nullptr) return e;
  const int64_t n4 = (int64_t)a.B * a.T * a.Hk * a.Dk / 4;  // Dk is a multiple of 8
  const int64_t blocks = (2 * n4 + 255) / 256;
  hipLaunchKernelGGL(head_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.part, ng, n4,
                     static_cast<bf16*>(a.dq), static_cast<bf16*>(a.dk));
  e = hipGetLastError();
  note_launch(s);
  return e;
}

}  // namespace

bool chunk_bf16_ok(const ChunkArgs& a) {
  return a.Dk % 8 == 0 && a.Dv % 8 == 0 && a.Dk > 48 && a.Dk <= 256 && a.L >= 1 && a.L <= kN;
}

// When the (chunk, kv head, batch row) grid has fewer than 256 workgroups
// (one round of a 256-CU device) and 2 to 16 value heads share a kv head,
// the value heads of a kv head go to ng groups, ng the smallest divisor of
// their count that gives at least 256 workgroups (or all of them): each
// workgroup forms fewer heads, and the per-workgroup set-up (QK, KK, the final
// products) repeats as little as it can.
int chunk_head_split(int64_t B, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv, int64_t L,
                     int64_t nch, bool bf16) {
  const int64_t rep = Hv / Hk, wg = nch * Hk * B;
  if (!(bf16 && Dk % 8 == 0 && Dv % 8 == 0 && Dk > 48 && Dk <= 256 && L >= 1 && L <= kN &&
        rep >= 2 && rep <= 16 && wg < 256))
    return 0;
  int64_t ng = 2;
  while (ng < rep && (rep % ng != 0 || wg * ng < 256)) ++ng;
  return static_cast<int>(rep / ng);
}

hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t s) {
  if (!chunk_bf16_ok(a)) return hipErrorInvalidValue;
  const int jt = (a.Dk + 15) / 16;
  if (jt <= 4) return launch_jt<4>(a, s);
  if (jt <= 8) return launch_jt<8>(a, s);
  if (jt <= 12) return launch_jt<12>(a, s);
  return launch_jt<16>(a, s);
}

}  // namespace gdr
