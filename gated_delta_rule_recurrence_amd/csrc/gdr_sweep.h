// Sequential sweeps of the gated delta rule on gfx950.
//
// Forward sweep: the state recurrence of mlx issue #4614 (recurrence statement
// under the accuracy table):  S <- g S;  S <- S + outer(beta (v - S k), k);
// y = S q.  It writes y, the final state, a state checkpoint every L steps and
// the per-step residual e_t = v_t - g_t S_{t-1} k_t (forward-with-save, mlx-lm
// PR #1217, "What this PR adds").
//
// Reverse sweep: the state-gradient recurrence of the VJP, swept backwards in
// time.  With H = dL/dS after step t (dS_T at t = T):
//     G = H + outer(dy_t, q_t);   c_t = G k_t = H k_t + dy_t (q_t . k_t);
//     dv_t = beta_t c_t;          H <- g_t (G - outer(dv_t, k_t))
// It writes dv, c_t, dS0 and H at every chunk boundary.
//
// Mapping.  A workgroup of 256 threads owns 16 R consecutive rows of the
// [Dv x Dk] state of one (batch row, value head): 16 row groups of R rows, one
// row group per 16-lane DPP row.  Lane p of a row group holds the columns
// {4p + 64m + x : m < NC/4, x < 4} of its R rows in VGPRs for the whole sweep,
// so each row's Dk-reduction is a 4-stage DPP butterfly inside the DPP row and
// the state never leaves the chip between checkpoints.  Rows are independent
// in both recurrences (they couple only through the outputs), which is what
// lets a head be split over several workgroups.  k, q, v / dy, g and beta are
// staged into LDS 16 steps at a time with 16-byte loads, double-buffered: the
// next block is fetched into registers while the current one is consumed.
// Inside a block the step loop is unrolled by two over two operand register
// sets, so the LDS operands of step t+1 are read while step t computes.
//
// Decay is applied lazily: the state is kept as S = sigma * St with a scalar
// sigma shared by the workgroup (every row of one head sees the same g_t).
// A step multiplies sigma by g_t and adds (d / sigma) k^T to St, one FMA per
// element instead of a multiply and an FMA.  When sigma falls below 2^-60 it
// is folded back into St (St *= sigma, sigma = 1), so sigma never underflows,
// 1/sigma <= 2^60, and the decay never has to be divided out: sigma is only a
// running product of g.  Contribution s reaches step t through the same t - s
// roundings as in the direct form.  The reverse sweep keeps H = tau * Ht the
// same way.
#pragma once

#include <type_traits>

#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {
namespace sweep {

constexpr int kThreads = 256;
constexpr int kStage = 16;            // time steps per LDS block
constexpr float kRescale = 0x1p-60f;  // fold the lazy decay below this

template <int NC, int R>
struct SweepLayout {
  static constexpr int RW = 16 * R;    // rows per workgroup
  static constexpr int DKP = 16 * NC;  // padded Dk covered by a row group
  static constexpr int K_OFF = 0;
  static constexpr int Q_OFF = kStage * DKP;
  static constexpr int X_OFF = 2 * kStage * DKP;  // v (forward) or dy (reverse)
  static constexpr int G_OFF = X_OFF + kStage * RW;
  static constexpr int B_OFF = G_OFF + kStage;
  static constexpr int QK_OFF = B_OFF + kStage;   // q_t . k_t (reverse sweep)
  static constexpr int BUF = QK_OFF + kStage;     // one LDS buffer, floats
};

// 16-byte vector of raw input elements.
struct alignas(16) Raw16 {
  uint32_t w[4];
};

template <typename TIn>
__device__ __forceinline__ void unpack(const Raw16& r, float* out);

template <>
__device__ __forceinline__ void unpack<float>(const Raw16& r, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(r.w[i]);
}

template <>
__device__ __forceinline__ void unpack<bf16>(const Raw16& r, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(r.w[i] << 16);
    out[2 * i + 1] = __uint_as_float(r.w[i] & 0xffff0000u);
  }
}

// Global -> register -> LDS staging of one block of kStage steps.
// VEC: k/q rows and v/dy rows are read as 16-byte vectors (needs Dk and Dv to
// be multiples of the vector width; the base pointers are 16-byte aligned by
// the ABI).  Otherwise element by element.  Loads are unconditional and
// branch-free (an out-of-range slot reads offset 0 of the same tensor and is
// zeroed on the way into LDS), so no load has to complete before the block in
// flight is consumed.
template <typename TIn, int NC, int R, bool VEC>
struct Stager {
  using Lo = SweepLayout<NC, R>;
  static constexpr int VW = VEC ? 16 / (int)sizeof(TIn) : 1;  // elements/slot
  static constexpr int NKV = kStage * Lo::DKP / VW;  // slots in a k block
  static constexpr int NXV = kStage * Lo::RW / VW;   // slots in an x block
  static constexpr int SK = (NKV + kThreads - 1) / kThreads;
  static constexpr int SX = (NXV + kThreads - 1) / kThreads;
  static_assert(Lo::DKP % VW == 0 && Lo::RW % VW == 0, "vector width");
  static_assert(2 * SK + SX + 1 <= 64, "ok mask bits");
  using Slot = typename std::conditional<VEC, Raw16, TIn>::type;

  Slot kr[SK], qr[SK], xr[SX];
  TIn gb;  // g (threads 0..15) or beta (threads 16..31) of one step
  uint8_t mk;  // mask byte of the step (0: an identity step)
  bool log_g = false;  // g holds log of the decay
  const uint8_t* mask = nullptr;
  uint64_t ok;
  bool full;  // every slot of the block is in range (no zero fill needed)

  __device__ __forceinline__ void fetch(int blk, int T, int Hk, int Hv,
                                        int Dk, int Dv, int b, int h, int hk,
                                        int rowbase, const TIn* __restrict__ k,
                                        const TIn* __restrict__ q,
                                        const TIn* __restrict__ x,
                                        const TIn* __restrict__ g,
                                        const TIn* __restrict__ beta) {
    const int tid = threadIdx.x;
    const int t0 = blk * kStage;
    uint64_t m = 0;
#pragma unroll
    for (int u = 0; u < SK; ++u) {
      const int vi = tid + kThreads * u;
      const int s = vi / (Lo::DKP / VW);
      const int c = (vi - s * (Lo::DKP / VW)) * VW;
      const bool good = vi < NKV && t0 + s < T && c < Dk;
      const int64_t off =
          good ? (((int64_t)b * T + t0 + s) * Hk + hk) * Dk + c : 0;
      kr[u] = *reinterpret_cast<const Slot*>(k + off);
      qr[u] = *reinterpret_cast<const Slot*>(q + off);
      m |= (uint64_t)good << u;
    }
#pragma unroll
    for (int u = 0; u < SX; ++u) {
      const int vi = tid + kThreads * u;
      const int s = vi / (Lo::RW / VW);
      const int r = (vi - s * (Lo::RW / VW)) * VW;
      const bool good = vi < NXV && t0 + s < T && rowbase + r < Dv;
      const int64_t off =
          good ? (((int64_t)b * T + t0 + s) * Hv + h) * Dv + rowbase + r : 0;
      xr[u] = *reinterpret_cast<const Slot*>(x + off);
      m |= (uint64_t)good << (SK + u);
    }
    {
      const int s = tid & 15;
      const bool good = tid < 32 && t0 + s < T;
      const int64_t off = good ? ((int64_t)b * T + t0 + s) * Hv + h : 0;
      gb = (tid < 16 ? g : beta)[off];
      mk = *mask_byte(mask, b, T, t0 + s, good);
      m |= (uint64_t)good << (SK + SX);
    }
    ok = m;
    full = t0 + kStage <= T && Dk == Lo::DKP && rowbase + Lo::RW <= Dv;
  }

  __device__ __forceinline__ void store(float* __restrict__ buf) const {
    if (full)
      store_impl<false>(buf);
    else
      store_impl<true>(buf);
  }

 private:
  template <bool CHECK>
  __device__ __forceinline__ void store_impl(float* __restrict__ buf) const {
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < SK; ++u) {
      const int vi = tid + kThreads * u;
      if (vi < NKV) {
        const bool good = !CHECK || ((ok >> u) & 1);
        const int s = vi / (Lo::DKP / VW);
        const int c = (vi - s * (Lo::DKP / VW)) * VW;
        write(buf + Lo::K_OFF + s * Lo::DKP + c, kr[u], good);
        write(buf + Lo::Q_OFF + s * Lo::DKP + c, qr[u], good);
      }
    }
#pragma unroll
    for (int u = 0; u < SX; ++u) {
      const int vi = tid + kThreads * u;
      if (vi < NXV) {
        const bool good = !CHECK || ((ok >> (SK + u)) & 1);
        const int s = vi / (Lo::RW / VW);
        const int r = (vi - s * (Lo::RW / VW)) * VW;
        write(buf + Lo::X_OFF + s * Lo::RW + r, xr[u], good);
      }
    }
    if (tid < 32) {
      const bool good = !CHECK || ((ok >> (SK + SX)) & 1);
      // an identity step: g = 1, beta = 0
      const float val = mk == 0 ? (tid < 16 ? 1.f : 0.f) : decay_of(to_f32(gb), tid < 16 && log_g);
      buf[(tid < 16 ? Lo::G_OFF : Lo::B_OFF) + (tid & 15)] = good ? val : 0.f;
    }
  }

  __device__ __forceinline__ static void write(float* dst, const Raw16& r,
                                               bool good) {
    float v[VW];
    unpack<TIn>(r, v);
#pragma unroll
    for (int i = 0; i < VW; i += 4) {
      float4 f;
      f.x = good ? v[i] : 0.f;
      f.y = good ? v[i + 1] : 0.f;
      f.z = good ? v[i + 2] : 0.f;
      f.w = good ? v[i + 3] : 0.f;
      *reinterpret_cast<float4*>(dst + i) = f;
    }
  }
  __device__ __forceinline__ static void write(float* dst, const TIn& r,
                                               bool good) {
    *dst = good ? to_f32(r) : 0.f;
  }
};

// Select element `i` of a small register array without dynamic indexing.
template <int N>
__device__ __forceinline__ float pick(const float (&a)[N], int i) {
  float r = a[0];
#pragma unroll
  for (int j = 1; j < N; ++j)
    if (i == j) r = a[j];
  return r;
}

// Store v[0..R) to the R consecutive elements o .. o+R-1 of p (R consecutive
// state rows of one step of a [.., Dv] tensor).  One vector store when all R
// rows exist and the address is R-element aligned, else element by element.
template <typename T, int R>
__device__ __forceinline__ void st_rows(T* __restrict__ p, int64_t o,
                                        const float (&v)[R], int nvalid,
                                        bool aligned) {
  if (nvalid >= R && aligned) {
    if constexpr (std::is_same<T, float>::value) {
      if constexpr (R == 1) {
        p[o] = v[0];
      } else if constexpr (R == 2) {
        *reinterpret_cast<float2*>(p + o) = make_float2(v[0], v[1]);
      } else {
        static_assert(R == 4, "rows per lane");
        *reinterpret_cast<float4*>(p + o) = make_float4(v[0], v[1], v[2], v[3]);
      }
    } else {
      uint32_t w[R];
#pragma unroll
      for (int r = 0; r < R; ++r) w[r] = from_f32<T>(v[r]).bits;
      if constexpr (R == 1) {
        p[o] = from_f32<T>(v[0]);
      } else if constexpr (R == 2) {
        *reinterpret_cast<uint32_t*>(p + o) = w[0] | (w[1] << 16);
      } else {
        static_assert(R == 4, "rows per lane");
        *reinterpret_cast<uint2*>(p + o) =
            make_uint2(w[0] | (w[1] << 16), w[2] | (w[3] << 16));
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < nvalid) st(p, o + r, v[r]);
  }
}

// Load this lane's part of rows [row0, row0+R) of a [Dv][Dk] matrix.
template <int NC, int R>
__device__ __forceinline__ void tile_load(float (&S)[R][NC],
                                          const float* __restrict__ M, int row0,
                                          int p, int Dk, int Dv) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = 4 * p + 64 * (c / 4) + (c % 4);
      const int row = row0 + r;
      S[r][c] = (M != nullptr && row < Dv && col < Dk)
                    ? M[(int64_t)row * Dk + col]
                    : 0.f;
    }
}

// Store scale * (this lane's part of rows [row0, row0+R)).
template <int NC, int R>
__device__ __forceinline__ void tile_store(const float (&S)[R][NC], float scale,
                                           float* __restrict__ M, int row0,
                                           int p, int Dk, int Dv) {
  float v[R][NC];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) v[r][c] = scale * S[r][c];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
    if (row >= Dv) continue;
#pragma unroll
    for (int m = 0; m < NC / 4; ++m) {
      const int col = 4 * p + 64 * m;
      float* dst = M + (int64_t)row * Dk + col;
      if (col + 3 < Dk && (Dk & 3) == 0) {
        *reinterpret_cast<float4*>(dst) =
            make_float4(v[r][4 * m], v[r][4 * m + 1], v[r][4 * m + 2],
                        v[r][4 * m + 3]);
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (col + x < Dk) dst[x] = v[r][4 * m + x];
      }
    }
  }
}

template <int NC>
__device__ __forceinline__ void lds_cols(float (&out)[NC],
                                         const float* __restrict__ src, int p) {
#pragma unroll
  for (int m = 0; m < NC / 4; ++m) {
    const float4 v4 = *reinterpret_cast<const float4*>(src + 4 * p + 64 * m);
    out[4 * m + 0] = v4.x;
    out[4 * m + 1] = v4.y;
    out[4 * m + 2] = v4.z;
    out[4 * m + 3] = v4.w;
  }
}

// Operands of one time step, read from an LDS block.
template <int NC, int R>
struct StepOps {
  float k[NC], q[NC], x[R], g, beta, qk;
};

template <int NC, int R, bool WITH_QK>
__device__ __forceinline__ void load_ops(StepOps<NC, R>& o,
                                         const float* __restrict__ buf, int s,
                                         int p, int rg) {
  using Lo = SweepLayout<NC, R>;
  lds_cols<NC>(o.k, buf + Lo::K_OFF + s * Lo::DKP, p);
  lds_cols<NC>(o.q, buf + Lo::Q_OFF + s * Lo::DKP, p);
#pragma unroll
  for (int r = 0; r < R; ++r) o.x[r] = buf[Lo::X_OFF + s * Lo::RW + rg * R + r];
  o.g = buf[Lo::G_OFF + s];
  o.beta = buf[Lo::B_OFF + s];
  o.qk = WITH_QK ? buf[Lo::QK_OFF + s] : 0.f;
}

// FAST: L is a multiple of kStage (checkpoints fall on block starts) and the
// vectorised staging applies.
template <typename TIn, int NC, int R, bool FAST>
__global__ __launch_bounds__(kThreads) void fwd_sweep_kernel(FwdSweepArgs a) {
  using Lo = SweepLayout<NC, R>;
  using St_ = Stager<TIn, NC, R, FAST>;
  __shared__ __align__(16) float lds[2][Lo::BUF];
  // Fully unrolled 16-step blocks where the registers allow it (R <= 2 keeps
  // two waves per SIMD; at R = 4 the unrolled block would drop to one).
  constexpr bool kUnroll = FAST && R <= 2;

  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ v = static_cast<const TIn*>(a.v);
  const TIn* __restrict__ g = static_cast<const TIn*>(a.g);
  const TIn* __restrict__ beta = static_cast<const TIn*>(a.beta);
  TIn* __restrict__ y = static_cast<TIn*>(a.y);

  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const int tid = threadIdx.x;
  const int p = tid & 15;   // column part inside the DPP row
  const int rg = tid >> 4;  // row group 0..15
  const int h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (Hv / Hk);
  const int rowbase = blockIdx.x * Lo::RW;
  const int row0 = rowbase + rg * R;
  const int64_t bh = (int64_t)b * Hv + h;
  const int64_t mat = (int64_t)Dv * Dk;

  // S = sig * St
  float St[R][NC];
  float sig = 1.f;
  tile_load<NC, R>(St, a.S0 ? a.S0 + bh * a.s0_stride * mat : nullptr, row0, p, Dk, Dv);

  const int nblk = (T + kStage - 1) / kStage;
  St_ stg;
  stg.log_g = a.log_g;
  stg.mask = a.mask;
  if (nblk > 0) {
    stg.fetch(0, T, Hk, Hv, Dk, Dv, b, h, hk, rowbase, k, q, v, g, beta);
    stg.store(lds[0]);
  }
  __syncthreads();

  const int my_row = row0 + p;  // row written by lanes p < R
  const bool writer = (p < R) && (my_row < Dv);
  const int64_t out0 = ((int64_t)b * T * Hv + h) * Dv + my_row;  // (b,0,h,row)
  const int64_t rows0 = ((int64_t)b * T * Hv + h) * Dv + row0;   // (b,0,h,row0)
  const int64_t tstep = (int64_t)Hv * Dv;
  const int nrow = Dv - row0;  // rows of this row group that exist (if < R)
  const bool rows_aligned = (Dv % R) == 0;
  float* __restrict__ E = a.E;
  float* __restrict__ Sck = a.Sck;
  int to_ckpt = 0;  // generic path: steps until the next checkpoint
  int ckpt_slot = 0;

  // Per-step outputs are captured, not stored: after the dots of block step
  // s, lane p == s keeps y_{tbase+s-1} and e_{tbase+s} of its R rows (every
  // lane of a DPP row holds the same sums), and the block's outputs leave in
  // one store per lane at the end of the block.
  float ycap[R], ecap[R];
#pragma unroll
  for (int r = 0; r < R; ++r) ycap[r] = ecap[r] = 0.f;

  // One forward step (block step s) with operands `cur`; `oth` holds the
  // operands of the previous step (its q is q_{t-1}, for the read-out
  // y_{t-1}) and, once the dots have consumed it, is refilled with the
  // operands of block step s_next.
  auto step = [&](const StepOps<NC, R>& cur, StepOps<NC, R>& oth,
                  const float* __restrict__ buf, int s, int s_next)
                  __attribute__((always_inline)) {
    if (!FAST) {
      if (to_ckpt == 0) {
        if (Sck != nullptr)
          tile_store<NC, R>(St, sig, Sck + (bh * a.nch + ckpt_slot) * mat,
                            row0, p, Dk, Dv);
        ++ckpt_slot;
        to_ckpt = a.L;
      }
      --to_ckpt;
    }
    // dots on the state before step t: St k_t (for the update) and
    // St q_{t-1} (the read-out y_{t-1} of the previous step)
    float pk[R], pq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float ak = St[r][0] * cur.k[0], aq = St[r][0] * oth.q[0];
#pragma unroll
      for (int c = 1; c < NC; ++c) {
        ak = fmaf(St[r][c], cur.k[c], ak);
        aq = fmaf(St[r][c], oth.q[c], aq);
      }
      pk[r] = ak;
      pq[r] = aq;
    }
    load_ops<NC, R, false>(oth, buf, s_next, p, rg);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      pk[r] = rowsum16(pk[r]);
      pq[r] = rowsum16(pq[r]);
    }
    // u_t = (g_t S) k_t,  e_t = v_t - u_t,  d_t = beta_t e_t
    const float gs = cur.g * sig;
    float d[R], e[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      e[r] = cur.x[r] - gs * pk[r];
      d[r] = cur.beta * e[r];
    }
    const bool mine = p == s;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      ycap[r] = mine ? sig * pq[r] : ycap[r];
      ecap[r] = mine ? e[r] : ecap[r];
    }
    // S_t = g_t S + d k^T  ==  sig' (St + (d / sig') k^T) with sig' = g_t sig
    const bool fold = gs < kRescale;
    const float sig_new = fold ? 1.f : gs;
    const float inv = __builtin_amdgcn_rcpf(sig_new);
    if (fold) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) St[r][c] *= gs;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float coef = d[r] * inv;
#pragma unroll
      for (int c = 0; c < NC; ++c) St[r][c] = fmaf(coef, cur.k[c], St[r][c]);
    }
    sig = sig_new;
  };

  // A and B alternate as the operand sets of consecutive steps.  The refill
  // index is clamped to the block's last step, so after a block both sets, and
  // in particular B, hold that step's q: q_{t-1} for the next block's first
  // step and for the final read-out.  B.q is zero before the first step.
  StepOps<NC, R> A, B;
#pragma unroll
  for (int c = 0; c < NC; ++c) B.q[c] = 0.f;
  // One staged block.  FULL blocks (16 steps, unrolled) and the others
  // (a short last block, or every block when unrolling is off) are separate
  // instantiations, so the main loop carries no code for the short case.
  auto run_block = [&](int blk, auto full) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full)::value;
    const float* __restrict__ cur = lds[blk & 1];
    if (blk + 1 < nblk)
      stg.fetch(blk + 1, T, Hk, Hv, Dk, Dv, b, h, hk, rowbase, k, q, v, g,
                beta);
    const int tbase = blk * kStage;
    const int nsteps = FULL ? kStage : min(kStage, T - tbase);
    if (FAST && Sck != nullptr && (tbase % a.L) == 0)
      tile_store<NC, R>(St, sig, Sck + (bh * a.nch + tbase / a.L) * mat, row0,
                        p, Dk, Dv);
    load_ops<NC, R, false>(A, cur, 0, p, rg);
    if constexpr (FULL) {
      // every LDS offset is a compile-time constant
#pragma unroll
      for (int s = 0; s < kStage; s += 2) {
        step(A, B, cur, s, s + 1);
        step(B, A, cur, s + 1, s + 2 < kStage ? s + 2 : kStage - 1);
      }
    } else {
      const int slast = nsteps - 1;
      int s = 0;
      for (; s + 1 < nsteps; s += 2) {
        step(A, B, cur, s, s + 1);
        step(B, A, cur, s + 1, min(s + 2, slast));
      }
      if (s < nsteps) step(A, B, cur, s, slast);
    }
    if (p < nsteps) {
      const int64_t o = rows0 + (int64_t)(tbase + p) * tstep;
      if (E != nullptr) st_rows<float, R>(E, o, ecap, nrow, rows_aligned);
      if (y != nullptr && tbase + p > 0) st_rows<TIn, R>(y, o - tstep, ycap, nrow, rows_aligned);
    }
    if (blk + 1 < nblk) stg.store(lds[(blk + 1) & 1]);
    __syncthreads();
  };
  const int nfull = kUnroll ? T / kStage : 0;
  int blk = 0;
  for (; blk < nfull; ++blk) run_block(blk, std::true_type{});
  for (; blk < nblk; ++blk) run_block(blk, std::false_type{});

  if (T > 0) {
    const float* qlast = B.q;
    float pq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float aq = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) aq = fmaf(St[r][c], qlast[c], aq);
      pq[r] = rowsum16(aq);
    }
    if (writer && y != nullptr) st(y, out0 + (int64_t)(T - 1) * tstep, sig * pick<R>(pq, p));
  }
  if (a.ST != nullptr)
    tile_store<NC, R>(St, sig, a.ST + bh * mat, row0, p, Dk, Dv);
}

template <typename TIn, int NC, int R, bool FAST>
__global__ __launch_bounds__(kThreads) void bwd_sweep_kernel(BwdSweepArgs a) {
  using Lo = SweepLayout<NC, R>;
  using St_ = Stager<TIn, NC, R, FAST>;
  __shared__ __align__(16) float lds[2][Lo::BUF];
  // Fully unrolled 16-step blocks where the registers allow it (R <= 2 keeps
  // two waves per SIMD; at R = 4 the unrolled block would drop to one).
  constexpr bool kUnroll = FAST && R <= 2;

  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ g = static_cast<const TIn*>(a.g);
  const TIn* __restrict__ beta = static_cast<const TIn*>(a.beta);
  const TIn* __restrict__ dy = static_cast<const TIn*>(a.dy);
  TIn* __restrict__ dv = static_cast<TIn*>(a.dv);

  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const int tid = threadIdx.x;
  const int p = tid & 15;
  const int rg = tid >> 4;
  const int h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (Hv / Hk);
  const int rowbase = blockIdx.x * Lo::RW;
  const int row0 = rowbase + rg * R;
  const int64_t bh = (int64_t)b * Hv + h;
  const int64_t mat = (int64_t)Dv * Dk;

  // H (dL/dS after the step being processed) = tau * Ht
  float Ht[R][NC];
  float tau = 1.f;
  tile_load<NC, R>(Ht, a.dST ? a.dST + bh * mat : nullptr, row0, p, Dk, Dv);
  // slot nch-1 holds dL/dS_T for the last chunk
  if (a.nch > 0)
    tile_store<NC, R>(Ht, 1.f, a.Hck + (bh * a.nch + a.nch - 1) * mat, row0,
                      p, Dk, Dv);

  const int nblk = (T + kStage - 1) / kStage;
  St_ stg;
  stg.log_g = a.log_g;
  stg.mask = a.mask;
  if (nblk > 0) {
    stg.fetch(nblk - 1, T, Hk, Hv, Dk, Dv, b, h, hk, rowbase, k, q, dy, g,
              beta);
    stg.store(lds[(nblk - 1) & 1]);
  }
  __syncthreads();

  const int64_t rows0 = ((int64_t)b * T * Hv + h) * Dv + row0;  // (b,0,h,row0)
  const int64_t tstep = (int64_t)Hv * Dv;
  const int nrow = Dv - row0;
  const bool rows_aligned = (Dv % R) == 0;
  float* __restrict__ C = a.C;
  float* __restrict__ Hck = a.Hck;

  // generic path: H after step t is saved when t % L == 0 and t > 0, in slot
  // t / L - 1
  int last_chunk = (T - 1) / (a.L > 0 ? a.L : 1);
  int to_ckpt = T - 1 - last_chunk * a.L;  // steps until t % L == 0

  // c_t and dv_t of block step s are captured by lane p == s and stored at
  // the end of the block (as in the forward sweep).
  float ccap[R], dvcap[R];
#pragma unroll
  for (int r = 0; r < R; ++r) ccap[r] = dvcap[r] = 0.f;

  auto step = [&](const StepOps<NC, R>& op, StepOps<NC, R>& oth,
                  const float* __restrict__ buf, int t, int s, int s_next)
                  __attribute__((always_inline)) {
    load_ops<NC, R, true>(oth, buf, s_next, p, rg);
    // c_t = G k_t = tau (Ht k_t) + dy_t (q_t . k_t)
    float c[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float a0 = Ht[r][0] * op.k[0];
#pragma unroll
      for (int j = 1; j < NC; ++j) a0 = fmaf(Ht[r][j], op.k[j], a0);
      c[r] = fmaf(tau, rowsum16(a0), op.x[r] * op.qk);
    }
    float dvr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) dvr[r] = op.beta * c[r];
    const bool mine = p == s;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      ccap[r] = mine ? c[r] : ccap[r];
      dvcap[r] = mine ? dvr[r] : dvcap[r];
    }
    // H_t = g_t (tau Ht + dy q^T - dv k^T) = tau' (Ht + (dy q^T - dv k^T)/tau)
    const float inv = __builtin_amdgcn_rcpf(tau);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float cy = op.x[r] * inv, cv = -dvr[r] * inv;
#pragma unroll
      for (int j = 0; j < NC; ++j)
        Ht[r][j] = fmaf(cv, op.k[j], fmaf(cy, op.q[j], Ht[r][j]));
    }
    const float gt = op.g * tau;
    const bool fold = gt < kRescale;
    if (fold) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NC; ++j) Ht[r][j] *= gt;
    }
    tau = fold ? 1.f : gt;
    if (!FAST) {
      if (to_ckpt == 0) {
        if (t > 0)
          tile_store<NC, R>(Ht, tau, Hck + (bh * a.nch + last_chunk - 1) * mat,
                            row0, p, Dk, Dv);
        --last_chunk;
        to_ckpt = a.L;
      }
      --to_ckpt;
    }
  };

  // Blocks run last to first; only the last block of the sequence can be
  // short, and it is the first one processed.
  auto run_block = [&](int blk, auto full) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full)::value;
    float* __restrict__ cur = lds[blk & 1];
    // q_t . k_t of this block: row group rg handles step rg
    {
      float kq[NC], qv[NC];
      lds_cols<NC>(kq, cur + Lo::K_OFF + rg * Lo::DKP, p);
      lds_cols<NC>(qv, cur + Lo::Q_OFF + rg * Lo::DKP, p);
      float z = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) z = fmaf(kq[c], qv[c], z);
      z = rowsum16(z);
      if (p == 0) cur[Lo::QK_OFF + rg] = z;
    }
    __syncthreads();
    if (blk > 0)
      stg.fetch(blk - 1, T, Hk, Hv, Dk, Dv, b, h, hk, rowbase, k, q, dy, g,
                beta);
    const int tbase = blk * kStage;
    const int nsteps = FULL ? kStage : min(kStage, T - tbase);
    StepOps<NC, R> A, B;
    load_ops<NC, R, true>(A, cur, nsteps - 1, p, rg);
    if constexpr (FULL) {
#pragma unroll
      for (int s = kStage - 1; s >= 1; s -= 2) {
        step(A, B, cur, tbase + s, s, s - 1);
        step(B, A, cur, tbase + s - 1, s - 1, s - 2 > 0 ? s - 2 : 0);
      }
    } else {
      int s = nsteps - 1;
      for (; s >= 1; s -= 2) {
        step(A, B, cur, tbase + s, s, s - 1);
        step(B, A, cur, tbase + s - 1, s - 1, max(s - 2, 0));
      }
      if (s == 0) step(A, B, cur, tbase, 0, 0);
    }
    if (p < nsteps) {
      const int64_t o = rows0 + (int64_t)(tbase + p) * tstep;
      st_rows<float, R>(C, o, ccap, nrow, rows_aligned);
      st_rows<TIn, R>(dv, o, dvcap, nrow, rows_aligned);
    }
    if (FAST && tbase > 0 && (tbase % a.L) == 0)
      tile_store<NC, R>(Ht, tau, Hck + (bh * a.nch + tbase / a.L - 1) * mat,
                        row0, p, Dk, Dv);
    if (blk > 0) stg.store(lds[(blk - 1) & 1]);
    __syncthreads();
  };
  int blk = nblk - 1;
  if (!kUnroll) {
    for (; blk >= 0; --blk) run_block(blk, std::false_type{});
  } else {
    if (blk >= 0 && T % kStage != 0) run_block(blk--, std::false_type{});
    for (; blk >= 0; --blk) run_block(blk, std::true_type{});
  }
  if (a.dS0 != nullptr)
    tile_store<NC, R>(Ht, tau, a.dS0 + bh * mat, row0, p, Dk, Dv);
}

template <typename TIn, int NC, int R, bool FAST>
hipError_t fwd_launch(const FwdSweepArgs& a, hipStream_t s) {
  using Lo = SweepLayout<NC, R>;
  dim3 grid((a.Dv + Lo::RW - 1) / Lo::RW, a.Hv, a.B);
  hipLaunchKernelGGL((fwd_sweep_kernel<TIn, NC, R, FAST>), grid,
                     dim3(kThreads), 0, s, a);
  const hipError_t e = hipGetLastError();
  note_launch(s);
  return e;
}

template <typename TIn, int NC, int R, bool FAST>
hipError_t bwd_launch(const BwdSweepArgs& a, hipStream_t s) {
  using Lo = SweepLayout<NC, R>;
  dim3 grid((a.Dv + Lo::RW - 1) / Lo::RW, a.Hv, a.B);
  hipLaunchKernelGGL((bwd_sweep_kernel<TIn, NC, R, FAST>), grid,
                     dim3(kThreads), 0, s, a);
  const hipError_t e = hipGetLastError();
  note_launch(s);
  return e;
}

// Columns per lane: the smallest multiple of 4 with 16 * NC >= Dk.
inline int pick_nc(int Dk) { return 4 * ((Dk + 63) / 64); }

// The vectorised, block-aligned-checkpoint kernels need 16-byte rows of k, q
// and v / dy, and L a multiple of the staging block.
template <typename TIn>
bool fast_ok(int Dk, int Dv, int L) {
  const int vw = 16 / (int)sizeof(TIn);
  return Dk % vw == 0 && Dv % vw == 0 && L % kStage == 0;
}

// Rows per lane R: one workgroup owns 16 R rows of a head, one wave per
// SIMD per workgroup.  Pick the largest R that still gives two workgroups
// per CU (so two waves share each SIMD and hide each other's dependency
// stalls, with every workgroup resident in one round); fall back to R = 1.
inline int pick_r(int B, int Hv, int Dv, int num_cu) {
  for (int R = 4; R >= 2; R /= 2) {
    const long wgs = (long)B * Hv * ((Dv + 16 * R - 1) / (16 * R));
    if (wgs >= 2L * num_cu) return R;
  }
  return 1;
}

template <typename TIn, bool FAST, int R>
hipError_t fwd_dispatch_nc(const FwdSweepArgs& a, hipStream_t s) {
  switch (pick_nc(a.Dk)) {
    case 4: return fwd_launch<TIn, 4, R, FAST>(a, s);
    case 8: return fwd_launch<TIn, 8, R, FAST>(a, s);
    case 12: return fwd_launch<TIn, 12, R, FAST>(a, s);
    case 16: return fwd_launch<TIn, 16, R, FAST>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, bool FAST, int R>
hipError_t bwd_dispatch_nc(const BwdSweepArgs& a, hipStream_t s) {
  switch (pick_nc(a.Dk)) {
    case 4: return bwd_launch<TIn, 4, R, FAST>(a, s);
    case 8: return bwd_launch<TIn, 8, R, FAST>(a, s);
    case 12: return bwd_launch<TIn, 12, R, FAST>(a, s);
    case 16: return bwd_launch<TIn, 16, R, FAST>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t fwd_dispatch(const FwdSweepArgs& a, int num_cu, hipStream_t s) {
  if (!fast_ok<TIn>(a.Dk, a.Dv, a.L)) return fwd_dispatch_nc<TIn, false, 1>(a, s);
  switch (pick_r(a.B, a.Hv, a.Dv, num_cu)) {
    case 4: return fwd_dispatch_nc<TIn, true, 4>(a, s);
    case 2: return fwd_dispatch_nc<TIn, true, 2>(a, s);
    default: return fwd_dispatch_nc<TIn, true, 1>(a, s);
  }
}

template <typename TIn>
hipError_t bwd_dispatch(const BwdSweepArgs& a, int num_cu, hipStream_t s) {
  if (!fast_ok<TIn>(a.Dk, a.Dv, a.L)) return bwd_dispatch_nc<TIn, false, 1>(a, s);
  switch (pick_r(a.B, a.Hv, a.Dv, num_cu)) {
    case 4: return bwd_dispatch_nc<TIn, true, 4>(a, s);
    case 2: return bwd_dispatch_nc<TIn, true, 2>(a, s);
    default: return bwd_dispatch_nc<TIn, true, 1>(a, s);
  }
}

}  // namespace sweep
}  // namespace gdr
