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
//     G = H + outer(dy_t, q_t);   c_t = G k_t;   dv_t = beta_t c_t;
//     H <- g_t (G - outer(dv_t, k_t))
// It writes dv, c_t, dS0 and H at every chunk boundary.  Only multiplications
// by g occur, never a division.
//
// Mapping.  A workgroup of 256 threads owns 16 R consecutive rows of the
// [Dv x Dk] state of one (batch row, value head): 16 row groups of R rows, one
// row group per 16-lane DPP row.  Lane p of a row group holds the columns
// {4p + 64m + x : m < NC/4, x < 4} of its R rows in VGPRs for the whole sweep,
// so each row's Dk-reduction is a 4-stage DPP butterfly inside the DPP row and
// the state never leaves the chip between checkpoints.  Rows are independent
// in both recurrences (they couple only through the outputs), which is what
// lets a head be split over several workgroups.  k, q, v / dy, g and beta are
// staged into LDS 16 steps at a time, double-buffered, the next block being
// fetched into registers while the current one is consumed.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;
constexpr int kStage = 16;  // time steps per LDS block

template <int NC, int R>
struct SweepLayout {
  static constexpr int RW = 16 * R;    // rows per workgroup
  static constexpr int DKP = 16 * NC;  // padded Dk covered by a row group
  static constexpr int K_OFF = 0;
  static constexpr int Q_OFF = kStage * DKP;
  static constexpr int X_OFF = 2 * kStage * DKP;  // v (forward) or dy (reverse)
  static constexpr int G_OFF = X_OFF + kStage * RW;
  static constexpr int B_OFF = G_OFF + kStage;
  static constexpr int SIZE = B_OFF + kStage;
  static constexpr int PF = (SIZE + kThreads - 1) / kThreads;
};

// Fetch one block of kStage steps (steps blk*kStage ...) into registers.
// x is the per-row tensor [B][T][Hv][Dv] (v or dy).  The loads are
// unconditional and branch-free: an element outside the tensor is read from
// offset 0 of the same tensor and masked to zero later, in stage_store, so
// no load has to complete before the current block is consumed.
template <typename TIn, int NC, int R, int N>
__device__ __forceinline__ void stage_fetch(
    TIn (&raw)[N], uint64_t& okmask, int blk, int T, int Hk, int Hv, int Dk,
    int Dv, int b, int h, int hk, int rowbase, const TIn* __restrict__ k,
    const TIn* __restrict__ q, const TIn* __restrict__ x,
    const TIn* __restrict__ g, const TIn* __restrict__ beta) {
  using Lo = SweepLayout<NC, R>;
  static_assert(N == Lo::PF && N <= 64, "prefetch register count");
  const int tid = threadIdx.x;
  const int64_t bt0 = (int64_t)b * T + (int64_t)blk * kStage;  // (b, first t)
  uint64_t mask = 0;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int idx = tid + kThreads * u;
    // decode the slot without branches
    const bool in_k = idx < Lo::Q_OFF;
    const bool in_q = !in_k && idx < Lo::X_OFF;
    const bool in_x = !in_k && !in_q && idx < Lo::G_OFF;
    const bool in_g = idx >= Lo::G_OFF && idx < Lo::B_OFF;
    const bool in_b = idx >= Lo::B_OFF && idx < Lo::SIZE;
    const int jk = in_k ? idx : idx - Lo::Q_OFF;  // offset inside the k or q block
    const int sk = jk / Lo::DKP, col = jk - sk * Lo::DKP;
    const int jx = idx - Lo::X_OFF;
    const int sx = jx / Lo::RW, r = jx - sx * Lo::RW;
    const int sg = in_g ? idx - Lo::G_OFF : idx - Lo::B_OFF;
    const int s = (in_k || in_q) ? sk : (in_x ? sx : sg);
    const bool t_ok = (int64_t)blk * kStage + s < T;
    bool ok;
    int64_t off;
    const TIn* base;
    if (in_k || in_q) {
      ok = t_ok && col < Dk;
      off = ((bt0 + s) * Hk + hk) * Dk + col;
      base = in_k ? k : q;
    } else if (in_x) {
      ok = t_ok && rowbase + r < Dv;
      off = ((bt0 + s) * Hv + h) * Dv + rowbase + r;
      base = x;
    } else {
      ok = t_ok && (in_g || in_b);
      off = (bt0 + s) * Hv + h;
      base = in_g ? g : beta;
    }
    raw[u] = base[ok ? off : 0];
    mask |= (uint64_t)ok << u;
  }
  okmask = mask;
}

template <typename TIn, int NC, int R, int N>
__device__ __forceinline__ void stage_store(float* __restrict__ buf,
                                            const TIn (&raw)[N],
                                            uint64_t okmask) {
  using Lo = SweepLayout<NC, R>;
  static_assert(N == Lo::PF, "prefetch register count");
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int idx = threadIdx.x + kThreads * u;
    if (idx < Lo::SIZE) buf[idx] = ((okmask >> u) & 1) ? to_f32(raw[u]) : 0.f;
  }
}

// Select element `i` of a small register array without dynamic indexing.
template <int N>
__device__ __forceinline__ float pick(const float (&a)[N], int i) {
  float r = a[0];
#pragma unroll
  for (int j = 1; j < N; ++j)
    if (i == j) r = a[j];
  return r;
}

// Load/store this lane's part of rows [row0, row0+R) of a [Dv][Dk] matrix.
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

template <int NC, int R>
__device__ __forceinline__ void tile_store(const float (&S)[R][NC],
                                           float* __restrict__ M, int row0,
                                           int p, int Dk, int Dv) {
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = 4 * p + 64 * (c / 4) + (c % 4);
      const int row = row0 + r;
      if (row < Dv && col < Dk) M[(int64_t)row * Dk + col] = S[r][c];
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

template <typename TIn, int NC, int R>
__global__ __launch_bounds__(kThreads) void fwd_sweep_kernel(FwdSweepArgs a) {
  using Lo = SweepLayout<NC, R>;
  __shared__ __align__(16) float lds[2][Lo::SIZE];

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

  float S[R][NC];
  tile_load<NC, R>(S, a.S0 ? a.S0 + bh * mat : nullptr, row0, p, Dk, Dv);

  const int nblk = (T + kStage - 1) / kStage;
  TIn pre[Lo::PF];
  uint64_t pre_ok = 0;
  if (nblk > 0) {
    stage_fetch<TIn, NC, R>(pre, pre_ok, 0, T, Hk, Hv, Dk, Dv, b, h, hk, rowbase, k, q,
                            v, g, beta);
    stage_store<TIn, NC, R>(lds[0], pre, pre_ok);
  }
  __syncthreads();

  float qprev[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) qprev[c] = 0.f;
  const int my_row = row0 + p;  // row written by lanes p < R
  const bool writer = (p < R) && (my_row < Dv);

  int to_ckpt = 0;  // steps until the next checkpoint (t % L == 0)
  int ckpt_slot = 0;
  for (int blk = 0; blk < nblk; ++blk) {
    const float* __restrict__ cur = lds[blk & 1];
    if (blk + 1 < nblk)
      stage_fetch<TIn, NC, R>(pre, pre_ok, blk + 1, T, Hk, Hv, Dk, Dv, b, h, hk,
                              rowbase, k, q, v, g, beta);
    const int tbase = blk * kStage;
    const int nsteps = min(kStage, T - tbase);
    for (int s = 0; s < nsteps; ++s) {
      const int t = tbase + s;
      float kk[NC], qq[NC];
      lds_cols<NC>(kk, cur + Lo::K_OFF + s * Lo::DKP, p);
      lds_cols<NC>(qq, cur + Lo::Q_OFF + s * Lo::DKP, p);
      if (to_ckpt == 0) {
        if (a.Sck != nullptr)
          tile_store<NC, R>(S, a.Sck + (bh * a.nch + ckpt_slot) * mat, row0, p,
                            Dk, Dv);
        ++ckpt_slot;
        to_ckpt = a.L;
      }
      --to_ckpt;
      // dots on the state before step t: S k_t (for the update) and
      // S q_{t-1} (= y_{t-1}, the read-out of the previous step)
      float pk[R], pq[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float ak = 0.f, aq = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          ak = fmaf(S[r][c], kk[c], ak);
          aq = fmaf(S[r][c], qprev[c], aq);
        }
        pk[r] = rowsum16(ak);
        pq[r] = rowsum16(aq);
      }
      if (t > 0 && writer)
        st(y, ((int64_t)(b * (int64_t)T + t - 1) * Hv + h) * Dv + my_row,
           pick<R>(pq, p));
      const float gt = cur[Lo::G_OFF + s];
      const float bt = cur[Lo::B_OFF + s];
      float d[R], e[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        e[r] = cur[Lo::X_OFF + s * Lo::RW + rg * R + r] - gt * pk[r];
        d[r] = bt * e[r];
      }
      if (a.E != nullptr && writer)
        a.E[((int64_t)(b * (int64_t)T + t) * Hv + h) * Dv + my_row] =
            pick<R>(e, p);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < NC; ++c) S[r][c] = fmaf(d[r], kk[c], gt * S[r][c]);
#pragma unroll
      for (int c = 0; c < NC; ++c) qprev[c] = qq[c];
    }
    if (blk + 1 < nblk) stage_store<TIn, NC, R>(lds[(blk + 1) & 1], pre, pre_ok);
    __syncthreads();
  }

  if (T > 0) {
    float pq[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float aq = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) aq = fmaf(S[r][c], qprev[c], aq);
      pq[r] = rowsum16(aq);
    }
    if (writer)
      st(y, ((int64_t)(b * (int64_t)T + T - 1) * Hv + h) * Dv + my_row,
         pick<R>(pq, p));
  }
  if (a.ST != nullptr) tile_store<NC, R>(S, a.ST + bh * mat, row0, p, Dk, Dv);
}

template <typename TIn, int NC, int R>
__global__ __launch_bounds__(kThreads) void bwd_sweep_kernel(BwdSweepArgs a) {
  using Lo = SweepLayout<NC, R>;
  __shared__ __align__(16) float lds[2][Lo::SIZE];

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

  float H[R][NC];
  tile_load<NC, R>(H, a.dST ? a.dST + bh * mat : nullptr, row0, p, Dk, Dv);
  // slot nch-1 holds dL/dS_T for the last chunk
  if (a.nch > 0)
    tile_store<NC, R>(H, a.Hck + (bh * a.nch + a.nch - 1) * mat, row0, p, Dk,
                      Dv);

  const int nblk = (T + kStage - 1) / kStage;
  TIn pre[Lo::PF];
  uint64_t pre_ok = 0;
  if (nblk > 0) {
    stage_fetch<TIn, NC, R>(pre, pre_ok, nblk - 1, T, Hk, Hv, Dk, Dv, b, h, hk,
                            rowbase, k, q, dy, g, beta);
    stage_store<TIn, NC, R>(lds[(nblk - 1) & 1], pre, pre_ok);
  }
  __syncthreads();

  const int my_row = row0 + p;
  const bool writer = (p < R) && (my_row < Dv);

  // H after step t is saved when t % L == 0 and t > 0, in slot t / L - 1
  int last_chunk = (T - 1) / (a.L > 0 ? a.L : 1);
  int to_ckpt = T - 1 - last_chunk * a.L;  // steps until t % L == 0
  for (int blk = nblk - 1; blk >= 0; --blk) {
    const float* __restrict__ cur = lds[blk & 1];
    if (blk > 0)
      stage_fetch<TIn, NC, R>(pre, pre_ok, blk - 1, T, Hk, Hv, Dk, Dv, b, h, hk,
                              rowbase, k, q, dy, g, beta);
    const int tbase = blk * kStage;
    const int nsteps = min(kStage, T - tbase);
    for (int s = nsteps - 1; s >= 0; --s) {
      const int t = tbase + s;
      float kk[NC], qq[NC];
      lds_cols<NC>(kk, cur + Lo::K_OFF + s * Lo::DKP, p);
      lds_cols<NC>(qq, cur + Lo::Q_OFF + s * Lo::DKP, p);
      const float gt = cur[Lo::G_OFF + s];
      const float bt = cur[Lo::B_OFF + s];
      float c[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float dyr = cur[Lo::X_OFF + s * Lo::RW + rg * R + r];
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          H[r][j] = fmaf(dyr, qq[j], H[r][j]);  // G = H + dy q^T
          acc = fmaf(H[r][j], kk[j], acc);
        }
        c[r] = rowsum16(acc);
      }
      float dvr[R];
#pragma unroll
      for (int r = 0; r < R; ++r) dvr[r] = bt * c[r];
      if (writer) {
        const int64_t o = ((int64_t)(b * (int64_t)T + t) * Hv + h) * Dv + my_row;
        a.C[o] = pick<R>(c, p);
        st(dv, o, pick<R>(dvr, p));
      }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < NC; ++j)
          H[r][j] = gt * fmaf(-dvr[r], kk[j], H[r][j]);
      if (to_ckpt == 0) {
        if (t > 0)
          tile_store<NC, R>(H, a.Hck + (bh * a.nch + last_chunk - 1) * mat,
                            row0, p, Dk, Dv);
        --last_chunk;
        to_ckpt = a.L;
      }
      --to_ckpt;
    }
    if (blk > 0) stage_store<TIn, NC, R>(lds[(blk - 1) & 1], pre, pre_ok);
    __syncthreads();
  }
  if (a.dS0 != nullptr) tile_store<NC, R>(H, a.dS0 + bh * mat, row0, p, Dk, Dv);
}

template <typename TIn, int NC, int R>
hipError_t fwd_launch(const FwdSweepArgs& a, hipStream_t s) {
  using Lo = SweepLayout<NC, R>;
  dim3 grid((a.Dv + Lo::RW - 1) / Lo::RW, a.Hv, a.B);
  hipLaunchKernelGGL((fwd_sweep_kernel<TIn, NC, R>), grid, dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

template <typename TIn, int NC, int R>
hipError_t bwd_launch(const BwdSweepArgs& a, hipStream_t s) {
  using Lo = SweepLayout<NC, R>;
  dim3 grid((a.Dv + Lo::RW - 1) / Lo::RW, a.Hv, a.B);
  hipLaunchKernelGGL((bwd_sweep_kernel<TIn, NC, R>), grid, dim3(kThreads), 0,
                     s, a);
  return hipGetLastError();
}

// Columns per lane: the smallest multiple of 4 with 16 * NC >= Dk.
int pick_nc(int Dk) { return 4 * ((Dk + 63) / 64); }

template <typename TIn>
hipError_t fwd_dispatch(const FwdSweepArgs& a, hipStream_t s) {
  switch (pick_nc(a.Dk)) {
    case 4: return fwd_launch<TIn, 4, 2>(a, s);
    case 8: return fwd_launch<TIn, 8, 2>(a, s);
    case 12: return fwd_launch<TIn, 12, 2>(a, s);
    case 16: return fwd_launch<TIn, 16, 2>(a, s);
  }
  return hipErrorInvalidValue;
}

template <typename TIn>
hipError_t bwd_dispatch(const BwdSweepArgs& a, hipStream_t s) {
  switch (pick_nc(a.Dk)) {
    case 4: return bwd_launch<TIn, 4, 2>(a, s);
    case 8: return bwd_launch<TIn, 8, 2>(a, s);
    case 12: return bwd_launch<TIn, 12, 2>(a, s);
    case 16: return bwd_launch<TIn, 16, 2>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_sweep(const FwdSweepArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? fwd_dispatch<gdr::bf16>(a, s) : fwd_dispatch<float>(a, s);
}

hipError_t launch_bwd_sweep(const BwdSweepArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? bwd_dispatch<gdr::bf16>(a, s) : bwd_dispatch<float>(a, s);
}

}  // namespace gdr
