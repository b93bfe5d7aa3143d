// Short-sequence forward of the gated delta rule on gfx950: decode (T = 1)
// and other calls of a few steps, with the state in and out (in place when
// S0 and S_T are the same buffer).  Same recurrence as the sweeps (mlx issue
// #4614, recurrence statement under the accuracy table):
//   S <- g_t S;  e_t = v_t - S k_t;  S <- S + beta_t e_t k_t^T;  y_t = S q_t
// At T = 1 the call streams the state once (read, update, write), so it is
// bound by HBM bytes: 2 Dv Dk 4 per (batch row, value head).
//
// Mapping: a 16-lane DPP row owns one state row i; lane p holds the columns
// 64 m + 4 p .. +3 (m < NC / 4) in registers, loaded and stored with 16-byte
// accesses.  Per step the row forms S_i.k, S_i.q and k.q in one pass (three
// 16-lane DPP sums), then
//   u = g (S_i.k),  e = v_i - u,  d = beta e,
//   y_i = g (S_i.q) + d (k.q)   (= (g S_i + d k) . q),
//   S_i <- g S_i + d k.
// Rows are independent, so a row is read completely before it is written and
// S0 == S_T is safe.  Checkpoints (slot j = the state before step j C) and
// the residuals e_t are written when a save buffer is given.
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kThreads = 256;  // 16 rows per workgroup
constexpr int kMaxT = 8;

template <typename TIn, int NC, bool VEC>
__global__ __launch_bounds__(kThreads) void decode_kernel(FwdSweepArgs a) {
  constexpr int NQ = NC / 4;  // 4-column groups per lane
  const TIn* __restrict__ q = static_cast<const TIn*>(a.q);
  const TIn* __restrict__ k = static_cast<const TIn*>(a.k);
  const TIn* __restrict__ v = static_cast<const TIn*>(a.v);
  const TIn* __restrict__ g = static_cast<const TIn*>(a.g);
  const TIn* __restrict__ beta = static_cast<const TIn*>(a.beta);
  TIn* __restrict__ y = static_cast<TIn*>(a.y);
  const int T = a.T, Hk = a.Hk, Hv = a.Hv, Dk = a.Dk, Dv = a.Dv;
  const int tid = threadIdx.x, p = tid & 15;
  const int i = blockIdx.x * 16 + (tid >> 4);
  const int h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (Hv / Hk);
  const bool rok = i < Dv;
  const int64_t bh = (int64_t)b * Hv + h;
  const int64_t mat = (int64_t)Dv * Dk;
  const int64_t row = (int64_t)(rok ? i : 0) * Dk;  // clamped into the matrix

  // state row, raw loads then masked
  float S[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) S[c] = 0.f;
  if (a.S0 != nullptr) {
    Quad<float, VEC> sr[NQ];
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int c = 64 * u + 4 * p;
      const bool ok = rok && c < Dk;
      sr[u].load(a.S0 + bh * mat + row, c, ok, Dk - c);
      m |= Quad<float, VEC>::mask(ok, Dk - c) << (4 * u);
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const f4 x = sr[u].get((m >> (4 * u)) & 15u);
#pragma unroll
      for (int e = 0; e < 4; ++e) S[4 * u + e] = x[e];
    }
  }
  auto store_row = [&](float* dst) __attribute__((always_inline)) {
    if (!rok) return;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int c = 64 * u + 4 * p;
      if (c >= Dk) continue;
      float* o = dst + row + c;
      if (VEC) {
        *reinterpret_cast<f4*>(o) = f4{S[4 * u], S[4 * u + 1], S[4 * u + 2], S[4 * u + 3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (c + e < Dk) o[e] = S[4 * u + e];
      }
    }
  };

  for (int t = 0; t < T; ++t) {
    if (a.Sck != nullptr && t % a.L == 0) store_row(a.Sck + (bh * a.nch + t / a.L) * mat);
    const int64_t kq = (((int64_t)b * T + t) * Hk + hk) * Dk;
    const int64_t gi = ((int64_t)b * T + t) * Hv + h;
    Quad<TIn, VEC> kr[NQ], qr[NQ];
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int c = 64 * u + 4 * p;
      const bool ok = c < Dk;
      kr[u].load(k + kq, c, ok, Dk - c);
      qr[u].load(q + kq, c, ok, Dk - c);
      m |= Quad<TIn, VEC>::mask(ok, Dk - c) << (4 * u);
    }
    const float vi = ld(v, gi * Dv + (rok ? i : 0));
    // an identity step (mask byte 0) has g = 1, beta = 0
    const bool skip = skipped(a.mask, b, T, t);
    const float gt = skip ? 1.f : decay_of(ld(g, gi), a.log_g);
    const float bt = skip ? 0.f : ld(beta, gi);
    float kk[NC], sk = 0.f, sq = 0.f, kqd = 0.f;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const f4 kx = kr[u].get((m >> (4 * u)) & 15u), qx = qr[u].get((m >> (4 * u)) & 15u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kk[4 * u + e] = kx[e];
        sk = fmaf(S[4 * u + e], kx[e], sk);
        sq = fmaf(S[4 * u + e], qx[e], sq);
        kqd = fmaf(kx[e], qx[e], kqd);
      }
    }
    sk = rowsum16(sk);
    sq = rowsum16(sq);
    kqd = rowsum16(kqd);
    const float e = vi - gt * sk;
    const float d = bt * e;
#pragma unroll
    for (int c = 0; c < NC; ++c) S[c] = fmaf(gt, S[c], d * kk[c]);
    if (p == 0 && rok) {
      const int64_t o = gi * Dv + i;
      st(y, o, fmaf(gt, sq, d * kqd));
      if (a.E != nullptr) a.E[o] = e;
    }
  }
  if (a.ST != nullptr) store_row(a.ST + bh * mat);
}

template <typename TIn, bool VEC>
hipError_t launch_nc(const FwdSweepArgs& a, hipStream_t s) {
  const dim3 grid((a.Dv + 15) / 16, a.Hv, a.B);
  const int nc = 4 * ((a.Dk + 63) / 64);
  switch (nc) {
    case 4: hipLaunchKernelGGL((decode_kernel<TIn, 4, VEC>), grid, dim3(kThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_kernel<TIn, 8, VEC>), grid, dim3(kThreads), 0, s, a); break;
    case 12: hipLaunchKernelGGL((decode_kernel<TIn, 12, VEC>), grid, dim3(kThreads), 0, s, a); break;
    case 16: hipLaunchKernelGGL((decode_kernel<TIn, 16, VEC>), grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t e = hipGetLastError();
  note_launch(s);
  return e;
}

template <typename TIn>
hipError_t launch(const FwdSweepArgs& a, hipStream_t s) {
  // 16-byte row accesses need every 4-column group to start on a 4-element
  // boundary
  return a.Dk % 4 == 0 ? launch_nc<TIn, true>(a, s) : launch_nc<TIn, false>(a, s);
}

}  // namespace

bool decode_ok(int64_t T) { return T >= 1 && T <= kMaxT; }

hipError_t launch_decode(const FwdSweepArgs& a, bool bf16, hipStream_t s) {
  return bf16 ? launch<gdr::bf16>(a, s) : launch<float>(a, s);
}

}  // namespace gdr
