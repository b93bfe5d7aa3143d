// In-bounds probes of the device helpers the kernels are built on, compiled
// into a test-only library (libgdr_probe.so, not part of libgdr.so):
//   * split3_quad: the exact three-piece bf16 split of fp32 values;
//   * lds_read_tr16 (ds_read_b64_tr_b16): which elements each lane receives;
//   * tile_operand: the MFMA operand it gathers from a swizzled bf16 tile;
//   * compute peaks: loops of one instruction kind (fp32 FMA on the vector
//     ALU, bf16 and fp32 MFMA) whose launch the host times, so that the
//     benchmark can report what this build reaches on the device next to
//     the published peaks (fp32 vector code here is built without packed
//     FP32 instructions, so its peak is the non-packed rate).
// The tests compare the outputs with CPU models of the same definitions.
// Every kernel indexes only within the buffers the host sizes below, and
// each entry point checks its sizes before launching.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../gated_delta_rule_recurrence_amd/csrc/gdr_device.h"

namespace {

// n4 groups of four floats -> three planes of packed bf16 pieces
__global__ void split3_probe(const float* __restrict__ x, uint2* __restrict__ pieces, int n4) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 v = reinterpret_cast<const float4*>(x)[i];
  uint2 hi, mid, lo;
  gdr::split3_quad(gdr::f4{v.x, v.y, v.z, v.w}, hi, mid, lo);
  pieces[i] = hi;
  pieces[n4 + i] = mid;
  pieces[2 * n4 + i] = lo;
}

// One wave.  LDS holds 1024 uint16 values v[e] = e ^ 0x5a5a; lane l names
// the 8-byte block at element offset 4 * blk[l] (blk[l] < 256) and receives
// four uint16 through the transposing read.
__global__ void tr16_probe(const int* __restrict__ blk, uint16_t* __restrict__ out) {
  __shared__ __align__(16) uint16_t t[1024];
  const int l = threadIdx.x;
  for (int e = l; e < 1024; e += 64) t[e] = (uint16_t)(e ^ 0x5a5a);
  __syncthreads();
  const uint2 r = gdr::lds_read_tr16(t + 4 * blk[l]);
  out[4 * l + 0] = (uint16_t)(r.x & 0xffffu);
  out[4 * l + 1] = (uint16_t)(r.x >> 16);
  out[4 * l + 2] = (uint16_t)(r.y & 0xffffu);
  out[4 * l + 3] = (uint16_t)(r.y >> 16);
}

// One wave.  A swizzled [64][RS] bf16 tile (RS = 192: 384-byte rows, an odd
// multiple of 128) holds value(r, c) = (r * 192 + c) ^ 0x3c3c at row r,
// column c, stored at block (c / 4) ^ tile_swz(r); each lane gathers the
// operand tile_operand(k0, n0) and writes its eight values.
constexpr int kRS = 192;
__global__ void tile_operand_probe(int k0, int n0, uint16_t* __restrict__ out) {
  __shared__ __align__(16) uint16_t t[64 * kRS];
  const int l = threadIdx.x;
  for (int e = l; e < 64 * kRS; e += 64) {
    const int r = e / kRS, c = e % kRS;
    const int o = r * kRS + 4 * ((c >> 2) ^ gdr::tile_swz(r)) + (c & 3);
    t[o] = (uint16_t)((r * kRS + c) ^ 0x3c3c);
  }
  __syncthreads();
  const uint4 v = gdr::tile_operand<kRS>(t, k0, n0, l & 15, l >> 4);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  for (int e = 0; e < 8; ++e) out[8 * l + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
}

// Compute peaks.  Every thread (fma) or wave (mfma) runs independent chains
// of one instruction for `iters` iterations and writes the sum of its
// accumulators, one float per thread.  The values converge or count
// exactly, so the tests can check them:
//   fma:  a <- a * 0.5 + 1 from a = k (k = 0..7), eight chains, 128 FMAs per
//         iteration: every chain reaches 2 exactly, the sum is 16;
//   mfma: operands of ones (x, y: the bf16 / fp32 one from the host), four
//         accumulators from zero: each bf16 MFMA adds 32 to every element,
//         each fp32 one 4; a thread's sum is 4 * 4 * that * iters.
__global__ __launch_bounds__(256) void fma_peak(float* __restrict__ out, int iters, float m,
                                                float c) {
  float a[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) a[k] = (float)k;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 16; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) a[k] = fmaf(a[k], m, c);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += a[k];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_bf16_peak(float* __restrict__ out, int iters,
                                                      uint32_t one2) {
  const uint4 x = {one2, one2, one2, one2};
  gdr::f4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = gdr::f4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = gdr::mfma_bf16(x, x, acc[u]);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) s += (acc[u][0] + acc[u][1]) + (acc[u][2] + acc[u][3]);
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_f32_peak(float* __restrict__ out, int iters,
                                                     float one) {
  gdr::f4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = gdr::f4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = gdr::mfma(one, one, acc[u]);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) s += (acc[u][0] + acc[u][1]) + (acc[u][2] + acc[u][3]);
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// x: 4 * n4 floats; pieces: 3 * n4 uint2 (device pointers).  0 or -1.
int gdr_probe_split3(const float* x, uint32_t* pieces, int n4, void* stream) {
  if (x == nullptr || pieces == nullptr || n4 <= 0) return -1;
  const int threads = 256;
  hipLaunchKernelGGL(split3_probe, dim3((n4 + threads - 1) / threads), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), x, reinterpret_cast<uint2*>(pieces), n4);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// blk: 64 ints in [0, 256); out: 256 uint16 (device pointers).  The host
// cannot see blk, so the caller guarantees its range (the test builds it).
int gdr_probe_tr16(const int* blk, uint16_t* out, void* stream) {
  if (blk == nullptr || out == nullptr) return -1;
  hipLaunchKernelGGL(tr16_probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), blk, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// k0 in {0, 32}, n0 a multiple of 16 below 192; out: 512 uint16.
int gdr_probe_tile_operand(int k0, int n0, uint16_t* out, void* stream) {
  if (out == nullptr || (k0 != 0 && k0 != 32) || n0 < 0 || n0 % 16 != 0 || n0 + 16 > kRS)
    return -1;
  hipLaunchKernelGGL(tile_operand_probe, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                     k0, n0, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// kind 0: fp32 FMA, 1: bf16 MFMA (16x16x32), 2: fp32 MFMA (16x16x4); blocks
// workgroups of 256 threads, out: 256 * blocks floats (device).  Flops per
// launch: kind 0: 256 * blocks * iters * 256; kinds 1, 2: blocks * 4 waves *
// iters * 4 * (16384 or 2048).  0 or -1.
int gdr_probe_peak(int kind, int blocks, int iters, float* out, void* stream) {
  if (out == nullptr || blocks < 1 || blocks > 65535 || iters < 1 || iters > (1 << 20) ||
      kind < 0 || kind > 2)
    return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(fma_peak, dim3(blocks), dim3(256), 0, s, out, iters, 0.5f, 1.0f);
  else if (kind == 1)
    hipLaunchKernelGGL(mfma_bf16_peak, dim3(blocks), dim3(256), 0, s, out, iters,
                       0x3f803f80u);  // two bf16 ones
  else
    hipLaunchKernelGGL(mfma_f32_peak, dim3(blocks), dim3(256), 0, s, out, iters, 1.0f);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
