// Internal launch interface between the C ABI (gdr_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

// Forward sweep: state recurrence with save.
//
// Time runs in tiles of L steps (nch tiles).  The state before tile c is
// saved to slot c / ck_every of Sck when c % ck_every == 0 (Sck holds nslot
// slots per (batch row, value head)).  The state before the first tile is
// S0 + (bh * s0_stride + s) * Dv * Dk: s0_stride = 1 for a [B][Hv][Dv][Dk]
// S0, and the save buffer's slot count when the forward replays from it.
// seg > 0 (chunked forward only) replays segment by segment: the grid's
// batch dimension is B * ceil(nch / seg), and segment s runs tiles
// s * seg .. from slot s of S0.
struct FwdSweepArgs {
  int B, T, Hk, Hv, Dk, Dv, L, nch;
  int ck_every, nslot, s0_stride, seg;
  int log_g;  // g holds log of the decay
  const uint8_t* mask;  // [B][T], 0 = identity step; may be null
  const void* q;
  const void* k;
  const void* v;
  const void* g;
  const void* beta;
  const float* S0;  // may be null (zeros)
  void* y;     // may be null (a replay writes no outputs)
  float* ST;   // may be null
  float* Sck;  // [B][Hv][nslot][Dv][Dk] or null (inference)
  float* E;    // [B][T][Hv][Dv] or null (inference, or C > 64)
};

// Reverse sweep of the state gradient.
struct BwdSweepArgs {
  int B, T, Hk, Hv, Dk, Dv, L, nch;
  int log_g;  // g holds log of the decay
  const uint8_t* mask;  // [B][T], 0 = identity step; may be null
  const void* q;
  const void* k;
  const void* g;
  const void* beta;
  const void* dy;
  const float* dST;  // may be null (zeros)
  void* dv;
  float* dS0;  // may be null
  float* Hck;  // [B][Hv][nch][Dv][Dk]: slot j = dL/dS after chunk j
  float* C;    // [B][T][Hv][Dv]: G_t k_t
};

// Chunk-parallel contraction: dq, dk, dg, dbeta.
struct ChunkArgs {
  int B, T, Hk, Hv, Dk, Dv, L, nch;
  int log_g;  // g holds log of the decay; dg is then dL/dlog g
  const uint8_t* mask;  // [B][T], 0 = identity step; may be null
  const void* q;
  const void* k;
  const void* g;
  const void* beta;
  const void* dy;
  const float* Sck;
  const float* E;
  const float* Hck;
  const float* C;
  void* dq;
  void* dk;
  void* dg;
  void* dbeta;
  // may be null; else (chunk_head_split) each workgroup takes hpw of the
  // Hv/Hk value heads of a kv head and writes their dq, dk terms here,
  // [2][Hv/Hk/hpw][B][T][Hk][Dk] fp32 (dq, then dk), and a second kernel sums
  // them over the head groups in ascending order
  float* part;
  int hpw;
};

// Chunked sweeps (per-chunk matrices on MFMA): the sequential sweeps'
// arguments plus the per-(batch row, value head, chunk) records written by a
// prep kernel.
struct FwdChunkedArgs {
  FwdSweepArgs s;
  float* prep;    // [B][Hv][nch][kChunkPrepStride]: the forward records
  float* prep_b;  // may be null; else the reverse sweep's records are formed
                  // here too, by the same prep launch
};
struct BwdChunkedArgs {
  BwdSweepArgs s;
  const float* prep;  // [B][Hv][nch][kChunkPrepStride]: the reverse records
  int own_prep;       // 1: form them here first (prep is then writable);
                      // 0: a replay's prep launch formed them
  float* sink;        // [B][Hv][nch][64]: store target of out-of-range lanes
};
// What the prep kernels read.
struct ChunkedSweepShape {
  int B, T, Hk, Hv, Dk, Dv, L, nch;
  int log_g;
  int pair_grid;  // set by the launch: one prep workgroup per pair of value heads
  const uint8_t* mask;
  const void* q;
  const void* k;
  const void* g;
  const void* beta;
};

// Floats per prep record: two [64][64] matrices in MFMA A-fragment order
// (fp32, or three bf16 pieces each: 1.5 times the floats), three per-step
// vectors of 64 and 64 floats that nothing reads (a store target for lanes
// outside the tensors).
constexpr int kChunkPrepStride = 3 * 64 * 64 + 4 * 64;

// Whether the chunked sweeps take this shape, and the floats of their prep
// records.
bool chunked_sweep_ok(int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv, int64_t L, int64_t T,
                      bool bf16);
int64_t chunked_prep_floats(int64_t B, int64_t Hv, int64_t nch);
hipError_t launch_fwd_chunked(const FwdChunkedArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_chunked(const BwdChunkedArgs& a, bool bf16, hipStream_t s);

// Short-sequence forward (decode): whether it takes T steps, and its launch.
bool decode_ok(int64_t T);
hipError_t launch_decode(const FwdSweepArgs& a, bool bf16, hipStream_t s);

hipError_t launch_fwd_sweep(const FwdSweepArgs& a, bool bf16, hipStream_t s);
hipError_t launch_bwd_sweep(const BwdSweepArgs& a, bool bf16, hipStream_t s);

// Compute units of the current device (cached per device).
int device_cu_count();
// After each kernel launch: records the caller's next measurement event on s,
// if gdr_set_launch_events has set one for this launch (include/gdr.h).
void note_launch(hipStream_t s);
hipError_t launch_bwd_chunk(const ChunkArgs& a, bool bf16, hipStream_t s);
// The eight-wave chunk kernel for bf16 inputs (gdr_chunk_bf16.hip): whether it
// takes the shape (Dk, Dv multiples of 8, 48 < Dk <= 256), and its launch.
bool chunk_bf16_ok(const ChunkArgs& a);
hipError_t launch_chunk_bf16(const ChunkArgs& a, hipStream_t s);
// How many value heads that kernel gives a workgroup when it splits a kv
// head's value heads over several (a.part, then the sum over the groups):
// short sequences, whose (chunk, kv head) grid would leave much of the device
// idle; 0 when it does not split.
int chunk_head_split(int64_t B, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv, int64_t L,
                     int64_t nch, bool bf16);

}  // namespace gdr
