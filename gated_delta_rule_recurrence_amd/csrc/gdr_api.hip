// Host side of the C ABI declared in include/gdr.h: argument validation, size
// queries and kernel launches.  Every check runs on the host before anything
// is enqueued, so a rejected call touches neither the device nor the stream.
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/gdr.h"
#include "gdr_internal.h"

namespace {

constexpr int64_t kMaxDim = 256;      // Dk, Dv
constexpr int64_t kMaxTile = 64;      // steps of one tile of the kernels
constexpr int64_t kMaxChunk = INT64_C(1) << 30;  // checkpoint interval C
constexpr int64_t kMaxGrid = 65535;   // B and Hv index grid y/z
constexpr int64_t kMaxIndex = INT64_C(1) << 62;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxIndex / a) return false;
  *out = a * b;
  return true;
}

int64_t round_up256(int64_t x) { return (x + 255) & ~int64_t(255); }

// a + b on byte counts already bounded by kMaxIndex
bool add_ok(int64_t a, int64_t b, int64_t* out) {
  if (a > kMaxIndex - b) return false;
  *out = a + b;
  return true;
}

// The kernels' tile: C itself up to 64 steps, else the largest divisor of C
// that is at most 64 (64 for a multiple of 64), so that tiles never straddle
// a checkpoint.
int64_t tile_of(int64_t C) {
  if (C <= kMaxTile) return C;
  for (int64_t d = kMaxTile; d > 1; --d)
    if (C % d == 0) return d;
  return 1;
}

struct Sizes {
  int64_t L;       // tile length
  int64_t m;       // tiles per checkpoint interval (C = m L)
  int64_t ntiles;  // ceil(T / L)
  int64_t nseg;    // saved states: ceil(T / C)
  bool chunked;    // the chunked sweeps take tiles of L steps
  bool replay;     // C > 64: the backward replays the tiles from the saved states
  int64_t state;   // elements of one [B][Hv][Dv][Dk] tensor
  int64_t rows;    // elements of one [B][T][Hv][Dv] tensor
  int64_t ckpt_bytes, ws_bytes, fws_bytes;
  int64_t e_off;   // save buffer: the residuals (C <= 64)
  // backward workspace: state-gradient tiles at 0, then
  int64_t c_off;   // the per-step vectors c
  int64_t k_off;   // the reverse sweep's store sinks (chunked)
  int64_t p_off;   // the reverse records (chunked)
  int64_t rs_off;  // replay: the tile states
  int64_t re_off;  // replay: the residuals
  int64_t rp_off;  // replay: the forward prep records (chunked; else 0)
  int hpw;         // > 0: the chunk kernel gives a workgroup hpw value heads
  int64_t hp_off;  // hpw > 0: the head groups' dq, dk terms
};

int check_shape(const gdr_shape* s, Sizes* z) {
  if (s == nullptr) return GDR_ERR_NULL_ARG;
  if (s->B < 0 || s->T < 0 || s->Hk < 1 || s->Hv < 1 || s->Dk < 1 ||
      s->Dv < 1)
    return GDR_ERR_BAD_SHAPE;
  if (s->Hv % s->Hk != 0) return GDR_ERR_HEAD_RATIO;
  if (s->Dk > kMaxDim || s->Dv > kMaxDim || s->B > kMaxGrid ||
      s->Hv > kMaxGrid)
    return GDR_ERR_UNSUPPORTED_DIM;
  if (s->chunk < 1 || s->chunk > kMaxChunk) return GDR_ERR_BAD_CHUNK;
  if (s->dtype != GDR_F32 && s->dtype != GDR_BF16) return GDR_ERR_BAD_DTYPE;
  if (s->decay != GDR_DECAY_G && s->decay != GDR_DECAY_LOG) return GDR_ERR_BAD_DECAY;
  if (s->T > INT32_MAX / 2) return GDR_ERR_OVERFLOW;

  Sizes r{};
  r.L = tile_of(s->chunk);
  r.m = s->chunk / r.L;
  r.ntiles = (s->T + r.L - 1) / r.L;
  r.nseg = (s->T + s->chunk - 1) / s->chunk;
  r.replay = s->chunk > kMaxTile;
  r.chunked = gdr::chunked_sweep_ok(s->Hk, s->Hv, s->Dk, s->Dv, r.L, s->T,
                                    s->dtype == GDR_BF16);
  int64_t bh, mat, x, tiles, b_tiles, b_rows, b_seg;
  if (!mul_ok(s->B, s->Hv, &bh) || !mul_ok(s->Dv, s->Dk, &mat) ||
      !mul_ok(bh, mat, &r.state) || !mul_ok(r.state, r.ntiles, &tiles) ||
      !mul_ok(s->B, s->T, &x) || !mul_ok(x, s->Hv, &x) ||
      !mul_ok(x, s->Dv, &r.rows) || !mul_ok(tiles, 4, &b_tiles) ||
      !mul_ok(r.rows, 4, &b_rows) || !mul_ok(r.state * 4, r.nseg, &b_seg))
    return GDR_ERR_OVERFLOW;
  int64_t prep = 0, sinks = 0;
  if (r.chunked && (!mul_ok(gdr::chunked_prep_floats(1, 1, r.ntiles), bh, &prep) ||
                    !mul_ok(prep, 4, &prep) || !mul_ok(bh * 256, r.ntiles, &sinks)))
    return GDR_ERR_OVERFLOW;
  // save buffer: a state every C steps, and (C <= 64) the residuals
  if (r.replay) {
    r.ckpt_bytes = b_seg;
  } else {
    r.e_off = round_up256(b_tiles);
    if (!add_ok(r.e_off, b_rows, &r.ckpt_bytes)) return GDR_ERR_OVERFLOW;
  }
  r.fws_bytes = prep;
  // backward workspace
  int64_t end;
  r.c_off = round_up256(b_tiles);
  if (!add_ok(r.c_off, b_rows, &end)) return GDR_ERR_OVERFLOW;
  if (r.chunked) {
    r.k_off = round_up256(end);
    if (!add_ok(r.k_off, sinks, &end)) return GDR_ERR_OVERFLOW;
    r.p_off = round_up256(end);
    if (!add_ok(r.p_off, prep, &end)) return GDR_ERR_OVERFLOW;
  }
  if (r.replay) {
    r.rs_off = round_up256(end);
    if (!add_ok(r.rs_off, b_tiles, &end)) return GDR_ERR_OVERFLOW;
    r.re_off = round_up256(end);
    if (!add_ok(r.re_off, b_rows, &end)) return GDR_ERR_OVERFLOW;
    if (r.chunked) {
      r.rp_off = round_up256(end);
      if (!add_ok(r.rp_off, prep, &end)) return GDR_ERR_OVERFLOW;
    }
  }
  // element counts must also index as int64 inside the kernels
  int64_t qk;
  if (!mul_ok(s->B, s->T, &qk) || !mul_ok(qk, s->Hk, &qk) ||
      !mul_ok(qk, s->Dk, &qk))
    return GDR_ERR_OVERFLOW;
  r.hpw = gdr::chunk_head_split(s->B, s->Hk, s->Hv, s->Dk, s->Dv, r.L, r.ntiles,
                                s->dtype == GDR_BF16);
  if (r.hpw > 0) {
    int64_t pb;  // [2][Hv/Hk/hpw] x qk floats
    if (!mul_ok(qk, 8 * (s->Hv / s->Hk / r.hpw), &pb)) return GDR_ERR_OVERFLOW;
    r.hp_off = round_up256(end);
    if (!add_ok(r.hp_off, pb, &end)) return GDR_ERR_OVERFLOW;
  }
  r.ws_bytes = end;
  if (z) *z = r;
  return GDR_OK;
}

bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

}  // namespace

// ---- scratch of gdr_forward_noalloc ---------------------------------------
// The chunked forward's per-chunk records live here for callers that cannot
// allocate.  Each device that loads the library holds its own copy for the
// life of the process.  In host code `scratch` is only a stand-in for the
// symbol: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is handed to kernels.  Nothing in it has to
// start at zero: the prep kernel writes every record the sweep then reads.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up on its first use on
// that device, with that device current), or nullptr if HIP fails.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

// ---- gdr_set_launch_events -------------------------------------------------
// The caller's events (process-wide: set while no other thread calls in), and
// how many kernels the current call of this host thread has launched.
hipEvent_t launch_events[GDR_MAX_LAUNCH_EVENTS];
int n_launch_events = 0;
thread_local int launch_count = 0;

// A call's end (on success): the events past its last launch, so that every
// set event is recorded once per call.
int end_call(int status, void* stream) {
  if (status == GDR_OK)
    for (int i = launch_count; i < n_launch_events; ++i)
      (void)hipEventRecord(launch_events[i], static_cast<hipStream_t>(stream));
  return status;
}

// gdr_forward's pointer checks (required pointers, alignment)
int forward_pointers_ok(const gdr_shape* shape, const void* q, const void* k, const void* v,
                        const void* g, const void* beta, const float* S0, const void* y,
                        const float* S_T, const void* ckpt, const void* workspace) {
  const bool has_tokens = shape->B > 0 && shape->T > 0;
  if (has_tokens && (!q || !k || !v || !g || !beta || !y))
    return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q, k, v, g, beta, S0, y, S_T, ckpt, workspace};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return GDR_ERR_ALIGNMENT;
  return GDR_OK;
}

// gdr_forward after check_shape: the caller's workspace, or the
// no-allocation scratch array
int forward_checked(const gdr_shape* shape, const Sizes& z, const void* q, const void* k,
                    const void* v, const void* g, const void* beta, const float* S0,
                    const uint8_t* mask, void* y, float* S_T, void* ckpt, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const bool has_tokens = shape->B > 0 && shape->T > 0;
  const bool has_state = shape->B > 0;
  const int pst = forward_pointers_ok(shape, q, k, v, g, beta, S0, y, S_T, ckpt, workspace);
  if (pst != GDR_OK) return pst;
  if (has_tokens && z.fws_bytes > 0 &&
      (workspace == nullptr || workspace_bytes < static_cast<size_t>(z.fws_bytes)))
    return GDR_ERR_WORKSPACE;
  if (!has_state) return GDR_OK;

  gdr::FwdSweepArgs a{};
  a.B = (int)shape->B;
  a.T = (int)shape->T;
  a.Hk = (int)shape->Hk;
  a.Hv = (int)shape->Hv;
  a.Dk = (int)shape->Dk;
  a.Dv = (int)shape->Dv;
  const bool decode = has_tokens && gdr::decode_ok(shape->T);
  const bool chunked = has_tokens && !decode && z.chunked;
  if (chunked) {
    // tiles of L steps, a saved state every m tiles
    a.L = (int)z.L;
    a.nch = (int)z.ntiles;
    a.ck_every = (int)z.m;
  } else {
    // the per-step kernels save a state every C steps
    a.L = (int)shape->chunk;
    a.nch = (int)z.nseg;
    a.ck_every = 1;
  }
  a.nslot = (int)z.nseg;
  a.s0_stride = 1;
  a.seg = 0;
  a.log_g = shape->decay == GDR_DECAY_LOG;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.S0 = S0;
  a.mask = mask;
  a.y = y;
  a.ST = S_T;
  if (ckpt != nullptr) {
    a.Sck = static_cast<float*>(ckpt);
    // C > 64 saves no residuals: the backward replays them
    if (!z.replay) a.E = reinterpret_cast<float*>(static_cast<char*>(ckpt) + z.e_off);
  }
  if (!has_tokens && S_T == nullptr) return GDR_OK;
  const bool bf16 = shape->dtype == GDR_BF16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (decode) {
    err = gdr::launch_decode(a, bf16, s);
  } else if (chunked) {
    gdr::FwdChunkedArgs c{};
    c.s = a;
    c.prep = static_cast<float*>(workspace);
    err = gdr::launch_fwd_chunked(c, bf16, s);
  } else {
    err = gdr::launch_fwd_sweep(a, bf16, s);
  }
  return err == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

}  // namespace

extern "C" {

int gdr_num_chunks(const gdr_shape* shape, int64_t* out) {
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  if (out == nullptr) return GDR_ERR_NULL_ARG;
  *out = z.nseg;
  return GDR_OK;
}

int gdr_checkpoint_bytes(const gdr_shape* shape, size_t* out) {
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  if (out == nullptr) return GDR_ERR_NULL_ARG;
  *out = static_cast<size_t>(z.ckpt_bytes);
  return GDR_OK;
}

int gdr_forward_workspace_bytes(const gdr_shape* shape, size_t* out) {
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  if (out == nullptr) return GDR_ERR_NULL_ARG;
  *out = static_cast<size_t>(z.fws_bytes);
  return GDR_OK;
}

int gdr_backward_workspace_bytes(const gdr_shape* shape, size_t* out) {
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  if (out == nullptr) return GDR_ERR_NULL_ARG;
  *out = static_cast<size_t>(z.ws_bytes);
  return GDR_OK;
}

int gdr_forward(const gdr_shape* shape, const void* q, const void* k,
                const void* v, const void* g, const void* beta,
                const float* S0, const uint8_t* mask, void* y, float* S_T,
                void* ckpt, void* workspace, size_t workspace_bytes,
                void* stream) {
  launch_count = 0;
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  return end_call(forward_checked(shape, z, q, k, v, g, beta, S0, mask, y, S_T, ckpt,
                                  workspace, workspace_bytes, stream),
                  stream);
}

int gdr_forward_noalloc(const gdr_shape* shape, const void* q, const void* k,
                        const void* v, const void* g, const void* beta,
                        const float* S0, const uint8_t* mask, void* y, float* S_T,
                        void* ckpt, void* stream) {
  launch_count = 0;
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  if (z.fws_bytes > static_cast<int64_t>(GDR_NOALLOC_SCRATCH_BYTES)) return GDR_ERR_SCRATCH_LIMIT;
  const int pst = forward_pointers_ok(shape, q, k, v, g, beta, S0, y, S_T, ckpt, nullptr);
  if (pst != GDR_OK) return pst;
  void* ws = nullptr;
  if (z.fws_bytes > 0 && shape->B > 0 && shape->T > 0) {
    ws = scratch_address();
    if (ws == nullptr) return GDR_ERR_HIP;
  }
  return end_call(forward_checked(shape, z, q, k, v, g, beta, S0, mask, y, S_T, ckpt, ws,
                                  ws != nullptr ? GDR_NOALLOC_SCRATCH_BYTES : 0, stream),
                  stream);
}

// gdr_backward's work (the entry point below adds the launch-event hook's
// bookkeeping)
static int backward_call(const gdr_shape* shape, const void* q, const void* k,
                         const void* v, const void* g, const void* beta, const uint8_t* mask,
                         const void* ckpt, const void* dy, const float* dS_T, void* dq,
                         void* dk, void* dv, void* dg, void* dbeta, float* dS0,
                         void* workspace, size_t workspace_bytes, void* stream) {
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  const bool has_tokens = shape->B > 0 && shape->T > 0;
  if (has_tokens && (!q || !k || !g || !beta || !ckpt || !dy || !dq || !dk ||
                     !dv || !dg || !dbeta || !workspace || (z.replay && !v)))
    return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q,  k,  v,  g,     beta, ckpt, dy,       dS_T,
                        dq, dk, dv, dg,    dbeta, dS0, workspace};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return GDR_ERR_ALIGNMENT;
  if (has_tokens && workspace_bytes < static_cast<size_t>(z.ws_bytes))
    return GDR_ERR_WORKSPACE;
  if (shape->B == 0) return GDR_OK;
  if (!has_tokens && dS0 == nullptr) return GDR_OK;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = shape->dtype == GDR_BF16;
  char* const ws = static_cast<char*>(workspace);
  hipError_t err;

  // the state before every tile and the residuals: saved by the forward
  // (C <= 64), or replayed here from the states it saved every C steps
  const float* Sck = static_cast<const float*>(ckpt);
  const float* E =
      reinterpret_cast<const float*>(static_cast<const char*>(ckpt) + z.e_off);
  if (has_tokens && z.replay) {
    gdr::FwdSweepArgs r{};
    r.B = (int)shape->B;
    r.T = (int)shape->T;
    r.Hk = (int)shape->Hk;
    r.Hv = (int)shape->Hv;
    r.Dk = (int)shape->Dk;
    r.Dv = (int)shape->Dv;
    r.L = (int)z.L;
    r.nch = (int)z.ntiles;
    r.ck_every = 1;
    r.nslot = (int)z.ntiles;
    r.s0_stride = (int)z.nseg;  // slot s of each (batch row, value head)
    r.log_g = shape->decay == GDR_DECAY_LOG;
    r.mask = mask;
    r.q = q;
    r.k = k;
    r.v = v;
    r.g = g;
    r.beta = beta;
    r.S0 = static_cast<const float*>(ckpt);
    r.y = nullptr;
    r.ST = nullptr;
    r.Sck = reinterpret_cast<float*>(ws + z.rs_off);
    r.E = reinterpret_cast<float*>(ws + z.re_off);
    if (z.chunked) {
      // one workgroup row per saved state, when the grid takes them
      r.seg = shape->B * z.nseg <= kMaxGrid ? (int)z.m : 0;
      gdr::FwdChunkedArgs fc{};
      fc.s = r;
      fc.prep = reinterpret_cast<float*>(ws + z.rp_off);
      fc.prep_b = reinterpret_cast<float*>(ws + z.p_off);  // and the reverse records
      err = gdr::launch_fwd_chunked(fc, bf16, s);
    } else {
      r.seg = 0;
      err = gdr::launch_fwd_sweep(r, bf16, s);
    }
    if (err != hipSuccess) return GDR_ERR_HIP;
    Sck = r.Sck;
    E = r.E;
  }

  gdr::BwdSweepArgs b{};
  b.B = (int)shape->B;
  b.T = (int)shape->T;
  b.Hk = (int)shape->Hk;
  b.Hv = (int)shape->Hv;
  b.Dk = (int)shape->Dk;
  b.Dv = (int)shape->Dv;
  b.L = (int)z.L;
  b.nch = (int)z.ntiles;
  b.log_g = shape->decay == GDR_DECAY_LOG;
  b.q = q;
  b.k = k;
  b.g = g;
  b.beta = beta;
  b.dy = dy;
  b.dST = dS_T;
  b.mask = mask;
  b.dv = dv;
  b.dS0 = dS0;
  if (has_tokens) {
    b.Hck = reinterpret_cast<float*>(ws);
    b.C = reinterpret_cast<float*>(ws + z.c_off);
  }
  if (has_tokens && z.chunked) {
    gdr::BwdChunkedArgs c{};
    c.s = b;
    // the reverse records: formed here, or (C > 64) by the replay's prep
    // launch together with the forward records
    c.prep = reinterpret_cast<const float*>(ws + z.p_off);
    c.own_prep = z.replay ? 0 : 1;
    c.sink = reinterpret_cast<float*>(ws + z.k_off);
    err = gdr::launch_bwd_chunked(c, bf16, s);
  } else {
    err = gdr::launch_bwd_sweep(b, bf16, s);
  }
  if (err != hipSuccess) return GDR_ERR_HIP;
  if (!has_tokens) return GDR_OK;

  gdr::ChunkArgs c{};
  c.B = b.B;
  c.T = b.T;
  c.Hk = b.Hk;
  c.Hv = b.Hv;
  c.Dk = b.Dk;
  c.Dv = b.Dv;
  c.L = b.L;
  c.nch = b.nch;
  c.log_g = b.log_g;
  c.q = q;
  c.k = k;
  c.g = g;
  c.beta = beta;
  c.dy = dy;
  c.mask = mask;
  c.Sck = Sck;
  c.E = E;
  c.Hck = b.Hck;
  c.C = b.C;
  c.dq = dq;
  c.dk = dk;
  c.dg = dg;
  c.dbeta = dbeta;
  c.part = z.hpw > 0 ? reinterpret_cast<float*>(ws + z.hp_off) : nullptr;
  c.hpw = z.hpw;
  err = gdr::launch_bwd_chunk(c, bf16, s);
  return err == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int gdr_set_launch_events(void* const* events, int n) {
  if (n < 0 || n > GDR_MAX_LAUNCH_EVENTS) return GDR_ERR_BAD_COUNT;
  if (n > 0 && events == nullptr) return GDR_ERR_NULL_ARG;
  for (int i = 0; i < n; ++i)
    if (events[i] == nullptr) return GDR_ERR_NULL_ARG;
  for (int i = 0; i < n; ++i) launch_events[i] = static_cast<hipEvent_t>(events[i]);
  n_launch_events = n;
  return GDR_OK;
}

int gdr_backward(const gdr_shape* shape, const void* q, const void* k,
                 const void* v, const void* g, const void* beta, const uint8_t* mask,
                 const void* ckpt,
                 const void* dy, const float* dS_T, void* dq, void* dk,
                 void* dv, void* dg, void* dbeta, float* dS0,
                 void* workspace, size_t workspace_bytes, void* stream) {
  launch_count = 0;
  return end_call(backward_call(shape, q, k, v, g, beta, mask, ckpt, dy, dS_T, dq, dk, dv,
                                dg, dbeta, dS0, workspace, workspace_bytes, stream),
                  stream);
}

const char* gdr_strerror(int status) {
  switch (status) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case GDR_ERR_BAD_SHAPE: return "B and T must be >= 0 and Hk, Hv, Dk, Dv >= 1";
    case GDR_ERR_HEAD_RATIO: return "Hv must be a multiple of Hk";
    case GDR_ERR_UNSUPPORTED_DIM: return "Dk and Dv must be <= 256, B and Hv <= 65535";
    case GDR_ERR_BAD_CHUNK: return "chunk must be in [1, 2^30]";
    case GDR_ERR_BAD_DTYPE: return "dtype must be GDR_F32 or GDR_BF16";
    case GDR_ERR_OVERFLOW: return "a tensor size overflows 64-bit indexing";
    case GDR_ERR_WORKSPACE: return "workspace is smaller than the size query returns";
    case GDR_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case GDR_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case GDR_ERR_BAD_DECAY: return "decay must be GDR_DECAY_G or GDR_DECAY_LOG";
    case GDR_ERR_SCRATCH_LIMIT:
      return "the forward workspace this shape needs exceeds the no-allocation scratch";
    case GDR_ERR_BAD_COUNT:
      return "the launch-event count must be in [0, GDR_MAX_LAUNCH_EVENTS]";
  }
  return "unknown gdr status";
}

const char* gdr_version(void) { return "0.7.0"; }

}  // extern "C"

namespace gdr {

void note_launch(hipStream_t s) {
  const int i = launch_count++;
  if (i < n_launch_events) (void)hipEventRecord(launch_events[i], s);
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
          hipSuccess ||
      n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace gdr
