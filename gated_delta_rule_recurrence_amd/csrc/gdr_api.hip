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
constexpr int64_t kMaxChunk = 64;     // chunk length C
constexpr int64_t kMaxGrid = 65535;   // B and Hv index grid y/z
constexpr int64_t kMaxIndex = INT64_C(1) << 62;

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > kMaxIndex / a) return false;
  *out = a * b;
  return true;
}

int64_t round_up256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct Sizes {
  int64_t nch;
  int64_t state;     // elements of one [B][Hv][Dv][Dk] tensor
  int64_t ckpt;      // elements of [B][Hv][nch][Dv][Dk]
  int64_t rows;      // elements of one [B][T][Hv][Dv] tensor
  int64_t ckpt_bytes, ws_bytes, fws_bytes;
  int64_t e_off, c_off;  // byte offsets of the per-step vectors
  int64_t p_off;         // byte offset of the backward prep records (or 0)
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
  r.nch = (s->T + s->chunk - 1) / s->chunk;
  int64_t bh, mat, x;
  if (!mul_ok(s->B, s->Hv, &bh) || !mul_ok(s->Dv, s->Dk, &mat) ||
      !mul_ok(bh, mat, &r.state) || !mul_ok(r.state, r.nch, &r.ckpt) ||
      !mul_ok(s->B, s->T, &x) || !mul_ok(x, s->Hv, &x) ||
      !mul_ok(x, s->Dv, &r.rows))
    return GDR_ERR_OVERFLOW;
  int64_t b1, b2;
  if (!mul_ok(r.ckpt, 4, &b1) || !mul_ok(r.rows, 4, &b2)) return GDR_ERR_OVERFLOW;
  r.e_off = round_up256(b1);
  r.c_off = r.e_off;
  if (r.e_off > kMaxIndex - b2) return GDR_ERR_OVERFLOW;
  r.ckpt_bytes = r.e_off + b2;
  r.ws_bytes = r.c_off + b2;
  r.fws_bytes = 0;
  r.p_off = 0;
  if (gdr::chunked_sweep_ok(s->Hk, s->Hv, s->Dk, s->Dv, s->chunk, s->T)) {
    // the chunked sweeps' prep records: the forward's whole workspace, and
    // a region after the backward's per-step vectors
    int64_t f;
    if (!mul_ok(gdr::chunked_prep_floats(1, 1, r.nch), bh, &f) ||
        !mul_ok(f, 4, &r.fws_bytes))
      return GDR_ERR_OVERFLOW;
    r.p_off = round_up256(r.ws_bytes);
    if (r.p_off > kMaxIndex - r.fws_bytes) return GDR_ERR_OVERFLOW;
    r.ws_bytes = r.p_off + r.fws_bytes;
  }
  // element counts must also index as int64 inside the kernels
  int64_t qk;
  if (!mul_ok(s->B, s->T, &qk) || !mul_ok(qk, s->Hk, &qk) ||
      !mul_ok(qk, s->Dk, &qk))
    return GDR_ERR_OVERFLOW;
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
  a.L = (int)shape->chunk;
  a.nch = (int)z.nch;
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
    a.E = reinterpret_cast<float*>(static_cast<char*>(ckpt) + z.e_off);
  }
  if (!has_tokens && S_T == nullptr) return GDR_OK;
  const bool bf16 = shape->dtype == GDR_BF16;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (has_tokens && gdr::decode_ok(shape->T)) {
    err = gdr::launch_decode(a, bf16, s);
  } else if (has_tokens && z.fws_bytes > 0) {
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
  *out = z.nch;
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
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  return forward_checked(shape, z, q, k, v, g, beta, S0, mask, y, S_T, ckpt, workspace,
                         workspace_bytes, stream);
}

int gdr_forward_noalloc(const gdr_shape* shape, const void* q, const void* k,
                        const void* v, const void* g, const void* beta,
                        const float* S0, const uint8_t* mask, void* y, float* S_T,
                        void* ckpt, void* stream) {
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
  return forward_checked(shape, z, q, k, v, g, beta, S0, mask, y, S_T, ckpt, ws,
                         ws != nullptr ? GDR_NOALLOC_SCRATCH_BYTES : 0, stream);
}

int gdr_backward(const gdr_shape* shape, const void* q, const void* k,
                 const void* g, const void* beta, const uint8_t* mask,
                 const void* ckpt,
                 const void* dy, const float* dS_T, void* dq, void* dk,
                 void* dv, void* dg, void* dbeta, float* dS0,
                 void* workspace, size_t workspace_bytes, void* stream) {
  Sizes z;
  const int st = check_shape(shape, &z);
  if (st != GDR_OK) return st;
  const bool has_tokens = shape->B > 0 && shape->T > 0;
  if (has_tokens && (!q || !k || !g || !beta || !ckpt || !dy || !dq || !dk ||
                     !dv || !dg || !dbeta || !workspace))
    return GDR_ERR_NULL_ARG;
  const void* ptrs[] = {q,  k,  g,  beta,  ckpt, dy,       dS_T, dq,
                        dk, dv, dg, dbeta, dS0,  workspace};
  for (const void* p : ptrs)
    if (p != nullptr && !aligned16(p)) return GDR_ERR_ALIGNMENT;
  if (has_tokens && workspace_bytes < static_cast<size_t>(z.ws_bytes))
    return GDR_ERR_WORKSPACE;
  if (shape->B == 0) return GDR_OK;
  if (!has_tokens && dS0 == nullptr) return GDR_OK;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = shape->dtype == GDR_BF16;

  gdr::BwdSweepArgs b{};
  b.B = (int)shape->B;
  b.T = (int)shape->T;
  b.Hk = (int)shape->Hk;
  b.Hv = (int)shape->Hv;
  b.Dk = (int)shape->Dk;
  b.Dv = (int)shape->Dv;
  b.L = (int)shape->chunk;
  b.nch = (int)z.nch;
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
    b.Hck = static_cast<float*>(workspace);
    b.C = reinterpret_cast<float*>(static_cast<char*>(workspace) + z.c_off);
  }
  hipError_t err;
  if (has_tokens && z.p_off > 0) {
    gdr::BwdChunkedArgs c{};
    c.s = b;
    c.prep = reinterpret_cast<float*>(static_cast<char*>(workspace) + z.p_off);
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
  c.Sck = static_cast<const float*>(ckpt);
  c.E = reinterpret_cast<const float*>(static_cast<const char*>(ckpt) +
                                       z.e_off);
  c.Hck = b.Hck;
  c.C = b.C;
  c.dq = dq;
  c.dk = dk;
  c.dg = dg;
  c.dbeta = dbeta;
  err = gdr::launch_bwd_chunk(c, bf16, s);
  return err == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

const char* gdr_strerror(int status) {
  switch (status) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case GDR_ERR_BAD_SHAPE: return "B and T must be >= 0 and Hk, Hv, Dk, Dv >= 1";
    case GDR_ERR_HEAD_RATIO: return "Hv must be a multiple of Hk";
    case GDR_ERR_UNSUPPORTED_DIM: return "Dk and Dv must be <= 256, B and Hv <= 65535";
    case GDR_ERR_BAD_CHUNK: return "chunk must be in [1, 64]";
    case GDR_ERR_BAD_DTYPE: return "dtype must be GDR_F32 or GDR_BF16";
    case GDR_ERR_OVERFLOW: return "a tensor size overflows 64-bit indexing";
    case GDR_ERR_WORKSPACE: return "workspace is smaller than the size query returns";
    case GDR_ERR_ALIGNMENT: return "a pointer is not 16-byte aligned";
    case GDR_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case GDR_ERR_BAD_DECAY: return "decay must be GDR_DECAY_G or GDR_DECAY_LOG";
    case GDR_ERR_SCRATCH_LIMIT:
      return "the forward workspace this shape needs exceeds the no-allocation scratch";
  }
  return "unknown gdr status";
}

const char* gdr_version(void) { return "0.5.0"; }

}  // extern "C"

namespace gdr {

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

hipError_t launch_fwd_sweep(const FwdSweepArgs& a, bool bf16, hipStream_t s) {
  const int cu = device_cu_count();
  return bf16 ? launch_fwd_sweep_bf16(a, cu, s) : launch_fwd_sweep_f32(a, cu, s);
}

hipError_t launch_bwd_sweep(const BwdSweepArgs& a, bool bf16, hipStream_t s) {
  const int cu = device_cu_count();
  return bf16 ? launch_bwd_sweep_bf16(a, cu, s) : launch_bwd_sweep_f32(a, cu, s);
}

}  // namespace gdr
