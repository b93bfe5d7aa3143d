/*
 * gdr.h - C ABI of the MI355X (gfx950) gated delta rule library (libgdr.so).
 *
 * The operation (mlx issue #4614 "mx.fast.gated_delta_update VJP: wrong
 * gradient w.r.t. g", recurrence statement under the accuracy table, and the
 * repro script's recurrence helper): for every batch row b and value head h,
 * reading kv head h / (Hv/Hk), with a state S[Dv][Dk] (fp32):
 *
 *     S <- g_t * S;   S <- S + outer(beta_t * (v_t - S k_t), k_t);   y_t = S q_t
 *
 * gdr_forward runs it and saves what the VJP needs (forward-with-save, mlx-lm
 * PR #1217 "Add Metal VJP kernel for gated_delta_update", section "What this
 * PR adds"); gdr_backward returns the gradients of q, k, v, g, beta and the
 * initial state from a deterministic reverse sweep (no atomics; fixed
 * reduction order, so repeated calls are bitwise identical on one GPU).
 *
 * Layouts (all dense, row-major, last index fastest, no strides):
 *   q, k, dq, dk      [B][T][Hk][Dk]      element type = shape.dtype
 *   v, y, dv, dy      [B][T][Hv][Dv]      element type = shape.dtype
 *   g, beta, dg, dbeta[B][T][Hv]          element type = shape.dtype
 *   S0, S_T, dS_T, dS0[B][Hv][Dv][Dk]     always fp32
 *   g is the decay itself and dg is dL/dg, unless shape.decay is
 *   GDR_DECAY_LOG (see gdr_decay).
 *
 * Ownership: every buffer is allocated and freed by the caller; all data
 * pointers are device pointers.  The library allocates nothing and is
 * reentrant; the only state it keeps between calls is the scratch array of
 * gdr_forward_noalloc and the event list of gdr_set_launch_events, each
 * with the concurrency rule stated there.  Work is enqueued on `stream`
 * (hipStream_t, NULL = the default stream) without any host synchronisation;
 * results are ready when the stream reaches that point.
 *
 * Errors: every function returns GDR_OK (0) or a negative gdr_status.  All
 * argument checks happen on the host before anything is enqueued, so a
 * rejected call has no effect.  Nothing crosses the ABI as an exception.
 * gdr_strerror() maps a status to a static string.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDR_OK = 0,
  GDR_ERR_NULL_ARG = -1,        /* a required pointer is NULL                  */
  GDR_ERR_BAD_SHAPE = -2,       /* B or T < 0, or Hk, Hv, Dk, Dv < 1            */
  GDR_ERR_HEAD_RATIO = -3,      /* Hv is not a multiple of Hk                   */
  GDR_ERR_UNSUPPORTED_DIM = -4, /* Dk or Dv > 256, or B or Hv > 65535           */
  GDR_ERR_BAD_CHUNK = -5,       /* chunk outside [1, 2^30]                      */
  GDR_ERR_BAD_DTYPE = -6,       /* dtype is not GDR_F32 or GDR_BF16             */
  GDR_ERR_OVERFLOW = -7,        /* a byte size does not fit in 63 bits          */
  GDR_ERR_WORKSPACE = -8,       /* workspace smaller than the size query says  */
  GDR_ERR_ALIGNMENT = -9,       /* a pointer is not 16-byte aligned             */
  GDR_ERR_HIP = -10,            /* the HIP runtime rejected a launch            */
  GDR_ERR_BAD_DECAY = -11,      /* decay is not GDR_DECAY_G or GDR_DECAY_LOG    */
  GDR_ERR_SCRATCH_LIMIT = -12,  /* gdr_forward_noalloc: the shape's forward
                                   workspace exceeds GDR_NOALLOC_SCRATCH_BYTES */
  GDR_ERR_BAD_COUNT = -13       /* gdr_set_launch_events: n outside
                                   0 .. GDR_MAX_LAUNCH_EVENTS               */
} gdr_status;

/* Size of the device-side scratch array behind gdr_forward_noalloc (128 MiB;
 * each device that loads the library holds one for the life of the
 * process). */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

typedef enum { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

/* How the g tensor carries the decay (mlx issue #4614, the note under the
 * accuracy table: models train the decay through its log, e.g. Qwen3.5's
 * A_log/dt_bias chain; the issue's repro script draws log g and takes
 * g = exp(log g)).
 *   GDR_DECAY_G:   g_t is the decay; gdr_backward's dg is dL/dg_t.
 *   GDR_DECAY_LOG: g holds lg_t = log of the decay; the kernels use
 *                  g_t = exp(lg_t) (fp32), and gdr_backward's dg is
 *                  dL/dlg_t = g_t dL/dg_t.  A forward and the backward that
 *                  uses its save buffer must use the same setting. */
typedef enum { GDR_DECAY_G = 0, GDR_DECAY_LOG = 1 } gdr_decay;

/* Problem description.  chunk = C >= 1, the checkpoint interval: the forward
 * saves the state every C steps (the "fixed-size chunks" of the pages'
 * chunked VJP, mlx-lm PR #1217 "What this PR adds"); the last chunk may be
 * shorter.  The kernels work in tiles of L steps: L = C for C <= 64, else
 * the largest divisor of C that is at most 64 (64 for a multiple of 64).
 *   C <= 64: the save buffer holds the state before every chunk and the
 *            per-step residuals; the backward reads them.
 *   C > 64:  the save buffer holds only the state before every chunk
 *            (ceil(T / C) states: less memory held from the forward to the
 *            backward); the backward first replays the forward tiles of each
 *            chunk from its saved state into its workspace (recompute), then
 *            runs as for C = L.
 * Results do not depend on C beyond fp32 rounding. */
typedef struct {
  int64_t B, T, Hk, Hv, Dk, Dv;
  int64_t chunk;
  int32_t dtype; /* gdr_dtype: element type of q,k,v,g,beta,y,dy and grads */
  int32_t decay; /* gdr_decay: what g holds (0 = the decay itself) */
} gdr_shape;

/* Number of saved states (chunks), ceil(T / chunk) (0 when T == 0). */
int gdr_num_chunks(const gdr_shape* shape, int64_t* out);

/* Bytes of the forward save buffer `ckpt`:
 *   state checkpoints  S_{jC} for j = 0..nchunks-1   [B][Hv][nchunks][Dv][Dk] fp32
 *   per-step residual  e_t = v_t - g_t S_{t-1} k_t    [B][T][Hv][Dv]           fp32
 *                      (chunk <= 64 only)
 * each region starting on a 256-byte boundary. */
int gdr_checkpoint_bytes(const gdr_shape* shape, size_t* out);

/* Bytes of the scratch buffer gdr_backward needs: the state-gradient
 * checkpoints (one per tile) and the per-step G_t k_t vectors, fp32, the
 * per-tile records of the chunked reverse sweep, for chunk > 64 the
 * replayed tile states, residuals and forward records, and, for bf16 inputs
 * whose (tile, kv head, batch row) grid is under 256 with 2 to 16 value
 * heads per kv head, the fp32 dq, dk terms of each group of value heads
 * (summed over the groups into dq, dk). */
int gdr_backward_workspace_bytes(const gdr_shape* shape, size_t* out);

/* Bytes of the scratch buffer gdr_forward needs.  Shapes with Dk <= 192 (or
 * Dk <= 256 for bf16 inputs with Dk a multiple of 8 and Dv of 4), a tile of
 * 16 to 64 steps and T at least one tile take the chunked forward
 * (the products inside a tile on matrix cores), which keeps two 64 x 64 fp32
 * matrices and three vectors per (batch row, value head, tile) here; every
 * other shape takes the sequential sweep and needs 0 bytes. */
int gdr_forward_workspace_bytes(const gdr_shape* shape, size_t* out);

/* The step mask (optional, both passes): mask[B][T] uint8, NULL means every
 * step is valid.  A step whose mask byte is 0 is an identity step: it leaves
 * the state unchanged (as g_t = 1, beta_t = 0 would), y_t is still the
 * read-out of the unchanged state, and gdr_backward returns dg_t = dbeta_t =
 * dv_t = 0 and no k_t gradient from it (dq_t and the read-out stay).  A batch
 * of sequences of unequal lengths, padded on either side, runs in one call
 * with it.  The pages name a mask argument of gated_delta_update (mlx-lm PR
 * #1217, "What this PR adds") but do not define it; this is the reading
 * taken.  The forward and the backward that uses its save buffer must get the
 * same mask. */

/* Forward pass.
 *   in : q, k, v, g, beta (shape.dtype); S0 (fp32, NULL means zeros);
 *        mask (see above, NULL means none)
 *   out: y (shape.dtype); S_T (fp32, NULL means not written);
 *        ckpt (gdr_checkpoint_bytes bytes, NULL means inference: nothing is
 *        saved and gdr_backward cannot follow).
 *   workspace: at least gdr_forward_workspace_bytes bytes of device memory
 *        (may be NULL when that is 0), contents ignored on entry and undefined
 *        on exit; GDR_ERR_WORKSPACE if smaller.
 * The algorithms (a per-step form for calls of up to 8 steps and for shapes
 * outside the chunked range, the chunked form otherwise) compute the
 * recurrence of mlx issue #4614 (recurrence statement under the accuracy
 * table) and write the same outputs; they differ in rounding order only.
 * S_T may be the S0 buffer (the state is then updated in place).
 * `stream` is a hipStream_t passed as void*. */
int gdr_forward(const gdr_shape* shape, const void* q, const void* k,
                const void* v, const void* g, const void* beta,
                const float* S0, const uint8_t* mask, void* y, float* S_T,
                void* ckpt, void* workspace, size_t workspace_bytes,
                void* stream);

/* gdr_forward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as gdr_forward, without the workspace:
 * the chunked forward's per-chunk records go to a scratch array inside the
 * library (GDR_NOALLOC_SCRATCH_BYTES per device, located once per device on
 * its first use).  The call allocates and frees nothing; the caller still
 * passes every input and output buffer (ckpt included, when saving).
 *   Limit: shapes whose gdr_forward_workspace_bytes exceeds
 *   GDR_NOALLOC_SCRATCH_BYTES are rejected with GDR_ERR_SCRATCH_LIMIT before
 *   anything is enqueued (at Hv = 64 and chunk 64 that is B * T up to about
 *   2,600 steps; shapes with a 0-byte workspace always pass).
 *   Concurrency: every call on one device shares that device's array, so
 *   calls whose work overlaps on one device (different streams, or other
 *   host threads) race on it and give undefined results; calls ordered on
 *   one stream are safe. */
int gdr_forward_noalloc(const gdr_shape* shape, const void* q, const void* k,
                        const void* v, const void* g, const void* beta,
                        const float* S0, const uint8_t* mask, void* y, float* S_T,
                        void* ckpt, void* stream);

/* Backward pass (VJP of gdr_forward for L = <dy, y> + <dS_T, S_T>).
 *   in : q, k, v, g, beta, dy (shape.dtype) - the same q, k, v, g, beta and
 *        mask given to gdr_forward; ckpt as written by that gdr_forward call;
 *        dS_T (fp32, NULL means zeros).  v is read only when chunk > 64 (to
 *        replay the tiles) and may be NULL otherwise.
 *   out: dq, dk (summed over the Hv/Hk value heads of each kv head, in
 *        ascending head order), dv, dg, dbeta (shape.dtype);
 *        dS0 (fp32, NULL means not written).
 *   workspace: at least gdr_backward_workspace_bytes bytes of device memory,
 *        contents ignored on entry and undefined on exit. */
int gdr_backward(const gdr_shape* shape, const void* q, const void* k,
                 const void* v, const void* g, const void* beta, const uint8_t* mask,
                 const void* ckpt,
                 const void* dy, const float* dS_T, void* dq, void* dk,
                 void* dv, void* dg, void* dbeta, float* dS0,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Measurement hook, for callers that time the library's kernels one by one
 * (a profiler-free per-kernel breakdown; not needed to compute anything).
 * While n > 0, every gdr_forward, gdr_forward_noalloc and gdr_backward call
 * records events[i] on its stream right after launching its i-th kernel
 * (counted from 0 in each call; launches past the n-th record nothing) and,
 * when it succeeds, the events past its last launch at its end, so that each
 * event is recorded once per call.  The time between two consecutive events,
 * or between an event the caller records before the call and events[0], is
 * then one kernel's (zero past the call's last kernel).  events holds n
 * hipEvent_t handles that the caller created and owns (with timing for
 * elapsed times); n = 0 clears the hook.  The setting is process-wide: set
 * it only while no other host thread calls into the library.  A chunked call
 * launches, in order: forward - the prep, the sweep; backward (chunk <= 64) -
 * the prep, the reverse sweep, the chunk kernel and, when it splits the
 * value heads (see gdr_backward_workspace_bytes), the sum of their dq, dk
 * terms.  Errors: GDR_ERR_BAD_COUNT (n outside 0 .. GDR_MAX_LAUNCH_EVENTS),
 * GDR_ERR_NULL_ARG (events, or one of its first n entries, is NULL, n > 0). */
#define GDR_MAX_LAUNCH_EVENTS 8
int gdr_set_launch_events(void* const* events, int n);

/* Static, human-readable text for a gdr_status value. */
const char* gdr_strerror(int status);

/* Library version as "major.minor.patch". */
const char* gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
