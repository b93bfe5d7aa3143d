/* Host-side checks of the C ABI (include/gdr.h) for a sanitizer build: the
 * size queries over many shapes (small, headline, long-context, checkpoint
 * intervals above one tile, near-overflow), and every argument-rejection path
 * of the entry points.  Nothing here reaches the device: every call either
 * only computes sizes or is rejected on the host.  Exits non-zero on the
 * first wrong status.  Built and run by tests/test_sanitizers.py. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gdr.h"

static int fails = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                              \
    }                                                                       \
  } while (0)

static gdr_shape shape(int64_t B, int64_t T, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv,
                       int64_t C, int32_t dtype) {
  gdr_shape s;
  memset(&s, 0, sizeof s);
  s.B = B; s.T = T; s.Hk = Hk; s.Hv = Hv; s.Dk = Dk; s.Dv = Dv; s.chunk = C;
  s.dtype = dtype; s.decay = GDR_DECAY_G;
  return s;
}

int main(void) {
  /* a 16-byte aligned address that is never dereferenced: every call below
   * is rejected or sized on the host */
  static char fake_buf[64] __attribute__((aligned(16)));
  void* F = fake_buf;
  void* M = fake_buf + 4; /* misaligned */
  size_t n = 0;
  int64_t nc = 0;

  /* size queries over a spread of shapes and intervals */
  const int64_t Cs[] = {1, 2, 7, 16, 50, 64, 65, 96, 97, 128, 512, 8192, (int64_t)1 << 30};
  const int64_t Ts[] = {0, 1, 8, 63, 64, 300, 2048, 8192};
  for (size_t i = 0; i < sizeof Cs / sizeof Cs[0]; ++i)
    for (size_t j = 0; j < sizeof Ts / sizeof Ts[0]; ++j)
      for (int dt = 0; dt < 2; ++dt) {
        gdr_shape s = shape(4, Ts[j], 16, 64, 192, 128, Cs[i], dt);
        EXPECT(gdr_checkpoint_bytes(&s, &n) == GDR_OK);
        EXPECT(gdr_forward_workspace_bytes(&s, &n) == GDR_OK);
        EXPECT(gdr_backward_workspace_bytes(&s, &n) == GDR_OK);
        EXPECT(gdr_num_chunks(&s, &nc) == GDR_OK);
        EXPECT(nc == (Ts[j] + Cs[i] - 1) / Cs[i]);
        s.Dk = 256;
        EXPECT(gdr_checkpoint_bytes(&s, &n) == GDR_OK);
        EXPECT(gdr_forward_workspace_bytes(&s, &n) == GDR_OK);
        EXPECT(gdr_backward_workspace_bytes(&s, &n) == GDR_OK);
        /* a small grid: the chunk kernel's head groups at Dk = 256 (bf16) */
        gdr_shape w = shape(1, Ts[j], 2, 4, 256, 128, Cs[i], dt);
        EXPECT(gdr_checkpoint_bytes(&w, &n) == GDR_OK);
        EXPECT(gdr_forward_workspace_bytes(&w, &n) == GDR_OK);
        EXPECT(gdr_backward_workspace_bytes(&w, &n) == GDR_OK);
      }

  /* shape errors */
  gdr_shape s = shape(1, 4, 2, 4, 8, 8, 2, GDR_F32);
  s.chunk = 0; EXPECT(gdr_checkpoint_bytes(&s, &n) == GDR_ERR_BAD_CHUNK);
  s.chunk = ((int64_t)1 << 30) + 1; EXPECT(gdr_checkpoint_bytes(&s, &n) == GDR_ERR_BAD_CHUNK);
  s = shape(1, 4, 3, 4, 8, 8, 2, GDR_F32); EXPECT(gdr_num_chunks(&s, &nc) == GDR_ERR_HEAD_RATIO);
  s = shape(1, 4, 2, 4, 300, 8, 2, GDR_F32);
  EXPECT(gdr_num_chunks(&s, &nc) == GDR_ERR_UNSUPPORTED_DIM);
  s = shape(1, (int64_t)1 << 40, 2, 4, 8, 8, 2, GDR_F32);
  EXPECT(gdr_num_chunks(&s, &nc) == GDR_ERR_OVERFLOW);
  s = shape(65535, (int64_t)1 << 30, 65535, 65535, 256, 256, 1, GDR_F32);
  EXPECT(gdr_checkpoint_bytes(&s, &n) == GDR_ERR_OVERFLOW);
  s = shape(1, 4, 2, 4, 8, 8, 2, 7); EXPECT(gdr_num_chunks(&s, &nc) == GDR_ERR_BAD_DTYPE);
  s = shape(1, 4, 2, 4, 8, 8, 2, GDR_F32); s.decay = 9;
  EXPECT(gdr_num_chunks(&s, &nc) == GDR_ERR_BAD_DECAY);
  EXPECT(gdr_num_chunks(NULL, &nc) == GDR_ERR_NULL_ARG);
  s = shape(1, 4, 2, 4, 8, 8, 2, GDR_F32);
  EXPECT(gdr_num_chunks(&s, NULL) == GDR_ERR_NULL_ARG);

  /* forward rejections: required pointers, alignment, workspace */
  s = shape(1, 64, 2, 4, 64, 32, 32, GDR_F32); /* chunked: needs a workspace */
  size_t ws = 0;
  EXPECT(gdr_forward_workspace_bytes(&s, &ws) == GDR_OK && ws > 0);
  EXPECT(gdr_forward(&s, NULL, F, F, F, F, NULL, NULL, F, F, F, F, ws, NULL) == GDR_ERR_NULL_ARG);
  EXPECT(gdr_forward(&s, F, F, F, F, F, NULL, NULL, NULL, F, F, F, ws, NULL) == GDR_ERR_NULL_ARG);
  EXPECT(gdr_forward(&s, F, M, F, F, F, NULL, NULL, F, F, F, F, ws, NULL) == GDR_ERR_ALIGNMENT);
  EXPECT(gdr_forward(&s, F, F, F, F, F, NULL, NULL, F, F, F, F, ws - 1, NULL) == GDR_ERR_WORKSPACE);
  EXPECT(gdr_forward(&s, F, F, F, F, F, NULL, NULL, F, F, F, NULL, ws, NULL) == GDR_ERR_WORKSPACE);
  EXPECT(gdr_forward_noalloc(&s, F, F, NULL, F, F, NULL, NULL, F, F, F, NULL) == GDR_ERR_NULL_ARG);
  EXPECT(gdr_forward_noalloc(&s, F, F, F, F, F, (const float*)M, NULL, F, F, F, NULL) ==
         GDR_ERR_ALIGNMENT);
  s = shape(1, 4096, 16, 64, 192, 128, 64, GDR_BF16);
  EXPECT(gdr_forward_noalloc(&s, F, F, F, F, F, NULL, NULL, F, F, F, NULL) ==
         GDR_ERR_SCRATCH_LIMIT);

  /* backward rejections */
  s = shape(1, 200, 2, 4, 64, 32, 128, GDR_F32); /* replay: needs v */
  EXPECT(gdr_backward_workspace_bytes(&s, &ws) == GDR_OK);
  EXPECT(gdr_backward(&s, F, F, NULL, F, F, NULL, F, F, NULL, F, F, F, F, F, NULL, F, ws, NULL) ==
         GDR_ERR_NULL_ARG);
  EXPECT(gdr_backward(&s, F, F, F, F, F, NULL, F, F, NULL, F, F, F, F, F, NULL, F, ws - 1, NULL) ==
         GDR_ERR_WORKSPACE);
  EXPECT(gdr_backward(&s, F, F, F, F, F, NULL, F, F, NULL, F, F, F, F, M, NULL, F, ws, NULL) ==
         GDR_ERR_ALIGNMENT);
  EXPECT(gdr_backward(NULL, F, F, F, F, F, NULL, F, F, NULL, F, F, F, F, F, NULL, F, ws, NULL) ==
         GDR_ERR_NULL_ARG);

  /* empty problems launch nothing */
  s = shape(0, 64, 2, 4, 64, 32, 32, GDR_F32);
  EXPECT(gdr_forward(&s, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                     NULL) == GDR_OK);
  EXPECT(gdr_backward(&s, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                      NULL, NULL, NULL, NULL, 0, NULL) == GDR_OK);

  /* every status has a message */
  for (int st = 0; st >= -13; --st) EXPECT(strstr(gdr_strerror(st), "unknown") == NULL);
  /* the launch-event hook: argument checks (set, then cleared before any launch) */
  {
    void* evs[GDR_MAX_LAUNCH_EVENTS + 1];
    for (int i = 0; i <= GDR_MAX_LAUNCH_EVENTS; ++i) evs[i] = F;
    EXPECT(gdr_set_launch_events(evs, GDR_MAX_LAUNCH_EVENTS + 1) == GDR_ERR_BAD_COUNT);
    EXPECT(gdr_set_launch_events(evs, -1) == GDR_ERR_BAD_COUNT);
    EXPECT(gdr_set_launch_events(NULL, 2) == GDR_ERR_NULL_ARG);
    evs[1] = NULL;
    EXPECT(gdr_set_launch_events(evs, 2) == GDR_ERR_NULL_ARG);
    EXPECT(gdr_set_launch_events(evs, 1) == GDR_OK);
    EXPECT(gdr_set_launch_events(NULL, 0) == GDR_OK);
  }
  EXPECT(strstr(gdr_strerror(-99), "unknown") != NULL);
  EXPECT(strlen(gdr_version()) >= 5);

  if (fails) {
    fprintf(stderr, "%d checks failed\n", fails);
    return 1;
  }
  printf("abi host checks passed\n");
  return 0;
}
