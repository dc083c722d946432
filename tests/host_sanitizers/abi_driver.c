/* abi_driver.c -- drives every entry point of include/forge.h through its argument checks,
 * built together with the host code (forge_host.cpp) under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  The kernel launchers are replaced by stubs that count calls and
 * refuse (launch_stubs.cpp), so no GPU is touched; device pointers are fake, aligned addresses
 * that the host code must never dereference.  Exit status 0 means every call returned the
 * expected status and left a message where it failed; any sanitizer report aborts the run. */
#include <float.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "forge.h"

extern int forge_stub_launches(void); /* launch_stubs.cpp */

static int g_fail = 0, g_calls = 0;

/* VALID: the call passes validation, so it may end at the device check (no GPU here)
 * or at the refusing launch stub (a GPU present), never elsewhere. */
#define VALID (-1)

static void expect(const char* what, forge_status got, int want, int line) {
  ++g_calls;
  int good = want == VALID ? (got == FORGE_ERR_DEVICE || got == FORGE_ERR_LAUNCH) : (int)got == want;
  if (good && got != FORGE_OK && forge_last_error()[0] == '\0') {
    fprintf(stderr, "line %d: %s: status %d but no message\n", line, what, (int)got);
    good = 0;
  }
  if (good && got == FORGE_OK && forge_last_error()[0] != '\0') {
    fprintf(stderr, "line %d: %s: FORGE_OK but message '%s'\n", line, what, forge_last_error());
    good = 0;
  }
  if (!good) {
    fprintf(stderr, "line %d: %s: got %d (%s: %s), want %d\n", line, what, (int)got, forge_status_string(got),
            forge_last_error(), want);
    ++g_fail;
  }
}
#define EXPECT(call, want) expect(#call, (call), (want), __LINE__)

/* fake device addresses, 1 TiB apart, 256-byte aligned */
static void* dev(int slot) { return (void*)(uintptr_t)(((uint64_t)(slot + 1)) << 40); }

static forge_tensor T(int slot, int32_t dt, int64_t r, int64_t c) {
  forge_tensor t;
  t.data = dev(slot);
  t.dtype = dt;
  t.rows = r;
  t.cols = c;
  t.ld = c;
  t.scale = NULL;
  return t;
}

static forge_hyper adam(void) {
  forge_hyper h;
  memset(&h, 0, sizeof h);
  h.lr = 1e-3f;
  h.beta1 = 0.9f;
  h.beta2 = 0.999f;
  h.eps = 1e-8f;
  h.weight_decay = 0.01f;
  h.momentum = 0.9f;
  h.alpha = 0.99f;
  h.momentum_decay = 4e-3f;
  return h;
}

static void* thread_body(void* arg) {
  /* forge_last_error is per thread: each thread sees the message of its own failure */
  const int k = (int)(intptr_t)arg;
  forge_hyper h = adam();
  float out[12];
  for (int i = 0; i < 2000; ++i) {
    forge_status s = forge_step_scalars(k ? 99 : FORGE_ADAMW, &h, k ? 1 : 0, out, 12);
    const char* want = k ? "unknown optimizer" : "step must be";
    if (s != FORGE_ERR_ARG || !strstr(forge_last_error(), want)) return (void*)1;
  }
  return NULL;
}

int main(void) {
  const int64_t N = 256, K = 384, Tk = 200;
  forge_hyper h = adam();
  forge_tensor X = T(0, FORGE_BF16, Tk, K), dY = T(1, FORGE_BF16, Tk, N), W = T(2, FORGE_BF16, N, K);
  forge_tensor m = T(3, FORGE_F32, N, K), v = T(4, FORGE_F32, N, K), dW = T(5, FORGE_F32, N, K);
  forge_tensor dX = T(6, FORGE_BF16, Tk, K);

  /* ---- fully valid calls end at the device check or the refusing stub */
  EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), VALID);
  EXPECT(forge_wgrad_gemm(&X, &dY, &dW, NULL), VALID);
  EXPECT(forge_optimizer_step(&dW, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), VALID);
  EXPECT(forge_dgrad(&dY, &W, &dX, NULL), VALID);
  EXPECT(forge_linear_backward_step(&X, &dY, &W, &dX, &m, &v, &h, FORGE_ADAMW, 3, 7, NULL, NULL), VALID);
  {
    void* ws = dev(7);
    const int64_t need = forge_backward_workspace_bytes(K);
    EXPECT(forge_linear_backward_step_fused(&X, &dY, &W, &dX, &m, &v, &h, FORGE_ADAMW, 3, 7, NULL, ws, need, NULL),
           VALID);
    EXPECT(forge_linear_backward_step_fused(&X, &dY, &W, &dX, &m, &v, &h, FORGE_ADAMW, 3, 7, NULL, ws, need - 1,
                                            NULL),
           FORGE_ERR_ARG);
    EXPECT(forge_linear_backward_step_fused(&X, &dY, &W, &dX, &m, &v, &h, FORGE_ADAMW, 3, 7, NULL, NULL, need, NULL),
           FORGE_ERR_ARG);
    EXPECT(forge_linear_backward_step_fused(&X, &dY, &W, &dX, &m, &v, &h, FORGE_ADAMW, 3, 7, NULL, W.data, need,
                                            NULL),
           FORGE_ERR_ALIAS);
    EXPECT(forge_linear_backward_step_fused(&X, &dY, &W, &dX, &m, &v, &h, FORGE_ADAMW, 3, 7, NULL, ws, INT64_MIN,
                                            NULL),
           FORGE_ERR_ARG);
    EXPECT(forge_linear_backward_step_fused_noalloc(&X, &dY, &W, &dX, &m, &v, &h, FORGE_ADAMW, 3, 7, NULL, NULL), VALID);
    if (forge_backward_workspace_bytes(-5) != -1 || forge_backward_workspace_bytes(INT64_MAX) != -1) {
      fprintf(stderr, "workspace size of a bad K\n");
      return 1;
    }
  }

  /* ---- NULL arguments */
  EXPECT(forge_wgrad_step(NULL, &dY, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_wgrad_step(&X, NULL, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_wgrad_step(&X, &dY, NULL, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_wgrad_step(&X, &dY, &W, NULL, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_wgrad_step(&X, &dY, &W, &m, NULL, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, NULL, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_wgrad_gemm(&X, &dY, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_optimizer_step(NULL, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_dgrad(NULL, &W, &dX, NULL), FORGE_ERR_ARG);
  EXPECT(forge_dgrad(&dY, NULL, &dX, NULL), FORGE_ERR_ARG);
  EXPECT(forge_dgrad(&dY, &W, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_linear_backward_step(&X, &dY, &W, NULL, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  {
    forge_tensor z = W;
    z.data = NULL;
    EXPECT(forge_wgrad_step(&X, &dY, &z, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  }
  /* a rule's state given or missing */
  EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, FORGE_SGD, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_wgrad_step(&X, &dY, &W, &m, NULL, &h, FORGE_LION, 1, 7, NULL, NULL), VALID);
  EXPECT(forge_wgrad_step(&X, &dY, &W, NULL, &v, &h, FORGE_RMSPROP, 1, 7, NULL, NULL), VALID);
  EXPECT(forge_wgrad_step(&X, &dY, &W, NULL, &v, &h, FORGE_LION, 1, 7, NULL, NULL), FORGE_ERR_ARG);

  /* ---- enums and step */
  const int32_t bad_opts[] = {-1, 8, 1000, INT32_MIN, INT32_MAX};
  for (size_t i = 0; i < sizeof bad_opts / sizeof bad_opts[0]; ++i)
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, bad_opts[i], 1, 7, NULL, NULL), FORGE_ERR_ARG);
  const int64_t bad_steps[] = {0, -1, INT64_MIN};
  for (size_t i = 0; i < sizeof bad_steps / sizeof bad_steps[0]; ++i)
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, FORGE_ADAMW, bad_steps[i], 7, NULL, NULL), FORGE_ERR_ARG);
  EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, FORGE_ADAMW, INT64_MAX, 7, NULL, NULL), VALID);
  EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, FORGE_NADAM, INT64_MAX, 7, NULL, NULL), VALID);
  EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, FORGE_RADAM, INT64_MAX, 7, NULL, NULL), VALID);
  {
    forge_hyper b = h;
    b.wd_mode = 3;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
    b.wd_mode = -1;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  }

  /* ---- hyper-parameters that give non-finite scalars; unused fields are ignored */
  {
    forge_hyper b = h;
    b.beta1 = 1.0f; /* outside [0, 1): a zero bias correction */
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
    b = h;
    b.lr = NAN;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
    b = h;
    b.lr = FLT_MAX;
    b.weight_decay = FLT_MAX; /* 1 - lr * wd overflows fp32 */
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
    b = h;
    b.momentum_decay = -1.0f;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_NADAM, 5, 7, NULL, NULL), FORGE_ERR_ARG);
    b = h;
    b.beta1 = NAN;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_NADAM, 5, 7, NULL, NULL), FORGE_ERR_ARG);
    b = h;
    b.eps = INFINITY;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
    b = h;
    b.beta1 = b.beta2 = b.eps = b.alpha = b.momentum = b.momentum_decay = NAN; /* SGD reads none of them */
    EXPECT(forge_wgrad_step(&X, &dY, &W, NULL, NULL, &b, FORGE_SGD, 1, 7, NULL, NULL), VALID);
    b = h;
    b.beta2 = 1.0f; /* RAdam: rho_inf infinite */
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &b, FORGE_RADAM, 1, 7, NULL, NULL), FORGE_ERR_ARG);
  }

  /* ---- dtypes, shapes, sizes */
  const int32_t bad_dt[] = {-1, 7, 1000, INT32_MIN};
  for (size_t i = 0; i < sizeof bad_dt / sizeof bad_dt[0]; ++i) {
    forge_tensor b = X;
    b.dtype = bad_dt[i];
    EXPECT(forge_wgrad_step(&b, &dY, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_DTYPE);
  }
  {
    forge_tensor b = X;
    b.dtype = FORGE_F32;
    EXPECT(forge_wgrad_step(&b, &dY, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_DTYPE);
    b = m;
    b.dtype = FORGE_BF16;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &b, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_DTYPE);
    b = W;
    b.dtype = FORGE_FP8_E4M3;
    EXPECT(forge_wgrad_step(&X, &dY, &b, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_DTYPE);
    EXPECT(forge_dgrad(&dY, &W, &dW, NULL), FORGE_ERR_DTYPE);
  }
  const int64_t huge[][2] = {{INT64_MAX, INT64_MAX}, {INT64_MAX, 2}, {(int64_t)1 << 40, (int64_t)1 << 40},
                             {(int64_t)1 << 62, 4}, {(int64_t)1 << 46, 1}, {-1, 5}, {5, INT64_MIN}};
  for (size_t i = 0; i < sizeof huge / sizeof huge[0]; ++i) {
    forge_tensor b = T(0, FORGE_F32, huge[i][0], huge[i][1]);
    const int want = FORGE_ERR_SHAPE;
    EXPECT(forge_wgrad_step(&b, &dY, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), want);
    EXPECT(forge_wgrad_gemm(&X, &b, &dW, NULL), want);
    EXPECT(forge_optimizer_step(&b, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), want);
    EXPECT(forge_dgrad(&b, &W, &dX, NULL), want);
    EXPECT(forge_dgrad(&dY, &b, &dX, NULL), want);
    EXPECT(forge_dgrad(&dY, &W, &b, NULL), want);
  }
  {
    /* large but representable: the kernels' 32-bit offsets refuse them */
    forge_tensor bx = T(0, FORGE_BF16, (int64_t)1 << 22, 1024), bd = T(1, FORGE_BF16, (int64_t)1 << 22, 256);
    EXPECT(forge_wgrad_step(&bx, &bd, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_SHAPE);
    forge_tensor bw = T(2, FORGE_BF16, 65536, 65536), bm = T(3, FORGE_F32, 65536, 65536), bv = T(4, FORGE_F32, 65536, 65536);
    forge_tensor by = T(1, FORGE_BF16, 8, 65536), bxx = T(0, FORGE_BF16, 8, 65536);
    EXPECT(forge_wgrad_step(&bxx, &by, &bw, &bm, &bv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_SHAPE);
    forge_tensor dy2 = T(1, FORGE_BF16, (int64_t)1 << 30, 128), dx2 = T(6, FORGE_BF16, (int64_t)1 << 30, 128);
    forge_tensor w2 = T(2, FORGE_BF16, 128, 128);
    EXPECT(forge_dgrad(&dy2, &w2, &dx2, NULL), FORGE_ERR_SHAPE);
  }
  {
    forge_tensor b = W;
    b.rows = 200;
    EXPECT(forge_wgrad_step(&X, &dY, &b, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_SHAPE);
    forge_tensor x2 = T(0, FORGE_BF16, Tk, 200), y2 = T(1, FORGE_BF16, Tk, N), w2 = T(2, FORGE_BF16, N, 200);
    forge_tensor m2 = T(3, FORGE_F32, N, 200), v2 = T(4, FORGE_F32, N, 200);
    EXPECT(forge_wgrad_step(&x2, &y2, &w2, &m2, &v2, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_SHAPE);
    forge_tensor y3 = T(1, FORGE_BF16, Tk + 1, N);
    EXPECT(forge_wgrad_step(&X, &y3, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_SHAPE);
    b = m;
    b.cols = 128;
    b.ld = 128;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &b, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_SHAPE);
  }

  /* ---- layout: stride and alignment */
  {
    forge_tensor b = X;
    b.ld = K + 8;
    EXPECT(forge_wgrad_step(&b, &dY, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_LAYOUT);
    b = W;
    b.data = (char*)dev(2) + 2;
    EXPECT(forge_wgrad_step(&X, &dY, &b, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_LAYOUT);
    forge_step_opts o = {(float*)((char*)dev(7) + 4), 1};
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, &o, NULL), FORGE_ERR_LAYOUT);
  }

  /* ---- 8-bit moments: formats, maps, scales */
  {
    forge_tensor qm = T(3, FORGE_I8_B64, N, K), qv = T(4, FORGE_U8_B64, N, K);
    qm.scale = dev(8);
    qv.scale = dev(9);
    EXPECT(forge_wgrad_step(&X, &dY, &W, &qm, &qv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), VALID);
    forge_tensor dm = qm, dv = qv;
    dm.dtype = FORGE_I8DYN_B64;
    dv.dtype = FORGE_U8DYN_B64;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &dm, &dv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), VALID);
    EXPECT(forge_wgrad_step(&X, &dY, &W, &qm, &dv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_DTYPE);
    EXPECT(forge_wgrad_step(&X, &dY, &W, &qm, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_DTYPE);
    EXPECT(forge_wgrad_step(&X, &dY, &W, &qv, &qm, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_DTYPE);
    forge_tensor b = qm;
    b.scale = NULL;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &b, &qv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
    b.scale = (char*)dev(8) + 2;
    EXPECT(forge_wgrad_step(&X, &dY, &W, &b, &qv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_LAYOUT);
    b.scale = (char*)dev(4) + 16; /* inside v's codes */
    EXPECT(forge_wgrad_step(&X, &dY, &W, &b, &qv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ALIAS);
    forge_tensor fx = T(0, FORGE_FP8_E4M3, Tk, K), fy = T(1, FORGE_FP8_E4M3, Tk, N);
    EXPECT(forge_wgrad_step(&fx, &fy, &W, &qm, &qv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ARG);
    fx.scale = dev(10);
    fy.scale = (char*)dev(10) + 4;
    EXPECT(forge_wgrad_step(&fx, &fy, &W, &qm, &qv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), VALID);
    fy.scale = (char*)dev(10) + 1;
    EXPECT(forge_wgrad_step(&fx, &fy, &W, &qm, &qv, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_LAYOUT);
  }

  /* ---- aliasing */
  {
    forge_tensor b = m;
    b.data = (char*)dev(2) + 256; /* inside W */
    EXPECT(forge_wgrad_step(&X, &dY, &W, &b, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ALIAS);
    b = W;
    b.data = dev(0); /* W on top of X */
    EXPECT(forge_wgrad_step(&X, &dY, &b, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ALIAS);
    forge_step_opts o = {(float*)dev(3), 1}; /* preround buffer on m */
    EXPECT(forge_wgrad_step(&X, &dY, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, &o, NULL), FORGE_ERR_ALIAS);
    b = dW;
    b.data = dev(1);
    EXPECT(forge_wgrad_gemm(&X, &dY, &b, NULL), FORGE_ERR_ALIAS);
    EXPECT(forge_optimizer_step(&b, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), VALID);
    b.data = dev(2);
    EXPECT(forge_optimizer_step(&b, &W, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ALIAS);
    b = dX;
    b.data = dev(1);
    EXPECT(forge_dgrad(&dY, &W, &b, NULL), FORGE_ERR_ALIAS);
    b.data = dev(3); /* dX on m: the backward step refuses before enqueueing dgrad */
    EXPECT(forge_linear_backward_step(&X, &dY, &W, &b, &m, &v, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_ALIAS);
  }

  /* ---- empty problems return before any device call */
  {
    forge_tensor x0 = T(0, FORGE_BF16, Tk, 0), w0 = T(2, FORGE_BF16, N, 0), m0 = T(3, FORGE_F32, N, 0),
                 v0 = T(4, FORGE_F32, N, 0);
    EXPECT(forge_wgrad_step(&x0, &dY, &w0, &m0, &v0, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_OK);
    forge_tensor d0 = T(5, FORGE_F32, 0, 0);
    EXPECT(forge_optimizer_step(&d0, &w0, &m0, &v0, &h, FORGE_ADAMW, 1, 7, NULL, NULL), FORGE_ERR_SHAPE);
    forge_tensor dy0 = T(1, FORGE_BF16, 0, N), dx0 = T(6, FORGE_BF16, 0, K);
    EXPECT(forge_dgrad(&dy0, &W, &dx0, NULL), FORGE_OK);
  }

  /* ---- host-only helpers */
  {
    float* out = (float*)malloc(12 * sizeof(float)); /* exactly the 12 scalars: no write past them */
    for (int opt = FORGE_ADAMW; opt <= FORGE_SGD_MOMENTUM; ++opt) {
      EXPECT(forge_step_scalars(opt, &h, 1, out, 1000), FORGE_OK);
      EXPECT(forge_step_scalars(opt, &h, INT64_MAX, out, 12), FORGE_OK);
      EXPECT(forge_step_scalars(opt, &h, 3, out, 0), FORGE_OK);
      EXPECT(forge_step_scalars(opt, &h, 3, NULL, 0), FORGE_OK);
      EXPECT(forge_step_scalars(opt, &h, 3, NULL, 4), FORGE_ERR_ARG);
      EXPECT(forge_step_scalars(opt, &h, 3, out, -5), FORGE_OK);
    }
    free(out);
    for (int s = -3; s < 12; ++s)
      if (!forge_status_string((forge_status)s) || !forge_status_string((forge_status)s)[0]) ++g_fail;
    if (forge_version() <= 0) ++g_fail;
    const char* id = forge_build_id();
    if (!id || !id[0]) ++g_fail;
    EXPECT(forge_device_check(-1), FORGE_ERR_DEVICE);
    EXPECT(forge_device_check(1 << 20), FORGE_ERR_DEVICE);
    EXPECT(forge_device_check(INT32_MIN), FORGE_ERR_DEVICE);
  }

  /* ---- per-thread error text */
  {
    pthread_t th[2];
    void* r[2] = {NULL, NULL};
    for (int k = 0; k < 2; ++k) pthread_create(&th[k], NULL, thread_body, (void*)(intptr_t)k);
    for (int k = 0; k < 2; ++k) pthread_join(th[k], &r[k]);
    if (r[0] || r[1]) {
      fprintf(stderr, "forge_last_error is not per thread\n");
      ++g_fail;
    }
  }

  if (forge_stub_launches() != 0 && forge_device_check(0) != FORGE_OK) {
    fprintf(stderr, "a launcher was reached without a device\n");
    ++g_fail;
  }
  printf("abi_driver: %d calls, %d failures, %d stub launches\n", g_calls, g_fail, forge_stub_launches());
  return g_fail ? 1 : 0;
}
