/*
 * Host-side checks of the C ABI's validation code under AddressSanitizer (built with the
 * host part of libdconv1d instrumented; no GPU needed and none used): every compute entry
 * point is called with arguments that fail validation, or with an empty batch, from
 * several threads at once, and the status codes and per-thread messages are checked.
 * No call here reaches a kernel launch: each one is rejected or is a no-op before any
 * device work, so it is safe whether or not a GPU is present. Exit status 0 when every
 * check passes; the sanitizer aborts with a report on any memory error.
 */
#include <pthread.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dconv1d.h"

#define X ((const float*)0x10000000)
#define OUT ((float*)0x20000000)
#define P ((const float*)0x30000000)
#define RM ((float*)0x40000000)
#define RV ((float*)0x40001000)
#define RES ((const float*)0x50000000)

static int failures;
static pthread_mutex_t mu = PTHREAD_MUTEX_INITIALIZER;

static void expect(int got, int want, const char* what) {
  const char* msg = dconv1d_last_error();
  int bad = got != want || (want != DCONV1D_OK && (msg == NULL || msg[0] == '\0')) ||
            (want == DCONV1D_OK && msg != NULL && msg[0] != '\0');
  if (bad) {
    pthread_mutex_lock(&mu);
    fprintf(stderr, "%s: got %d want %d (message '%s')\n", what, got, want, msg ? msg : "(null)");
    ++failures;
    pthread_mutex_unlock(&mu);
  }
}

typedef int (*block_fn)(const float*, const float*, const float*, const float*, const float*,
                        float, const float*, const float*, float*, int64_t, int64_t, int64_t,
                        int64_t, hipStream_t);

static void block_cases(block_fn fn, const char* name, int elem) {
  char what[128];
  struct { const float* x; float* out; const float* W; const float* rm; int64_t N, C, L, d;
           float eps; int code; } c[] = {
    {NULL, OUT, P, P, 2, 16, 512, 128, 1e-5f, DCONV1D_EINVAL},
    {X, NULL, P, P, 2, 16, 512, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, NULL, P, 2, 16, 512, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, NULL, 2, 16, 512, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, P, -1, 16, 512, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, P, 2, 0, 512, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, P, 2, 16, 0, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, P, 2, 16, 512, 0, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, P, 2, 16, 512, 128, -1.f, DCONV1D_EINVAL},
    {X, OUT, P, P, 2, 100000, 512, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, P, 2, 16384, 1 << 18, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, P, 2, 16, (int64_t)1 << 40, 128, 1e-5f, DCONV1D_EINVAL},
    {X, OUT, P, P, (int64_t)1 << 62, 16, 512, 128, 1e-5f, DCONV1D_EINVAL},
    {X, (float*)X, P, P, 2, 16, 512, 128, 1e-5f, DCONV1D_EALIAS},
    {X, (float*)((const char*)X + elem * 2 * 16 * 512 - elem), P, P, 2, 16, 512, 128, 1e-5f,
     DCONV1D_EALIAS},
    {X, OUT, P, P, 0, 16, 512, 128, 1e-5f, DCONV1D_OK},
    {NULL, NULL, P, P, 0, 16, 512, 128, 1e-5f, DCONV1D_OK},
  };
  for (size_t i = 0; i < sizeof(c) / sizeof(c[0]); ++i) {
    snprintf(what, sizeof(what), "%s case %zu", name, i);
    expect(fn(c[i].x, c[i].rm, P, P, P, c[i].eps, c[i].W, P, c[i].out, c[i].N, c[i].C, c[i].L,
              c[i].d, 0),
           c[i].code, what);
  }
}

static void other_cases(void) {
  /* training mode */
  expect(prenorm_dconv1d_fwd_train(X, RM, NULL, P, P, 1e-5f, 0.1f, P, NULL, OUT, NULL, NULL, 2,
                                   16, 512, 128, 0), DCONV1D_EINVAL, "train one running NULL");
  expect(prenorm_dconv1d_fwd_train(X, RM, RV, P, P, 1e-5f, 1.f / 0.f, P, NULL, OUT, NULL, NULL,
                                   2, 16, 512, 128, 0), DCONV1D_EINVAL, "train momentum inf");
  expect(prenorm_dconv1d_fwd_train(X, RM, RV, P, P, 1e-5f, 0.1f, P, NULL, OUT, NULL, NULL, 1,
                                   16, 1, 128, 0), DCONV1D_EINVAL, "train one value");
  expect(prenorm_dconv1d_fwd_train(X, (float*)((char*)OUT + 64), RV, P, P, 1e-5f, 0.1f, P, NULL,
                                   OUT, NULL, NULL, 2, 16, 512, 128, 0), DCONV1D_EALIAS,
         "train running_mean overlaps out");
  expect(prenorm_dconv1d_fwd_train_bf16((const uint16_t*)X, RM, RV, P, P, 1e-5f, 0.1f, P, NULL,
                                        (uint16_t*)OUT, (float*)X, NULL, 2, 16, 512, 128, 0),
         DCONV1D_EALIAS, "train bf16 save_mean overlaps x");
  expect(prenorm_dconv1d_fwd_train(NULL, NULL, NULL, P, P, 1e-5f, 0.1f, P, NULL, NULL, NULL,
                                   NULL, 0, 16, 512, 128, 0), DCONV1D_OK, "train empty batch");
  /* caller-normalised */
  expect(relu_dconv1d_residual_fwd(X, P, NULL, NULL, OUT, 2, 16, 512, 128, 0), DCONV1D_EINVAL,
         "external residual NULL");
  expect(relu_dconv1d_residual_fwd(X, P, NULL, RES, (float*)((const char*)RES + 64), 2, 16, 512,
                                   128, 0), DCONV1D_EALIAS, "external shifted residual");
  expect(relu_dconv1d_residual_fwd_bf16((const uint16_t*)X, P, NULL, (const uint16_t*)RES,
                                        (uint16_t*)X, 2, 16, 512, 128, 0), DCONV1D_EALIAS,
         "external bf16 out overlaps xn");
  expect(relu_dconv1d_residual_fwd(X, P, NULL, RES, (float*)RES, 0, 16, 512, 128, 0), DCONV1D_OK,
         "external in-place empty batch");
  /* Conv1d + GroupNorm */
  expect(conv1d_groupnorm_fwd(X, P, NULL, NULL, NULL, 1e-5f, 3, OUT, 16, 128, 256, 1024, 1, 1,
                              0), DCONV1D_EINVAL, "gn groups do not divide");
  expect(conv1d_groupnorm_fwd(X, P, NULL, NULL, NULL, 1e-5f, 32, OUT, 16, 128, 256, 4, 0, 2, 0),
         DCONV1D_EINVAL, "gn empty output");
  expect(conv1d_groupnorm_fwd(X, P, NULL, NULL, NULL, 1e-5f, 32, OUT, 16, 128, 256,
                              (int64_t)1 << 35, 1, 1, 0), DCONV1D_EINVAL, "gn huge T");
  expect(conv1d_groupnorm_fwd(X, P, NULL, NULL, NULL, 1e-5f, 32, (float*)((const char*)X + 1024),
                              16, 128, 256, 1024, 1, 1, 0), DCONV1D_EALIAS, "gn out overlaps x");
  expect(conv1d_groupnorm_fwd(NULL, P, NULL, NULL, NULL, 1e-5f, 32, NULL, 0, 128, 256, 1024, 1,
                              1, 0), DCONV1D_OK, "gn empty batch");
}

static void* worker(void* arg) {
  (void)arg;
  for (int rep = 0; rep < 20; ++rep) {
    block_cases(prenorm_dconv1d_fwd, "prenorm_dconv1d_fwd", 4);
    block_cases(prenorm_dconv1d_fwd_noalloc, "prenorm_dconv1d_fwd_noalloc", 4);
    block_cases((block_fn)prenorm_dconv1d_fwd_bf16, "prenorm_dconv1d_fwd_bf16", 2);
    other_cases();
  }
  return NULL;
}

int main(void) {
  enum { NT = 4 };
  pthread_t th[NT];
  for (int i = 0; i < NT; ++i) pthread_create(&th[i], NULL, worker, NULL);
  for (int i = 0; i < NT; ++i) pthread_join(th[i], NULL);
  /* a message outlives the call that set it and is cleared by the next one */
  expect(prenorm_dconv1d_fwd(X, P, P, P, P, 1e-5f, P, P, OUT, 2, 0, 512, 128, 0), DCONV1D_EINVAL,
         "message set");
  if (strstr(dconv1d_last_error(), "C must be") == NULL) {
    fprintf(stderr, "unexpected message '%s'\n", dconv1d_last_error());
    ++failures;
  }
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi_asan: all checks passed\n");
  return 0;
}
