/*
 * Plain C client of the C ABI in include/dconv1d.h (no Python, no C++): it uploads one
 * pre-norm block problem, runs prenorm_dconv1d_fwd and prenorm_dconv1d_fwd_train on the
 * null stream, checks two rejected calls (DCONV1D_EINVAL, DCONV1D_EALIAS) and the error
 * message, and writes the results for a caller to compare with a reference.
 *
 *   dconv1d_client IN OUT
 *
 * IN  (little-endian): int64 N, C, L, d; float32 eps, momentum; then float32 arrays
 *     x[N*C*L], running_mean[C], running_var[C], gamma[C], beta[C], W[C*C*3], b[C].
 * OUT: float32 out[N*C*L] (eval-mode BN), out_train[N*C*L], running_mean'[C],
 *     running_var'[C] (after one training-mode update).
 * Exit status 0 on success; a message on stderr otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dconv1d.h"

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));       \
      return 2;                                                               \
    }                                                                         \
  } while (0)

static int read_all(FILE* f, void* dst, size_t bytes) {
  return fread(dst, 1, bytes, f) == bytes ? 0 : -1;
}

static float* upload(const float* h, size_t n) {
  float* d = NULL;
  if (hipMalloc((void**)&d, n * sizeof(float) + 4) != hipSuccess) return NULL;
  if (n && hipMemcpy(d, h, n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", argv[1]);
    return 2;
  }
  int64_t dims[4];
  float par[2];
  if (read_all(f, dims, sizeof dims) || read_all(f, par, sizeof par)) {
    fprintf(stderr, "short header\n");
    return 2;
  }
  const int64_t N = dims[0], C = dims[1], L = dims[2], d = dims[3];
  const size_t nx = (size_t)(N * C * L), nw = (size_t)(C * C * 3), nc = (size_t)C;
  float* h = (float*)malloc((nx + 5 * nc + nw) * sizeof(float));
  if (!h || read_all(f, h, (nx + 5 * nc + nw) * sizeof(float))) {
    fprintf(stderr, "short input\n");
    return 2;
  }
  fclose(f);
  const float* hx = h;
  const float* hrm = hx + nx;
  const float* hrv = hrm + nc;
  const float* hg = hrv + nc;
  const float* hb = hg + nc;
  const float* hW = hb + nc;
  const float* hbias = hW + nw;

  float *x = upload(hx, nx), *rm = upload(hrm, nc), *rv = upload(hrv, nc);
  float *g = upload(hg, nc), *be = upload(hb, nc), *W = upload(hW, nw), *bias = upload(hbias, nc);
  float *out = upload(hx, nx), *out_t = upload(hx, nx);
  if (!x || !rm || !rv || !g || !be || !W || !bias || !out || !out_t) {
    fprintf(stderr, "device allocation failed\n");
    return 2;
  }

  int st = prenorm_dconv1d_fwd(x, rm, rv, g, be, par[0], W, bias, out, N, C, L, d, NULL);
  if (st != DCONV1D_OK) {
    fprintf(stderr, "prenorm_dconv1d_fwd: %d %s\n", st, dconv1d_last_error());
    return 1;
  }
  st = prenorm_dconv1d_fwd_train(x, rm, rv, g, be, par[0], par[1], W, bias, out_t, NULL, NULL,
                                 N, C, L, d, NULL);
  if (st != DCONV1D_OK) {
    fprintf(stderr, "prenorm_dconv1d_fwd_train: %d %s\n", st, dconv1d_last_error());
    return 1;
  }
  /* rejected calls: validated on the host, nothing is launched */
  st = prenorm_dconv1d_fwd(x, rm, rv, g, be, par[0], W, bias, out, N, 0, L, d, NULL);
  if (st != DCONV1D_EINVAL || strlen(dconv1d_last_error()) == 0) {
    fprintf(stderr, "C = 0 returned %d (%s), expected DCONV1D_EINVAL\n", st, dconv1d_last_error());
    return 1;
  }
  st = prenorm_dconv1d_fwd(x, rm, rv, g, be, par[0], W, bias, x, N, C, L, d, NULL);
  if (st != DCONV1D_EALIAS) {
    fprintf(stderr, "out == x returned %d, expected DCONV1D_EALIAS\n", st);
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());

  float* res = (float*)malloc((2 * nx + 2 * nc) * sizeof(float));
  if (!res) return 2;
  HIP_OK(hipMemcpy(res, out, nx * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(res + nx, out_t, nx * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(res + 2 * nx, rm, nc * sizeof(float), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(res + 2 * nx + nc, rv, nc * sizeof(float), hipMemcpyDeviceToHost));
  FILE* o = fopen(argv[2], "wb");
  if (!o || fwrite(res, sizeof(float), 2 * nx + 2 * nc, o) != 2 * nx + 2 * nc) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 2;
  }
  fclose(o);
  dconv1d_release();
  hipFree(x); hipFree(rm); hipFree(rv); hipFree(g); hipFree(be); hipFree(W); hipFree(bias);
  hipFree(out); hipFree(out_t);
  free(h);
  free(res);
  return 0;
}
