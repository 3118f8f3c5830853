/* A C caller of the HIP path with no Python in the process: device buffers
 * from hipMalloc, conv2d_grad_input and conv2d_forward through the C ABI on
 * a stream of the caller's own, each compared with the oracle's definition
 * (oracle/oracle.c, linked in) at the fp32 bar, max|gpu - oracle| /
 * max|oracle| <= 1e-4.  Built and run by tests/test_c_abi_from_c.py on a GPU;
 * exit status 0 when both match. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "conv2d_bwd.h"

void oracle_grad_input_gather(const double* go, const double* w, double* gi, int64_t N,
                              int64_t Ci, int64_t H, int64_t W, int64_t Co, int64_t KH,
                              int64_t KW, int64_t s, int64_t ph, int64_t pw, int64_t OH,
                              int64_t OW);
void oracle_conv2d_forward(const double* x, const double* w, double* y, int64_t N,
                           int64_t Ci, int64_t H, int64_t W, int64_t Co, int64_t KH,
                           int64_t KW, int64_t s, int64_t ph, int64_t pw, int64_t OH,
                           int64_t OW);

/* xorshift64 values in [-1, 1) */
static uint64_t rng_state = 88172645463325252ull;
static double draw(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return (double)(rng_state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static void fill(float* f, double* d, size_t n) {
  size_t i;
  for (i = 0; i < n; ++i) {
    f[i] = (float)draw();
    d[i] = f[i];
  }
}

static double rel_err(const float* got, const double* ref, size_t n) {
  double worst = 0.0, scale = 1e-30;
  size_t i;
  for (i = 0; i < n; ++i) {
    const double e = fabs((double)got[i] - ref[i]);
    if (!(e <= worst)) worst = e; /* NaN propagates */
    if (fabs(ref[i]) > scale) scale = fabs(ref[i]);
  }
  return worst / scale;
}

#define HIP_OK(call)                                      \
  do {                                                    \
    if ((call) != hipSuccess) {                           \
      printf("hip failure at line %d\n", __LINE__);       \
      return 2;                                           \
    }                                                     \
  } while (0)

int main(void) {
  /* stride 2, a 3x3 kernel, ragged channels and pixels: four classes */
  const conv2d_params p = {2, 9, 13, 11, 7, 3, 3, 2, 1, 1, 7, 6};
  const size_t n_go = (size_t)p.batch * p.out_channels * p.out_h * p.out_w;
  const size_t n_w = (size_t)p.out_channels * p.in_channels * p.kernel_h * p.kernel_w;
  const size_t n_gi = (size_t)p.batch * p.in_channels * p.in_h * p.in_w;
  float *go = malloc(n_go * 4), *w = malloc(n_w * 4), *gi = malloc(n_gi * 4);
  float *x = malloc(n_gi * 4), *y = malloc(n_go * 4);
  double *go64 = malloc(n_go * 8), *w64 = malloc(n_w * 8), *gi_ref = malloc(n_gi * 8);
  double *x64 = malloc(n_gi * 8), *y_ref = malloc(n_go * 8);
  float *d_go, *d_w, *d_gi, *d_x, *d_y;
  hipStream_t st;
  int rc_gi, rc_fwd;
  double err_gi, err_fwd;
  if (!go || !w || !gi || !x || !y || !go64 || !w64 || !gi_ref || !x64 || !y_ref) return 2;
  fill(go, go64, n_go);
  fill(w, w64, n_w);
  fill(x, x64, n_gi);

  HIP_OK(hipStreamCreate(&st));
  HIP_OK(hipMalloc((void**)&d_go, n_go * 4));
  HIP_OK(hipMalloc((void**)&d_w, n_w * 4));
  HIP_OK(hipMalloc((void**)&d_gi, n_gi * 4));
  HIP_OK(hipMalloc((void**)&d_x, n_gi * 4));
  HIP_OK(hipMalloc((void**)&d_y, n_go * 4));
  HIP_OK(hipMemcpy(d_go, go, n_go * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w, n_w * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, x, n_gi * 4, hipMemcpyHostToDevice));

  rc_gi = conv2d_grad_input(d_go, d_w, d_gi, &p, st);
  rc_fwd = conv2d_forward(d_x, d_w, d_y, &p, st);
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipMemcpy(gi, d_gi, n_gi * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(y, d_y, n_go * 4, hipMemcpyDeviceToHost));

  oracle_grad_input_gather(go64, w64, gi_ref, p.batch, p.in_channels, p.in_h, p.in_w,
                           p.out_channels, p.kernel_h, p.kernel_w, p.stride, p.padding_h,
                           p.padding_w, p.out_h, p.out_w);
  oracle_conv2d_forward(x64, w64, y_ref, p.batch, p.in_channels, p.in_h, p.in_w,
                        p.out_channels, p.kernel_h, p.kernel_w, p.stride, p.padding_h,
                        p.padding_w, p.out_h, p.out_w);
  err_gi = rel_err(gi, gi_ref, n_gi);
  err_fwd = rel_err(y, y_ref, n_go);
  printf("grad_input %d %.3e\n", rc_gi, err_gi);
  printf("forward %d %.3e\n", rc_fwd, err_fwd);

  HIP_OK(hipFree(d_go));
  HIP_OK(hipFree(d_w));
  HIP_OK(hipFree(d_gi));
  HIP_OK(hipFree(d_x));
  HIP_OK(hipFree(d_y));
  HIP_OK(hipStreamDestroy(st));
  free(go); free(w); free(gi); free(x); free(y);
  free(go64); free(w64); free(gi_ref); free(x64); free(y_ref);
  return (rc_gi == 0 && rc_fwd == 0 && err_gi <= 1e-4 && err_fwd <= 1e-4) ? 0 : 1;
}
