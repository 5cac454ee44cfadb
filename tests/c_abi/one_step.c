/* One MuonH step driven through the C ABI alone (include/muonh.h and the
 * HIP runtime for device memory; no Python, no torch).  A 300 x 200 fp32
 * weight (tall: Newton-Schulz runs on its transpose) with an fp32 gradient,
 * the fp32 Newton-Schulz path, one step at eta = 0.01.  Checks what Eq. (1)
 * of the Hyperball update fixes exactly: ||W_1||_F = R = ||W_0||_F, and the
 * pre-projection displacement ||W~ - W_0|| / ||W_0|| = eta, reported as the
 * effective LR in the statistics; plus the angle between W_0 and W_1,
 * measured by the chord 2 asin(||W_1 - W_0|| / 2R), against the closed form
 * atan2(eta sqrt(1 - c^2), 1 - eta c).
 * Prints "ok" and exits 0 on success. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "muonh.h"

#define R_ 300
#define C_ 200

static unsigned long long state = 0x9e3779b97f4a7c15ull;
static double uniform01(void) {   /* splitmix64 */
  unsigned long long z = (state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  z ^= z >> 31;
  return (double)(z >> 11) / 9007199254740992.0;
}

static int fail(const char* what) {
  fprintf(stderr, "one_step: %s (%s)\n", what, muonh_last_error());
  return 1;
}

int main(void) {
  const size_t n = (size_t)R_ * C_;
  float* hw = (float*)malloc(n * sizeof(float));
  float* hg = (float*)malloc(n * sizeof(float));
  float* hw1 = (float*)malloc(n * sizeof(float));
  if (!hw || !hg || !hw1) return fail("host allocation");
  for (size_t i = 0; i < n; ++i) {
    hw[i] = (float)(2.0 * uniform01() - 1.0);
    hg[i] = (float)(2.0 * uniform01() - 1.0);
  }
  void *w = NULL, *g = NULL, *m = NULL;
  if (hipMalloc(&w, n * 4) != hipSuccess || hipMalloc(&g, n * 4) != hipSuccess ||
      hipMalloc(&m, n * 4) != hipSuccess)
    return fail("hipMalloc");
  if (hipMemcpy(w, hw, n * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(g, hg, n * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(m, 0, n * 4) != hipSuccess)
    return fail("upload");

  muonh_matrix_desc d;
  memset(&d, 0, sizeof(d));
  d.w = w; d.g = g; d.m = m; d.rows = R_; d.cols = C_; d.g_dtype = MUONH_F32; d.radius = 0.0f;
  muonh_options o;
  muonh_default_options(&o);
  o.ns_dtype = MUONH_F32;
  muonh_handle* h = NULL;
  if (muonh_init(&h, &d, 1, &o, NULL) != MUONH_OK) return fail("muonh_init");
  const float eta = 0.01f;
  muonh_step_args a;
  memset(&a, 0, sizeof(a));
  a.elr = eta;
  if (muonh_step(h, &d, 1, &a, NULL) != MUONH_OK) return fail("muonh_step");
  float radius = 0.0f;
  muonh_stats st;
  if (muonh_get_radii(h, &radius, 1) != MUONH_OK) return fail("muonh_get_radii");
  if (muonh_get_stats(h, &st, 1) != MUONH_OK) return fail("muonh_get_stats");
  if (hipMemcpy(hw1, w, n * 4, hipMemcpyDeviceToHost) != hipSuccess) return fail("download");
  muonh_destroy(h);
  hipFree(w); hipFree(g); hipFree(m);

  double n0 = 0.0, n1 = 0.0, dd = 0.0;
  for (size_t i = 0; i < n; ++i) {
    const double e = (double)hw1[i] - hw[i];
    n0 += (double)hw[i] * hw[i];
    n1 += (double)hw1[i] * hw1[i];
    dd += e * e;
  }
  n0 = sqrt(n0); n1 = sqrt(n1);
  /* angle from the chord (stable for small angles, unlike acos of a dot) */
  const double angle = 2.0 * asin(sqrt(dd) / (2.0 * radius));
  const double closed = atan2(eta * sqrt(fmax(0.0, 1.0 - st.c * st.c)), 1.0 - eta * st.c);
  printf("R %.6f |W0| %.6f |W1| %.6f elr %.8f angle %.8f closed %.8f nonfinite %d\n",
         radius, n0, n1, st.elr, angle, closed, st.nonfinite);
  if (fabs(radius / n0 - 1.0) > 1e-6) return fail("R != ||W_0||");
  if (fabs(n1 / radius - 1.0) > 1e-5) return fail("||W_1|| != R");
  if (fabs(st.elr / eta - 1.0) > 1e-5) return fail("effective LR != eta");
  if (fabs(angle - closed) > 1e-4 * eta) return fail("angle differs from the closed form");
  if (st.nonfinite) return fail("non-finite statistics");
  printf("ok\n");
  free(hw); free(hg); free(hw1);
  return 0;
}
