/*
 * The library used from plain C: device memory from the HIP runtime, the
 * entry points of qknorm.h, no Python or torch anywhere.
 *
 * Inputs are chosen so that every expected value has a closed form.  With
 * eps = 0, a group of width n holding k nonzeros of equal magnitude m has sum
 * of squares k*m^2, mean square k*m^2/n, and normalises to
 * gamma_j * sign_j * sqrt(n/k) on the nonzeros and 0 elsewhere (RMSNorm as
 * defined on the SwiftQK verdict page, core discovery; per head n = head_dim,
 * layerwise n = the whole Q or K width, SwiftQK summary page, Abstract).
 * Powers of two for m, gamma with two significant bits and power-of-two widths
 * keep every fp32 step exact except the reciprocal square root, so each bf16
 * output is within one bf16 ulp of the closed form.
 *
 * Also: validation codes returned before any HIP call, the fused layerwise
 * call equal, byte for byte, to partial sums then apply, and the QKV
 * projection with a weight that selects columns of x (each output one exact
 * product), so its Q and K heads take the closed form of the norm and its V
 * heads copy x; the three projection calls (no workspace, a workspace, the
 * library's scratch) give the same bytes.
 *
 * Exit status 0 when every check passes; the first failure is printed.
 * With --validation-only it stops after the checks that need no GPU.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qknorm.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));            \
      return 1;                                                             \
    }                                                                       \
  } while (0)

#define EXPECT(cond, ...)                                                   \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, __VA_ARGS__);                                         \
      fputc('\n', stderr);                                                  \
      return 1;                                                             \
    }                                                                       \
  } while (0)

/* bf16 <-> float: the bf16 pattern is the high half of the fp32 pattern;
 * every value built here is exactly representable, so no rounding is needed */
static uint16_t to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* gamma_j = 1 + (j % 4) / 4: 1, 1.25, 1.5, 1.75 */
static float gamma_at(int j) { return 1.0f + (float)(j % 4) * 0.25f; }

/* one group: k = 1 + key % n nonzeros of magnitude 2^(key % 9 - 4), signs
 * alternating, written to x[0..n) */
static int fill_group(uint16_t* x, int n, unsigned key) {
  const int k = 1 + (int)(key % (unsigned)n);
  const float m = ldexpf(1.0f, (int)(key % 9u) - 4);
  for (int j = 0; j < n; ++j) x[j] = to_bf16(j < k ? ((j & 1) ? -m : m) : 0.0f);
  return k;
}

/* checks one normalised group against gamma * sign * sqrt(n/k) */
static int check_group(const uint16_t* y, int n, int k, const char* what, long where) {
  const double r = sqrt((double)n / (double)k);
  for (int j = 0; j < n; ++j) {
    const double got = from_bf16(y[j]);
    if (j >= k) {
      EXPECT(got == 0.0, "%s %ld: element %d should be 0, got %g", what, where, j, got);
      continue;
    }
    const double want = (double)gamma_at(j) * ((j & 1) ? -r : r);
    EXPECT(fabs(got - want) <= 8e-3 * fabs(want), "%s %ld: element %d = %.9g, closed form %.9g", what,
           where, j, got, want);
  }
  return 0;
}

static int validation(void) {
  /* returned before any HIP call */
  _Alignas(16) uint16_t g[128] = {0};
  EXPECT(qknorm_abi_version() == QKNORM_ABI_VERSION, "ABI version %d", qknorm_abi_version());
  EXPECT(qknorm_per_head(NULL, 4, 128, 1, 0, 128, g, NULL, 1e-6f, QKNORM_BF16, NULL) == QKNORM_E_NULLPTR,
         "NULL qkv not rejected");
  EXPECT(qknorm_per_head(NULL, 0, 128, 1, 0, 128, NULL, NULL, 1e-6f, QKNORM_BF16, NULL) == QKNORM_OK,
         "T = 0 must be a no-op");
  EXPECT(qknorm_per_head((void*)g, -1, 128, 1, 0, 128, g, NULL, 1e-6f, QKNORM_BF16, NULL) == QKNORM_E_SHAPE,
         "negative T not rejected");
  EXPECT(qknorm_per_head((void*)g, 4, 128, 1, 0, 128, g, NULL, -1.0f, QKNORM_BF16, NULL) == QKNORM_E_EPS,
         "negative eps not rejected");
  EXPECT(qknorm_per_head((void*)g, 4, 128, 1, 0, 128, g, NULL, 1e-6f, 9, NULL) == QKNORM_E_DTYPE,
         "unknown dtype not rejected");
  EXPECT(qknorm_layerwise((void*)g, 4, 128, 96, 32, g, g, 1e-6f, 5, QKNORM_BF16, NULL) == QKNORM_E_SHAPE,
         "a shard count that does not divide the widths not rejected");
  for (int c = QKNORM_E_HIP; c <= QKNORM_OK; ++c)
    EXPECT(qknorm_strerror(c) != NULL && qknorm_strerror(c)[0] != '\0', "no text for code %d", c);
  EXPECT(qknorm_qkv_proj_workspace_bytes(1, 32, 8, 128) == 4 * 6144 * 4, "workspace bytes at T = 1");
  EXPECT(qknorm_qkv_proj_workspace_bytes(65, 32, 8, 128) == 0, "no workspace above 64 tokens");
  EXPECT(qknorm_qkv_proj_workspace_bytes(-1, 32, 8, 128) == QKNORM_E_SHAPE, "negative T not rejected");
  EXPECT(qknorm_qkv_proj_per_head_ws(g, 256, g, 256, (void*)g, 512, 4, 256, 2, 1, 128, g, g, 0.0f, 0,
                                     QKNORM_BF16, NULL, 1 << 20, NULL) == QKNORM_E_NULLPTR,
         "a missing workspace not rejected");
  EXPECT(qknorm_qkv_proj_per_head_noalloc(g, 256, g, 256, (void*)g, 512, 4, 256, 2, 1, 128, g, g, 0.0f, 0,
                                          QKNORM_F32, NULL) == QKNORM_E_UNSUPPORTED,
         "fp32 projection not rejected");
  return 0;
}

static int per_head(void) {
  /* standalone [T, H, D] bf16, every head its own closed form */
  enum { T = 64, H = 48, D = 128 };
  const size_t n = (size_t)T * H * D;
  uint16_t* x = malloc(n * 2);
  uint16_t* y = malloc(n * 2);
  int* k = malloc(sizeof(int) * T * H);
  uint16_t g[D];
  EXPECT(x && y && k, "host allocation");
  for (int j = 0; j < D; ++j) g[j] = to_bf16(gamma_at(j));
  for (int i = 0; i < T * H; ++i) k[i] = fill_group(x + (size_t)i * D, D, (unsigned)(i * 7 + 3));
  void *dx, *dg;
  HIP_OK(hipMalloc(&dx, n * 2));
  HIP_OK(hipMalloc(&dg, sizeof g));
  HIP_OK(hipMemcpy(dx, x, n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dg, g, sizeof g, hipMemcpyHostToDevice));
  const int rc = qknorm_per_head(dx, T, H * D, H, 0, D, dg, NULL, 0.0f, QKNORM_BF16, NULL);
  EXPECT(rc == QKNORM_OK, "qknorm_per_head: %s", qknorm_strerror(rc));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(y, dx, n * 2, hipMemcpyDeviceToHost));
  for (int i = 0; i < T * H; ++i)
    if (check_group(y + (size_t)i * D, D, k[i], "per-head group", i)) return 1;
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dg));
  free(x);
  free(y);
  free(k);
  return 0;
}

static int layerwise(void) {
  /* rows [Q 4096 | K 1024 | V 1024] bf16, 8 shards; fused and two-phase */
  enum { T = 48, WQ = 4096, WK = 1024, LD = 6144, R = 8 };
  const size_t n = (size_t)T * LD;
  uint16_t* x = malloc(n * 2);
  uint16_t* y = malloc(n * 2);
  uint16_t* y2 = malloc(n * 2);
  uint16_t* gq = malloc(WQ * 2);
  uint16_t* gk = malloc(WK * 2);
  int kq[T], kk[T];
  EXPECT(x && y && y2 && gq && gk, "host allocation");
  for (int j = 0; j < WQ; ++j) gq[j] = to_bf16(gamma_at(j));
  for (int j = 0; j < WK; ++j) gk[j] = to_bf16(gamma_at(j));
  for (int t = 0; t < T; ++t) {
    kq[t] = fill_group(x + (size_t)t * LD, WQ, (unsigned)(t * 131 + 5));
    kk[t] = fill_group(x + (size_t)t * LD + WQ, WK, (unsigned)(t * 37 + 11));
    for (int c = WQ + WK; c < LD; ++c) x[(size_t)t * LD + c] = (uint16_t)(0x3F00u + (unsigned)(c + t) % 255u);
  }
  void *da, *db, *dgq, *dgk;
  float *pq, *pk;
  HIP_OK(hipMalloc(&da, n * 2));
  HIP_OK(hipMalloc(&db, n * 2));
  HIP_OK(hipMalloc(&dgq, WQ * 2));
  HIP_OK(hipMalloc(&dgk, WK * 2));
  HIP_OK(hipMalloc((void**)&pq, sizeof(float) * R * T));
  HIP_OK(hipMalloc((void**)&pk, sizeof(float) * R * T));
  HIP_OK(hipMemcpy(da, x, n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(db, x, n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dgq, gq, WQ * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dgk, gk, WK * 2, hipMemcpyHostToDevice));
  hipStream_t s;
  HIP_OK(hipStreamCreate(&s));
  int rc = qknorm_layerwise(da, T, LD, WQ, WK, dgq, dgk, 0.0f, R, QKNORM_BF16, s);
  EXPECT(rc == QKNORM_OK, "qknorm_layerwise: %s", qknorm_strerror(rc));
  rc = qknorm_partial_sumsq(db, T, LD, WQ, WK, R, pq, pk, QKNORM_BF16, s);
  EXPECT(rc == QKNORM_OK, "qknorm_partial_sumsq: %s", qknorm_strerror(rc));
  rc = qknorm_apply_scalar(db, T, LD, WQ, WK, pq, pk, R, WQ, WK, dgq, dgk, 0.0f, QKNORM_BF16, s);
  EXPECT(rc == QKNORM_OK, "qknorm_apply_scalar: %s", qknorm_strerror(rc));
  HIP_OK(hipStreamSynchronize(s));
  HIP_OK(hipMemcpy(y, da, n * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(y2, db, n * 2, hipMemcpyDeviceToHost));
  EXPECT(memcmp(y, y2, n * 2) == 0, "fused and two-phase layerwise differ");
  for (int t = 0; t < T; ++t) {
    if (check_group(y + (size_t)t * LD, WQ, kq[t], "layerwise Q of row", t)) return 1;
    if (check_group(y + (size_t)t * LD + WQ, WK, kk[t], "layerwise K of row", t)) return 1;
    EXPECT(memcmp(y + (size_t)t * LD + WQ + WK, x + (size_t)t * LD + WQ + WK, (LD - WQ - WK) * 2) == 0,
           "row %d: V columns changed", t);
  }
  HIP_OK(hipStreamDestroy(s));
  HIP_OK(hipFree(da));
  HIP_OK(hipFree(db));
  HIP_OK(hipFree(dgq));
  HIP_OK(hipFree(dgk));
  HIP_OK(hipFree(pq));
  HIP_OK(hipFree(pk));
  free(x);
  free(y);
  free(y2);
  free(gq);
  free(gk);
  return 0;
}

static int projection(void) {
  /* x [T, 256] bf16 holding two closed-form groups of 128 per row; w [512, 256]
   * with w[n][n % 256] = 1 and zeros elsewhere, so qkv[t][n] = x[t][n % 256]:
   * Q heads 0 and 1 are the two groups, the K head the first group again, the
   * V head a copy of the second group */
  enum { T = 5, HID = 256, HQ = 2, HKV = 1, D = 128, N = (HQ + 2 * HKV) * D };
  uint16_t *x = malloc((size_t)T * HID * 2), *w = calloc((size_t)N * HID, 2), *g = malloc(D * 2);
  uint16_t *y[3];
  int k[T][2];
  EXPECT(x && w && g, "host allocation");
  for (int j = 0; j < D; ++j) g[j] = to_bf16(gamma_at(j));
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < 2; ++h) k[t][h] = fill_group(x + (size_t)t * HID + h * D, D, (unsigned)(t * 17 + h * 5 + 1));
  for (int n = 0; n < N; ++n) w[(size_t)n * HID + n % HID] = to_bf16(1.0f);
  void *dx, *dw, *dg, *dy, *ws;
  const int64_t need = qknorm_qkv_proj_workspace_bytes(T, HQ, HKV, D);
  EXPECT(need == 4 * T * N * 4, "workspace bytes %lld", (long long)need);
  HIP_OK(hipMalloc(&dx, (size_t)T * HID * 2));
  HIP_OK(hipMalloc(&dw, (size_t)N * HID * 2));
  HIP_OK(hipMalloc(&dg, D * 2));
  HIP_OK(hipMalloc(&dy, (size_t)T * N * 2));
  HIP_OK(hipMalloc(&ws, (size_t)need));
  HIP_OK(hipMemcpy(dx, x, (size_t)T * HID * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dw, w, (size_t)N * HID * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dg, g, D * 2, hipMemcpyHostToDevice));
  for (int c = 0; c < 3; ++c) {
    y[c] = malloc((size_t)T * N * 2);
    EXPECT(y[c], "host allocation");
    HIP_OK(hipMemset(dy, 0xFF, (size_t)T * N * 2));
    int rc;
    if (c == 0)
      rc = qknorm_qkv_proj_per_head(dx, HID, dw, HID, dy, N, T, HID, HQ, HKV, D, dg, dg, 0.0f, 0,
                                    QKNORM_BF16, NULL);
    else if (c == 1)
      rc = qknorm_qkv_proj_per_head_ws(dx, HID, dw, HID, dy, N, T, HID, HQ, HKV, D, dg, dg, 0.0f, 0,
                                       QKNORM_BF16, ws, need, NULL);
    else
      rc = qknorm_qkv_proj_per_head_noalloc(dx, HID, dw, HID, dy, N, T, HID, HQ, HKV, D, dg, dg, 0.0f, 0,
                                            QKNORM_BF16, NULL);
    EXPECT(rc == QKNORM_OK, "projection call %d: %s", c, qknorm_strerror(rc));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(y[c], dy, (size_t)T * N * 2, hipMemcpyDeviceToHost));
    for (int t = 0; t < T; ++t) {
      const uint16_t* r = y[c] + (size_t)t * N;
      if (check_group(r, D, k[t][0], "projection Q head 0 of row", t)) return 1;
      if (check_group(r + D, D, k[t][1], "projection Q head 1 of row", t)) return 1;
      if (check_group(r + 2 * D, D, k[t][0], "projection K head of row", t)) return 1;
      EXPECT(memcmp(r + 3 * D, x + (size_t)t * HID + D, D * 2) == 0, "call %d row %d: V head is not x", c, t);
    }
  }
  EXPECT(memcmp(y[0], y[1], (size_t)T * N * 2) == 0, "workspace projection differs from the plain call");
  EXPECT(memcmp(y[0], y[2], (size_t)T * N * 2) == 0, "no-alloc projection differs from the plain call");
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(dw));
  HIP_OK(hipFree(dg));
  HIP_OK(hipFree(dy));
  HIP_OK(hipFree(ws));
  for (int c = 0; c < 3; ++c) free(y[c]);
  free(x);
  free(w);
  free(g);
  return 0;
}

int main(int argc, char** argv) {
  if (validation()) return 1;
  printf("validation codes ok\n");
  fflush(stdout);
  if (argc > 1 && strcmp(argv[1], "--validation-only") == 0) return 0;
  if (per_head()) return 1;
  printf("per-head closed forms ok\n");
  fflush(stdout);
  if (layerwise()) return 1;
  printf("layerwise closed forms ok, fused == two-phase\n");
  fflush(stdout);
  if (projection()) return 1;
  printf("projection closed forms ok, the three projection calls agree\n");
  return 0;
}
