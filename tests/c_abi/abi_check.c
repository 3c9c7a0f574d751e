/*
 * The C ABI of libw4a16 driven from plain C (no Python, no PyTorch): device
 * memory and a stream from the HIP runtime's C API, the library's calls as
 * include/w4a16.h declares them, and every result checked against the CPU
 * oracle (oracle/liboracle.so, linked as test infrastructure).
 *
 * Covers w4a16_matmul, w4a16_repack_tiled + w4a16_matmul_tiled,
 * w4a16_head_gather with argmax (an out-of-range id among the rows),
 * w4a16_batch_plan + w4a16_matmul_batch (a row-major problem and a tiled one
 * with its argmax), and host-side rejections.  Exit status 0 and a final
 * "abi_check ok" line when everything holds.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "w4a16.h"

/* the oracle (test infrastructure, oracle/oracle.c) */
void oracle_matmul(const uint8_t* packed, const uint16_t* scales, const uint16_t* x, int64_t N, int64_t K, int T,
                   double* y, double* a, int nthreads);
void oracle_gather(const int32_t* row_ids, int64_t n_ids, const uint8_t* packed, const uint16_t* scales,
                   int64_t n_rows, const uint16_t* x, int64_t K, int T, double* y, double* a, int nthreads);
void oracle_argmax(const double* y, const int32_t* ids, int64_t n, int T, int32_t* id_out, double* val_out,
                   double* gap_out);

static int failures = 0;
#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                        \
      fprintf(stderr, "\n");                               \
      ++failures;                                          \
    }                                                      \
  } while (0)
#define HIP(call)                                                            \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(2);                                                               \
    }                                                                        \
  } while (0)

/* test inputs: xorshift64, codes uniform, scales bf16 in [1e-3, 0.05), x bf16 in (-2, 2) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 7;
  rng_state ^= rng_state << 17;
  return rng_state;
}
static uint16_t bf16_of(float f) { /* truncation: any bf16 value serves as an input */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}
static double uniform(void) { return (double)(next_u64() >> 11) / 9007199254740992.0; }

static void make_weight(int64_t N, int64_t K, uint8_t** p, uint16_t** s) {
  *p = malloc((size_t)(N * K / 2));
  *s = malloc((size_t)(N * (K / 128)) * 2);
  for (int64_t i = 0; i < N * K / 2; ++i) (*p)[i] = (uint8_t)next_u64();
  for (int64_t i = 0; i < N * (K / 128); ++i) (*s)[i] = bf16_of((float)(1e-3 + 0.049 * uniform()));
}
static uint16_t* make_x(int T, int64_t K) {
  uint16_t* x = malloc((size_t)(T * K) * 2);
  for (int64_t i = 0; i < T * K; ++i) x[i] = bf16_of((float)(4.0 * uniform() - 2.0));
  return x;
}
static void* to_dev(const void* h, size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes));
  HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  return d;
}
static float* from_dev(const void* d, size_t n) {
  float* h = malloc(n * sizeof(float));
  HIP(hipMemcpy(h, d, n * sizeof(float), hipMemcpyDeviceToHost));
  return h;
}

/* |y - y_ref| <= 1e-3 * A + 1e-6 elementwise; NaN where the reference is NaN */
static int compare(const float* y, const double* ref, const double* a, int64_t n, const char* what) {
  int bad = 0;
  for (int64_t i = 0; i < n; ++i) {
    if (isnan(ref[i])) {
      if (!isnan(y[i])) ++bad;
      continue;
    }
    if (!(fabs((double)y[i] - ref[i]) <= 1e-3 * a[i] + 1e-6)) ++bad;
  }
  CHECK(bad == 0, "%s: %d of %lld outputs outside the tolerance", what, bad, (long long)n);
  return bad;
}

/* argmax ids equal the oracle's argmax of the GPU's own scores, bit for bit */
static void check_argmax(const float* y, const int32_t* ids, int64_t n, int T, const int32_t* got_id,
                         const float* got_val, const char* what) {
  double* yd = malloc((size_t)(n * T) * sizeof(double));
  for (int64_t i = 0; i < n * T; ++i) yd[i] = y[i];
  int32_t* rid = malloc((size_t)T * sizeof(int32_t));
  double* rval = malloc((size_t)T * sizeof(double));
  double* gap = malloc((size_t)T * sizeof(double));
  oracle_argmax(yd, ids, n, T, rid, rval, gap);
  for (int t = 0; t < T; ++t) {
    CHECK(got_id[t] == rid[t], "%s: row %d argmax id %d, oracle %d", what, t, got_id[t], rid[t]);
    CHECK((isnan(rval[t]) && isnan(got_val[t])) || (double)got_val[t] == rval[t], "%s: row %d argmax value", what, t);
  }
  free(yd);
  free(rid);
  free(rval);
  free(gap);
}

int main(void) {
  int dev_count = 0;
  if (hipGetDeviceCount(&dev_count) != hipSuccess || dev_count < 1) {
    fprintf(stderr, "no GPU\n");
    return 3;
  }
  HIP(hipSetDevice(0));
  hipStream_t st;
  HIP(hipStreamCreate(&st));
  CHECK(w4a16_abi_version() == W4A16_ABI_VERSION, "ABI version %d, header %d", w4a16_abi_version(), W4A16_ABI_VERSION);

  const int T = 5;
  const int64_t N = 1000, K = 1152; /* 63 tiles (the last one ragged), 9 groups */
  uint8_t* p;
  uint16_t* s;
  make_weight(N, K, &p, &s);
  uint16_t* x = make_x(T, K);
  double* yref = malloc((size_t)(T * N) * sizeof(double));
  double* aref = malloc((size_t)(T * N) * sizeof(double));
  oracle_matmul(p, s, x, N, K, T, yref, aref, 4);
  uint8_t* pd = to_dev(p, (size_t)(N * K / 2));
  uint16_t* sd = to_dev(s, (size_t)(N * (K / 128)) * 2);
  uint16_t* xd = to_dev(x, (size_t)(T * K) * 2);
  float* yd;
  HIP(hipMalloc((void**)&yd, (size_t)(T * N) * sizeof(float)));

  /* 1. w4a16_matmul */
  CHECK(w4a16_matmul(pd, sd, xd, yd, N, K, T, st) == W4A16_OK, "w4a16_matmul");
  HIP(hipStreamSynchronize(st));
  float* y = from_dev(yd, (size_t)(T * N));
  compare(y, yref, aref, T * N, "w4a16_matmul");
  free(y);

  /* 2. tiled layout */
  const size_t tb = w4a16_tiled_bytes(N, K);
  CHECK(tb == (size_t)((N + 15) / 16) * (size_t)(9 * 1024 + 2 * 256), "tiled bytes %zu", tb);
  void* tw;
  HIP(hipMalloc(&tw, tb));
  CHECK(w4a16_repack_tiled(pd, sd, N, K, tw, tb, st) == W4A16_OK, "w4a16_repack_tiled");
  HIP(hipMemsetAsync(yd, 0xFF, (size_t)(T * N) * sizeof(float), st));
  CHECK(w4a16_matmul_tiled(tw, xd, yd, N, K, T, st) == W4A16_OK, "w4a16_matmul_tiled");
  HIP(hipStreamSynchronize(st));
  y = from_dev(yd, (size_t)(T * N));
  compare(y, yref, aref, T * N, "w4a16_matmul_tiled");
  free(y);

  /* 3. gathered head with argmax; one id out of range (its row is NaN) */
  const int64_t n_ids = 300;
  int32_t* ids = malloc((size_t)n_ids * sizeof(int32_t));
  for (int64_t i = 0; i < n_ids; ++i) ids[i] = (int32_t)((i * 7919 + 13) % N);
  ids[17] = (int32_t)N + 5;
  int32_t* idsd = to_dev(ids, (size_t)n_ids * sizeof(int32_t));
  double* gref = malloc((size_t)(T * n_ids) * sizeof(double));
  double* garef = malloc((size_t)(T * n_ids) * sizeof(double));
  oracle_gather(ids, n_ids, p, s, N, x, K, T, gref, garef, 4);
  float *gd, *avd;
  int32_t* aid;
  HIP(hipMalloc((void**)&gd, (size_t)(T * n_ids) * sizeof(float)));
  HIP(hipMalloc((void**)&aid, (size_t)T * sizeof(int32_t)));
  HIP(hipMalloc((void**)&avd, (size_t)T * sizeof(float)));
  const size_t wsb = w4a16_workspace_bytes(n_ids, T);
  void* ws;
  HIP(hipMalloc(&ws, wsb));
  CHECK(w4a16_head_gather(idsd, n_ids, pd, sd, N, xd, K, T, gd, aid, avd, ws, wsb, st) == W4A16_OK,
        "w4a16_head_gather");
  HIP(hipStreamSynchronize(st));
  float* g = from_dev(gd, (size_t)(T * n_ids));
  int32_t ga[16];
  float gv[16];
  HIP(hipMemcpy(ga, aid, (size_t)T * sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP(hipMemcpy(gv, avd, (size_t)T * sizeof(float), hipMemcpyDeviceToHost));
  compare(g, gref, garef, T * n_ids, "w4a16_head_gather");
  check_argmax(g, ids, n_ids, T, ga, gv, "w4a16_head_gather");
  free(g);

  /* 4. grouped launch: the row-major matrix, and the tiled one with its argmax */
  float* yb;
  int32_t* bid;
  float* bval;
  HIP(hipMalloc((void**)&yb, (size_t)(T * N) * sizeof(float)));
  HIP(hipMalloc((void**)&bid, (size_t)T * sizeof(int32_t)));
  HIP(hipMalloc((void**)&bval, (size_t)T * sizeof(float)));
  void* ws2;
  const size_t wsb2 = w4a16_workspace_bytes(N, T);
  HIP(hipMalloc(&ws2, wsb2));
  HIP(hipMemsetAsync(yd, 0xFF, (size_t)(T * N) * sizeof(float), st));
  w4a16_problem probs[2];
  memset(probs, 0, sizeof(probs));
  probs[0].packed_u4 = pd;
  probs[0].scales_bf16 = sd;
  probs[0].x_bf16 = xd;
  probs[0].y_f32 = yd;
  probs[0].N = N;
  probs[0].K = K;
  probs[0].layout = W4A16_LAYOUT_ROW_MAJOR;
  probs[1] = probs[0];
  probs[1].packed_u4 = (const uint8_t*)tw;
  probs[1].scales_bf16 = NULL;
  probs[1].y_f32 = yb;
  probs[1].layout = W4A16_LAYOUT_TILED;
  probs[1].argmax_id = bid;
  probs[1].argmax_val = bval;
  probs[1].workspace = ws2;
  probs[1].workspace_bytes = wsb2;
  const size_t table_bytes = w4a16_batch_table_bytes(2);
  void* table_host = malloc(table_bytes);
  void* table_dev;
  CHECK(w4a16_batch_plan(probs, 2, T, table_host, table_bytes) == W4A16_OK, "w4a16_batch_plan");
  HIP(hipMalloc(&table_dev, table_bytes));
  HIP(hipMemcpy(table_dev, table_host, table_bytes, hipMemcpyHostToDevice));
  CHECK(w4a16_matmul_batch(table_host, table_dev, st) == W4A16_OK, "w4a16_matmul_batch");
  HIP(hipStreamSynchronize(st));
  float* y0 = from_dev(yd, (size_t)(T * N));
  float* y1 = from_dev(yb, (size_t)(T * N));
  int32_t bi[16];
  float bv[16];
  HIP(hipMemcpy(bi, bid, (size_t)T * sizeof(int32_t), hipMemcpyDeviceToHost));
  HIP(hipMemcpy(bv, bval, (size_t)T * sizeof(float), hipMemcpyDeviceToHost));
  compare(y0, yref, aref, T * N, "batch, row-major problem");
  compare(y1, yref, aref, T * N, "batch, tiled problem");
  check_argmax(y1, NULL, N, T, bi, bv, "batch argmax");
  free(y0);
  free(y1);

  /* 5. rejected on the host, nothing enqueued */
  CHECK(w4a16_matmul(NULL, sd, xd, yd, N, K, T, st) == W4A16_ERR_NULL_POINTER, "null packed");
  CHECK(w4a16_matmul(pd, sd, xd, yd, N, 1000, T, st) == W4A16_ERR_BAD_SHAPE, "K not a multiple of 128");
  CHECK(w4a16_matmul(pd, sd, xd, yd, N, K, W4A16_MAX_T + 1, st) == W4A16_ERR_BAD_SHAPE, "T too large");
  CHECK(w4a16_matmul(pd + 1, sd, xd, yd, N, K, T, st) == W4A16_ERR_MISALIGNED, "misaligned packed");
  CHECK(w4a16_head_gather(idsd, n_ids, pd, sd, N, xd, K, T, gd, aid, avd, ws, wsb - 1, st) == W4A16_ERR_WORKSPACE,
        "small workspace");
  CHECK(strlen(w4a16_status_string(W4A16_ERR_WORKSPACE)) > 0, "status string");

  HIP(hipStreamSynchronize(st));
  HIP(hipStreamDestroy(st));
  hipFree(pd);
  hipFree(sd);
  hipFree(xd);
  hipFree(yd);
  hipFree(tw);
  hipFree(idsd);
  hipFree(gd);
  hipFree(aid);
  hipFree(avd);
  hipFree(ws);
  hipFree(yb);
  hipFree(bid);
  hipFree(bval);
  hipFree(ws2);
  hipFree(table_dev);
  free(table_host);
  free(p);
  free(s);
  free(x);
  free(yref);
  free(aref);
  free(ids);
  free(gref);
  free(garef);
  if (failures) {
    fprintf(stderr, "abi_check: %d failures\n", failures);
    return 1;
  }
  printf("abi_check ok: matmul, tiled, gather with argmax, grouped launch with argmax (N=%lld K=%lld T=%d)\n",
         (long long)N, (long long)K, T);
  return 0;
}
