// Host-side argument checks of the C ABI (include/qmm.h), run against a build
// of the library whose host code is instrumented with AddressSanitizer and
// UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py builds both).
// Every call here either fails a host check or is zero-sized, so nothing is
// launched and no GPU is needed; the pointers are fake and never
// dereferenced. Extreme sizes (near 2^31, 2^63) probe the overflow guards of
// the size arithmetic, which UBSan turns into a failure if any of it wraps.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qmm.h"

static int failures = 0;

#define EXPECT(expr, want)                                                                                 \
  do {                                                                                                     \
    const long long got_ = (long long)(expr);                                                              \
    if (got_ != (long long)(want)) {                                                                       \
      fprintf(stderr, "FAIL line %d: %s = %lld, expected %lld\n", __LINE__, #expr, got_, (long long)(want)); \
      ++failures;                                                                                          \
    }                                                                                                      \
  } while (0)

static const void *const W = (const void *)0x10000;
static const float *const X = (const float *)0x20000;
static float *const Y = (float *)0x30000;
static const int32_t *const IDS = (const int32_t *)0x40000;

static int mm(const void *w, int t, int64_t rows, int64_t k, int64_t nb1, const void *x, int xt, int64_t n, float *y,
              int path) {
  return qmm_matmul_path(w, t, rows, k, nb1, x, xt, n, y, path, NULL);
}

int main() {
  const int64_t big = (int64_t)1 << 62;
  // row sizes and support queries
  EXPECT(qmm_row_bytes(QMM_TYPE_Q4_0, 4096), 2304);
  EXPECT(qmm_row_bytes(QMM_TYPE_Q8_0, 4096), 4352);
  EXPECT(qmm_row_bytes(QMM_TYPE_Q4_K, 11008), 43 * 144);
  EXPECT(qmm_row_bytes(QMM_TYPE_Q4_0, INT64_MAX), QMM_ERR_SHAPE);
  EXPECT(qmm_row_bytes(QMM_TYPE_Q4_0, INT64_MIN), QMM_ERR_SHAPE);
  EXPECT(qmm_row_bytes(QMM_TYPE_Q4_0, big), QMM_ERR_SHAPE);
  EXPECT(qmm_row_bytes(5, 4096), QMM_ERR_TYPE);
  EXPECT(qmm_row_bytes(-1, 4096), QMM_ERR_TYPE);
  EXPECT(qmm_supports(QMM_TYPE_Q4_0, 4096, 2304), 1);
  EXPECT(qmm_supports(QMM_TYPE_Q4_0, 4096, INT64_MAX), 0);
  EXPECT(qmm_supports(QMM_TYPE_Q4_0, big, 2304), 0);
  EXPECT(qmm_supports(QMM_TYPE_Q4_K, 256, 146), 0);
  for (int code = -9; code <= 0; ++code) {
    const char *s = qmm_status_string(code);
    if (s == NULL || strncmp(s, code == 0 ? "QMM_OK" : "QMM_ERR_", code == 0 ? 6 : 8) != 0) {
      fprintf(stderr, "FAIL: status string %d\n", code);
      ++failures;
    }
  }
  EXPECT(strcmp(qmm_status_string(-99), "unknown qmm status"), 0);
  EXPECT(strcmp(qmm_status_string(INT32_MIN), "unknown qmm status"), 0);

  // MUL_MAT checks, in the order the header states them
  EXPECT(mm(NULL, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_NULL);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, NULL, QMM_X_F32, 1, Y, 0), QMM_ERR_NULL);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F32, 1, NULL, 0), QMM_ERR_NULL);
  EXPECT(mm(W, 1, 16, 64, 36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_TYPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, X, 2, 1, Y, 0), QMM_ERR_TYPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 40, 36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, -1, 64, 36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, INT64_MAX, 64, 36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F32, INT64_MAX, Y, 0), QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, INT64_MAX - 31, 36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_SHAPE);
  // matrix bytes, activation and output elements beyond the stated bounds
  const int64_t kbig = ((int64_t)1 << 31) - 32, nbbig = (kbig / 32) * 18;
  EXPECT(mm(W, QMM_TYPE_Q4_0, (int64_t)1 << 30, 64, (int64_t)1 << 40, X, QMM_X_F32, 1, Y, 0), QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, kbig, nbbig, X, QMM_X_F32, ((int64_t)1 << 31) - 1, Y, 0), QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, ((int64_t)1 << 31) - 1, 64, 36, X, QMM_X_F32, ((int64_t)1 << 31) - 1, Y, 0),
         QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, ((int64_t)1 << 31) - 1, kbig, nbbig, X, QMM_X_F32, 0, Y, 0), QMM_OK);
  EXPECT(qmm_dequantize(W, QMM_TYPE_Q4_0, ((int64_t)1 << 31) - 1, kbig, nbbig, Y, NULL), QMM_ERR_SHAPE);
  EXPECT(qmm_get_rows(W, QMM_TYPE_Q4_0, 16, kbig, nbbig, IDS, ((int64_t)1 << 31) - 1, Y, NULL), QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 35, X, QMM_X_F32, 1, Y, 0), QMM_ERR_STRIDE);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, -36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_STRIDE);
  EXPECT(mm(W, QMM_TYPE_Q8_0, 16, 64, 36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_STRIDE);
  EXPECT(mm((const char *)W + 1, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F32, 1, Y, 0), QMM_ERR_ALIGN);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, (const char *)X + 2, QMM_X_F32, 1, Y, 0), QMM_ERR_ALIGN);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F32, 1, (float *)((char *)Y + 2), 0), QMM_ERR_ALIGN);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F32, 1, Y, 3), QMM_ERR_PATH);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F32, 9, Y, QMM_PATH_GEMV), QMM_ERR_PATH);
  EXPECT(mm(W, QMM_TYPE_Q4_K, 16, 96, 144, X, QMM_X_F32, 1, Y, 0), QMM_ERR_SHAPE);
  EXPECT(mm(W, QMM_TYPE_Q4_K, 2, 256, (int64_t)1 << 24, X, QMM_X_F32, 1, Y, 0), QMM_ERR_SHAPE);
  // zero-sized calls: valid, nothing launched
  EXPECT(mm(W, QMM_TYPE_Q4_0, 0, 64, 36, X, QMM_X_F32, 1, Y, 0), QMM_OK);
  EXPECT(mm(W, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F32, 0, Y, QMM_PATH_GEMM), QMM_OK);
  EXPECT(mm((const char *)W + 2, QMM_TYPE_Q4_0, 16, 64, 38, X, QMM_X_F32, 0, Y, 0), QMM_OK);
  EXPECT(qmm_matmul(W, QMM_TYPE_Q8_0, 0, 64, 68, X, 4, Y, NULL), QMM_OK);
  EXPECT(qmm_matmul_x16(W, QMM_TYPE_Q8_0, 5, 64, 68, (const uint16_t *)X, 0, Y, NULL), QMM_OK);
  EXPECT(qmm_dequantize(W, QMM_TYPE_Q4_0, 0, 64, 36, Y, NULL), QMM_OK);
  EXPECT(qmm_dequantize(W, QMM_TYPE_Q4_0, INT64_MAX, 64, 36, Y, NULL), QMM_ERR_SHAPE);
  // MUL_MAT with a workspace: the same checks, then the workspace's; the
  // size query agrees (no device here: no compute units, no split)
  EXPECT(qmm_matmul_ws(NULL, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F16, 600, Y, NULL, 0, NULL), QMM_ERR_NULL);
  EXPECT(qmm_matmul_ws(W, 1, 16, 64, 36, X, QMM_X_F16, 600, Y, NULL, 0, NULL), QMM_ERR_TYPE);
  EXPECT(qmm_matmul_ws(W, QMM_TYPE_Q4_0, 16, 64, 36, X, 7, 600, Y, NULL, 0, NULL), QMM_ERR_TYPE);
  EXPECT(qmm_matmul_ws(W, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F16, INT64_MAX, Y, NULL, 0, NULL), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_ws(W, QMM_TYPE_Q4_0, (int64_t)1 << 30, 64, (int64_t)1 << 40, X, QMM_X_F16, 600, Y, NULL, 0,
                       NULL), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_ws(W, QMM_TYPE_Q4_0, 16, 64, 36, X, QMM_X_F16, 0, Y, (void *)0x50001, -7, NULL), QMM_OK);
  EXPECT(qmm_matmul_ws(W, QMM_TYPE_Q4_0, 0, 64, 36, X, QMM_X_F16, 600, Y, NULL, 0, NULL), QMM_OK);
  EXPECT(qmm_matmul_workspace_bytes(1, 16, 64, 600, QMM_X_F16), QMM_ERR_TYPE);
  EXPECT(qmm_matmul_workspace_bytes(QMM_TYPE_Q4_0, 16, 64, 600, -1), QMM_ERR_TYPE);
  EXPECT(qmm_matmul_workspace_bytes(QMM_TYPE_Q4_0, 16, 40, 600, QMM_X_F16), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_workspace_bytes(QMM_TYPE_Q4_0, INT64_MIN, 64, 600, QMM_X_F16), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_workspace_bytes(QMM_TYPE_Q4_0, 16, INT64_MAX, 600, QMM_X_F16), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_workspace_bytes(QMM_TYPE_Q4_0, 16, 64, INT64_MAX, QMM_X_F16), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_workspace_bytes(QMM_TYPE_Q4_0, ((int64_t)1 << 31) - 1, kbig, (int64_t)1 << 30, QMM_X_F16),
         QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_workspace_bytes(QMM_TYPE_Q4_0, ((int64_t)1 << 31) - 1, kbig, 1 << 28, QMM_X_F16), 0);
  EXPECT(qmm_matmul_workspace_bytes(QMM_TYPE_Q4_K, 4096, 4096, 600, QMM_X_F16), 0);
  EXPECT(qmm_get_rows(W, QMM_TYPE_Q4_0, 16, 64, 36, IDS, 0, Y, NULL), QMM_OK);
  EXPECT(qmm_get_rows(W, QMM_TYPE_Q4_0, 16, 64, 36, NULL, 4, Y, NULL), QMM_ERR_NULL);
  EXPECT(qmm_get_rows(W, QMM_TYPE_Q4_0, 16, 64, 36, IDS, -1, Y, NULL), QMM_ERR_SHAPE);
  EXPECT(qmm_get_rows(W, QMM_TYPE_Q4_0, 16, 64, 36, IDS, INT64_MAX, Y, NULL), QMM_ERR_SHAPE);

  // batches: every descriptor is checked before anything is enqueued
  qmm_matmul_desc d[3];
  for (int i = 0; i < 3; ++i) {
    d[i].W = W;
    d[i].ggml_type = QMM_TYPE_Q4_0;
    d[i].n_rows = 16;
    d[i].k = 64;
    d[i].row_stride_bytes = 36;
    d[i].X = X;
    d[i].x_type = QMM_X_F32;
    d[i].n_tokens = 0;
    d[i].Y = Y;
  }
  EXPECT(qmm_matmul_batch(d, 3, NULL), QMM_OK);
  EXPECT(qmm_matmul_batch(d, 0, NULL), QMM_OK);
  EXPECT(qmm_matmul_batch(NULL, 0, NULL), QMM_OK);
  EXPECT(qmm_matmul_batch(NULL, 2, NULL), QMM_ERR_NULL);
  EXPECT(qmm_matmul_batch(d, -1, NULL), QMM_ERR_SHAPE);
  d[2].k = 48;
  EXPECT(qmm_matmul_batch(d, 3, NULL), QMM_ERR_SHAPE);
  d[2].k = 64;
  d[1].ggml_type = 9;
  EXPECT(qmm_matmul_batch(d, 3, NULL), QMM_ERR_TYPE);

  // MUL_MAT_ID sizes and checks
  EXPECT(qmm_matmul_id_workspace_bytes(8, 2, 0), 0);
  EXPECT(qmm_matmul_id_workspace_bytes(8, 2, 1), 0);  // one token: per-pair decode, no workspace
  EXPECT(qmm_matmul_id_workspace_bytes(-1, 2, 512), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id_workspace_bytes(8, INT64_MAX, 2), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id_workspace_bytes(8, 2, INT64_MAX), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id_workspace_bytes(INT64_MAX, 2, 512), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id_workspace_bytes_x16(8, 2, 512, 0, 1), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id_workspace_bytes_x16(8, 2, 512, 4096, 3), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id_workspace_bytes_x16(8, 2, (int64_t)1 << 30, INT64_MAX, 1), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id_workspace_bytes_x16(8, 2, (int64_t)1 << 29, (int64_t)1 << 20, 2), QMM_ERR_SHAPE);
  {
    const int64_t base = qmm_matmul_id_workspace_bytes(8, 2, 512);
    const int64_t x16 = qmm_matmul_id_workspace_bytes_x16(8, 2, 512, 4096, 1);
    if (!(base > 0 && x16 == base + 512 * 4096 * 2)) {
      fprintf(stderr, "FAIL: workspace sizes %lld / %lld\n", (long long)base, (long long)x16);
      ++failures;
    }
  }
  char ws[64];
  const int64_t nb1 = 36, nb2 = 16 * 36;
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, 4, 16, 64, nb1, nb2, X, 1, IDS, 2, 0, Y, ws, 64, NULL), QMM_OK);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, 4, 16, 64, nb1, nb2, X, 3, IDS, 2, 5, Y, ws, 64, NULL), QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, 4, 16, 64, nb1, nb2 - 2, X, 1, IDS, 2, 5, Y, ws, 64, NULL),
         QMM_ERR_STRIDE);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, 4, 16, 64, nb1, nb2, X, 1, NULL, 2, 5, Y, ws, 64, NULL), QMM_ERR_NULL);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, 4, 16, 64, nb1, nb2, X, 1, IDS, 2, 300, Y, NULL, 0, NULL),
         QMM_ERR_WORKSPACE);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, 4, 16, 64, nb1, nb2, X, 1, IDS, 2, 300, Y, ws, 64, NULL),
         QMM_ERR_WORKSPACE);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, INT64_MAX, 16, 64, nb1, nb2, X, 1, IDS, 2, 5, Y, ws, 64, NULL),
         QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, 4, 16, 64, nb1, nb2, X, 1, IDS, INT64_MAX, 5, Y, ws, 64, NULL),
         QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, ((int64_t)1 << 31) - 1, 16, 64, nb1, (int64_t)1 << 32, X, 1, IDS, 2, 5, Y,
                       ws, 64, NULL),
         QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id(W, QMM_TYPE_Q4_0, 4, 16, kbig, nbbig, 16 * nbbig, X, 2, IDS, 2, ((int64_t)1 << 30) - 1, Y, ws,
                       64, NULL),
         QMM_ERR_SHAPE);
  EXPECT(qmm_matmul_id_noalloc(W, QMM_TYPE_Q4_0, 4, 16, 64, nb1, nb2, X, 1, IDS, 2, 0, Y, NULL), QMM_OK);
  EXPECT(qmm_matmul_id_noalloc(W, QMM_TYPE_Q4_0, 4096, 16, 64, nb1, nb2, X, 1, IDS, 8, 1 << 20, Y, NULL),
         QMM_ERR_SCRATCH);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi checks ok\n");
  return 0;
}
