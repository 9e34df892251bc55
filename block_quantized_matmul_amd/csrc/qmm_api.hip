// C ABI entry points: argument validation, kernel choice and launch.
//
// The op is ggml's MUL_MAT of a block-quantized weight with activations
// ([Bind] "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section 2.3). Row
// strides follow the nb[1] = nb[0] * (ne[0] / block) + padding rule of
// [Graph] "llama.cpp 源码完全拆解(二)：ggml 计算图与内存分配器", section
// "ggml_tensor：一个图节点的全部字段". One-token and many-token calls use
// different kernels, as the batch-of-512 capability probe of [Load]
// "llama.cpp 源码完全拆解(三)：GGUF 装载、mmap 与张量放置", section "第六步"
// explains backends do; the switch point is QMM_GEMV_MAX_TOKENS.
//
// Every check runs on the host before any HIP call, so invalid arguments are
// reported without a GPU and nothing is enqueued. Setting QMM_TRACE=1 in the
// environment prints each dispatch decision to stderr.
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "common.h"
#include "launch.h"

// Scratch of qmm_matmul_id_noalloc: the routing table of the grouped
// MUL_MAT_ID routes, held in a file-scope device array so that the entry
// point allocates nothing. Each GPU the library runs on keeps its own copy
// until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: kernels are given the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[QMM_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;
// Bounds that keep every byte or element count the library computes on the
// host inside int64: a matrix or expert stack spans fewer than 2^62 bytes,
// an activation or output array holds fewer than 2^60 elements.
constexpr int64_t kMaxBytes = int64_t{1} << 62;
constexpr int64_t kMaxElems = int64_t{1} << 60;
// a * b <= limit, for a, b >= 0, without forming the product
bool product_within(int64_t a, int64_t b, int64_t limit) { return b == 0 || a <= limit / b; }

// Bytes and weights of one block of the type (0 for an unknown type). The
// 32-weight types follow [Bind] section 2.3 and the library's readings; Q4_K
// is a 256-weight super-block, a Q4_K tensor being ne[0] / 256 blocks
// ([Graph] "llama.cpp 源码完全拆解(二)：ggml 计算图与内存分配器", the figure
// notes on quantised matmul).
int block_bytes(int type) {
  switch (type) {
    case QMM_TYPE_Q4_0: return 18;
    case QMM_TYPE_Q4_1: return 20;
    case QMM_TYPE_Q5_0: return 22;
    case QMM_TYPE_Q5_1: return 24;
    case QMM_TYPE_Q8_0: return 34;
    case QMM_TYPE_Q4_K: return 144;
    default: return 0;
  }
}
int block_weights(int type) { return type == QMM_TYPE_Q4_K ? 256 : 32; }

bool trace_on() {
  static const bool on = [] {
    const char *e = getenv("QMM_TRACE");
    return e != nullptr && e[0] != '\0' && e[0] != '0';
  }();
  return on;
}

bool aligned(const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Checks shared by every entry point that takes a weight matrix.
// Q4_K weights are read only as whole 16-byte pieces (GGUF aligns tensor
// data to at least 32 bytes), so their rows must start 16-byte aligned.
int check_weights(const void *W, int type, int64_t n_rows, int64_t k, int64_t nb1) {
  if (W == nullptr) return QMM_ERR_NULL;
  const int bb = block_bytes(type), bw = block_weights(type);
  if (bb == 0) return QMM_ERR_TYPE;
  if (k <= 0 || k % bw != 0 || k > kMaxDim || n_rows < 0 || n_rows > kMaxDim) return QMM_ERR_SHAPE;
  if (nb1 % 2 != 0 || nb1 < (k / bw) * bb) return QMM_ERR_STRIDE;
  if (type == QMM_TYPE_Q4_K && nb1 % 16 != 0) return QMM_ERR_STRIDE;
  if (!product_within(n_rows, nb1, kMaxBytes)) return QMM_ERR_SHAPE;
  // the decode kernel addresses a Q4_K matrix with 32-bit offsets
  if (type == QMM_TYPE_Q4_K && (n_rows * nb1 >= (int64_t{1} << 32) || nb1 >= (int64_t{1} << 24))) return QMM_ERR_SHAPE;
  if (!aligned(W, type == QMM_TYPE_Q4_K ? 16 : 2)) return QMM_ERR_ALIGN;
  return QMM_OK;
}

const char *type_name(int t) {
  switch (t) {
    case QMM_TYPE_Q4_0: return "q4_0";
    case QMM_TYPE_Q4_1: return "q4_1";
    case QMM_TYPE_Q5_0: return "q5_0";
    case QMM_TYPE_Q5_1: return "q5_1";
    case QMM_TYPE_Q4_K: return "q4_k";
    default: return "q8_0";
  }
}

int status_of(hipError_t e) { return e == hipSuccess ? QMM_OK : QMM_ERR_HIP; }

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (nullptr if HIP cannot
// give it).
void *device_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int64_t qmm_row_bytes(int ggml_type, int64_t k) {
  const int bb = block_bytes(ggml_type), bw = block_weights(ggml_type);
  if (bb == 0) return QMM_ERR_TYPE;
  if (k <= 0 || k % bw != 0 || k > kMaxDim) return QMM_ERR_SHAPE;
  return (k / bw) * bb;
}

int qmm_supports(int ggml_type, int64_t k, int64_t row_stride_bytes) {
  const int bb = block_bytes(ggml_type), bw = block_weights(ggml_type);
  if (bb == 0 || k <= 0 || k % bw != 0 || k > kMaxDim) return 0;
  if (ggml_type == QMM_TYPE_Q4_K && row_stride_bytes % 16 != 0) return 0;
  return (row_stride_bytes % 2 == 0 && row_stride_bytes >= (k / bw) * bb) ? 1 : 0;
}

const char *qmm_status_string(int status) {
  switch (status) {
    case QMM_OK: return "QMM_OK";
    case QMM_ERR_NULL: return "QMM_ERR_NULL: a required pointer is NULL";
    case QMM_ERR_TYPE: return "QMM_ERR_TYPE: unsupported weight or activation type";
    case QMM_ERR_SHAPE:
      return "QMM_ERR_SHAPE: k must be a positive multiple of 32 (of 256 for Q4_K); sizes must be in [0, 2^31)";
    case QMM_ERR_STRIDE:
      return "QMM_ERR_STRIDE: row stride must be even (a multiple of 16 for Q4_K) and cover the row's blocks";
    case QMM_ERR_ALIGN: return "QMM_ERR_ALIGN: W needs 2-byte (Q4_K: 16-byte), X, Y and out 4-byte alignment";
    case QMM_ERR_HIP: return "QMM_ERR_HIP: the HIP runtime rejected the kernel launch";
    case QMM_ERR_PATH: return "QMM_ERR_PATH: unknown path, or GEMV forced with more than 8 tokens";
    case QMM_ERR_WORKSPACE: return "QMM_ERR_WORKSPACE: workspace missing or smaller than the call's *_workspace_bytes";
    case QMM_ERR_SCRATCH:
      return "QMM_ERR_SCRATCH: the call needs more than the QMM_NOALLOC_SCRATCH_BYTES of scratch the no-allocation "
             "entry point holds";
    default: return "unknown qmm status";
  }
}

static int check_matmul(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
                        const void *X, int x_type, int64_t n_tokens, const float *Y, int path) {
  if (X == nullptr || Y == nullptr) return QMM_ERR_NULL;
  int st = check_weights(W, ggml_type, n_rows, k, row_stride_bytes);
  if (st != QMM_OK) return st;
  if (x_type != QMM_X_F32 && x_type != QMM_X_F16) return QMM_ERR_TYPE;
  if (n_tokens < 0 || n_tokens > kMaxDim) return QMM_ERR_SHAPE;
  if (!product_within(n_tokens, k, kMaxElems) || !product_within(n_tokens, n_rows, kMaxElems)) return QMM_ERR_SHAPE;
  if (path != QMM_PATH_AUTO && path != QMM_PATH_GEMV && path != QMM_PATH_GEMM) return QMM_ERR_PATH;
  if (path == QMM_PATH_GEMV && n_tokens > QMM_GEMV_MAX_TOKENS) return QMM_ERR_PATH;
  if (!aligned(X, 4) || !aligned(Y, 4)) return QMM_ERR_ALIGN;
  return QMM_OK;
}

int qmm_matmul_path(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes, const void *X,
                    int x_type, int64_t n_tokens, float *Y, int path, void *stream) {
  const int st = check_matmul(W, ggml_type, n_rows, k, row_stride_bytes, X, x_type, n_tokens, Y, path);
  if (st != QMM_OK) return st;
  if (n_rows == 0 || n_tokens == 0) return QMM_OK;

  const bool gemv = path == QMM_PATH_GEMV || (path == QMM_PATH_AUTO && n_tokens <= QMM_GEMV_MAX_TOKENS);
  const bool x_f16 = x_type == QMM_X_F16;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (trace_on())
    fprintf(stderr, "qmm: %s %s rows=%lld k=%lld nb1=%lld tokens=%lld x=%s align4=%d\n", gemv ? "gemv" : "gemm",
            type_name(ggml_type), (long long)n_rows, (long long)k, (long long)row_stride_bytes, (long long)n_tokens,
            x_f16 ? "f16" : "f32", (int)(aligned(W, 4) && row_stride_bytes % 4 == 0));
  if (gemv) {
    const qmm::MatmulDesc d{W, ggml_type, n_rows, k, row_stride_bytes, X, x_f16, n_tokens, Y};
    return status_of(qmm::launch_gemv_batch(&d, 1, s));
  }
  return status_of(qmm::launch_gemm(W, ggml_type, n_rows, k, row_stride_bytes, X, x_f16, n_tokens, Y, s));
}

int qmm_matmul(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes, const float *X,
               int64_t n_tokens, float *Y, void *stream) {
  return qmm_matmul_path(W, ggml_type, n_rows, k, row_stride_bytes, X, QMM_X_F32, n_tokens, Y, QMM_PATH_AUTO, stream);
}

int qmm_matmul_x16(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
                   const uint16_t *X, int64_t n_tokens, float *Y, void *stream) {
  return qmm_matmul_path(W, ggml_type, n_rows, k, row_stride_bytes, X, QMM_X_F16, n_tokens, Y, QMM_PATH_AUTO, stream);
}

int64_t qmm_matmul_workspace_bytes(int ggml_type, int64_t n_rows, int64_t k, int64_t n_tokens, int x_type) {
  const int bb = block_bytes(ggml_type), bw = block_weights(ggml_type);
  if (bb == 0 || (x_type != QMM_X_F32 && x_type != QMM_X_F16)) return QMM_ERR_TYPE;
  if (k <= 0 || k % bw != 0 || k > kMaxDim || n_rows < 0 || n_rows > kMaxDim || n_tokens < 0 || n_tokens > kMaxDim)
    return QMM_ERR_SHAPE;
  if (!product_within(n_tokens, k, kMaxElems) || !product_within(n_tokens, n_rows, kMaxElems)) return QMM_ERR_SHAPE;
  if (n_rows == 0 || n_tokens <= QMM_GEMV_MAX_TOKENS) return 0;
  return qmm::gemm_split_bytes(ggml_type, n_rows, k, n_tokens, x_type == QMM_X_F16);
}

int qmm_matmul_ws(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes, const void *X,
                  int x_type, int64_t n_tokens, float *Y, void *workspace, int64_t workspace_bytes, void *stream) {
  const int st = check_matmul(W, ggml_type, n_rows, k, row_stride_bytes, X, x_type, n_tokens, Y, QMM_PATH_AUTO);
  if (st != QMM_OK) return st;
  const int64_t need = qmm_matmul_workspace_bytes(ggml_type, n_rows, k, n_tokens, x_type);
  if (need < 0) return static_cast<int>(need);
  if (need == 0) return qmm_matmul_path(W, ggml_type, n_rows, k, row_stride_bytes, X, x_type, n_tokens, Y,
                                        QMM_PATH_AUTO, stream);
  if (workspace == nullptr || workspace_bytes < need) return QMM_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return QMM_ERR_ALIGN;
  if (trace_on())
    fprintf(stderr, "qmm: gemm split %s rows=%lld k=%lld nb1=%lld tokens=%lld workspace=%lld\n", type_name(ggml_type),
            (long long)n_rows, (long long)k, (long long)row_stride_bytes, (long long)n_tokens, (long long)need);
  return status_of(qmm::launch_gemm_split(W, ggml_type, n_rows, k, row_stride_bytes, static_cast<const _Float16 *>(X),
                                          n_tokens, Y, workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

namespace {

// The many-token MUL_MATs of a batch that can share one two-group launch:
// fp16 activations, the same type, rows, k, row stride and tokens, at most
// qmm::kGemmMaxItems of them, in the order of their first descriptor.
struct GemmGroup {
  std::vector<int> idx;
};

std::vector<GemmGroup> gemm_groups(const qmm_matmul_desc *descs, int count) {
  std::vector<GemmGroup> groups;
  for (int i = 0; i < count; ++i) {
    const qmm_matmul_desc &d = descs[i];
    if (d.n_rows == 0 || d.n_tokens <= QMM_GEMV_MAX_TOKENS) continue;
    GemmGroup *to = nullptr;
    if (d.x_type == QMM_X_F16)
      for (GemmGroup &g : groups) {
        const qmm_matmul_desc &f = descs[g.idx[0]];
        if (f.x_type == QMM_X_F16 && f.ggml_type == d.ggml_type && f.n_rows == d.n_rows && f.k == d.k &&
            f.row_stride_bytes == d.row_stride_bytes && f.n_tokens == d.n_tokens &&
            static_cast<int>(g.idx.size()) < qmm::kGemmMaxItems) {
          to = &g;
          break;
        }
      }
    if (to == nullptr) {
      groups.emplace_back();
      to = &groups.back();
    }
    to->idx.push_back(i);
  }
  return groups;
}

// Workspace of a group: its merged launch's split, or that of qmm_matmul_ws
// for a lone fp16 MUL_MAT.
int64_t group_bytes(const qmm_matmul_desc *descs, const GemmGroup &g) {
  const qmm_matmul_desc &d = descs[g.idx[0]];
  const int n = static_cast<int>(g.idx.size());
  if (n > 1 && qmm::gemm_items_merge(d.ggml_type, n, d.n_rows, d.k, d.n_tokens))
    return qmm::gemm_items_split_bytes(d.ggml_type, n, d.n_rows, d.k, d.n_tokens);
  int64_t most = 0;
  for (int i : g.idx) {
    const qmm_matmul_desc &e = descs[i];
    if (e.x_type == QMM_X_F16) most = std::max(most, qmm::gemm_split_bytes(e.ggml_type, e.n_rows, e.k, e.n_tokens, true));
  }
  return most;
}

int check_batch(const qmm_matmul_desc *descs, int count) {
  if (count < 0) return QMM_ERR_SHAPE;
  if (count > 0 && descs == nullptr) return QMM_ERR_NULL;
  for (int i = 0; i < count; ++i) {
    const qmm_matmul_desc &d = descs[i];
    const int st = check_matmul(d.W, d.ggml_type, d.n_rows, d.k, d.row_stride_bytes, d.X, d.x_type, d.n_tokens, d.Y,
                                QMM_PATH_AUTO);
    if (st != QMM_OK) return st;
  }
  return QMM_OK;
}

// The batch after validation; with a workspace (of at least the batch's
// size), many-token launches split as qmm_matmul_ws does.
int run_batch(const qmm_matmul_desc *descs, int count, void *workspace, int64_t workspace_bytes, hipStream_t s) {
  std::vector<qmm::MatmulDesc> gemv;
  gemv.reserve(count);
  for (int i = 0; i < count; ++i) {
    const qmm_matmul_desc &d = descs[i];
    if (d.n_rows == 0 || d.n_tokens == 0 || d.n_tokens > QMM_GEMV_MAX_TOKENS) continue;
    gemv.push_back(qmm::MatmulDesc{d.W, d.ggml_type, d.n_rows, d.k, d.row_stride_bytes, d.X,
                                   d.x_type == QMM_X_F16, d.n_tokens, d.Y});
  }
  int merged = 0;
  for (const GemmGroup &g : gemm_groups(descs, count)) {
    const qmm_matmul_desc &d = descs[g.idx[0]];
    const int n = static_cast<int>(g.idx.size());
    if (n > 1 && qmm::gemm_items_merge(d.ggml_type, n, d.n_rows, d.k, d.n_tokens)) {
      const void *w[qmm::kGemmMaxItems];
      const _Float16 *x[qmm::kGemmMaxItems];
      float *y[qmm::kGemmMaxItems];
      for (int j = 0; j < n; ++j) {
        w[j] = descs[g.idx[j]].W;
        x[j] = static_cast<const _Float16 *>(descs[g.idx[j]].X);
        y[j] = descs[g.idx[j]].Y;
      }
      if (trace_on())
        fprintf(stderr, "qmm: gemm of %d %s rows=%lld k=%lld tokens=%lld in one launch%s\n", n, type_name(d.ggml_type),
                (long long)d.n_rows, (long long)d.k, (long long)d.n_tokens,
                workspace != nullptr && qmm::gemm_items_split_bytes(d.ggml_type, n, d.n_rows, d.k, d.n_tokens) > 0
                    ? ", last round split"
                    : "");
      if (qmm::launch_gemm_items(w, d.ggml_type, n, d.n_rows, d.k, d.row_stride_bytes, x, d.n_tokens, y, workspace,
                                 workspace_bytes, s) != hipSuccess)
        return QMM_ERR_HIP;
      ++merged;
      continue;
    }
    for (int i : g.idx) {
      const qmm_matmul_desc &e = descs[i];
      const bool x_f16 = e.x_type == QMM_X_F16;
      hipError_t err;
      if (workspace != nullptr && x_f16 && qmm::gemm_split_bytes(e.ggml_type, e.n_rows, e.k, e.n_tokens, true) > 0)
        err = qmm::launch_gemm_split(e.W, e.ggml_type, e.n_rows, e.k, e.row_stride_bytes,
                                     static_cast<const _Float16 *>(e.X), e.n_tokens, e.Y, workspace, workspace_bytes, s);
      else
        err = qmm::launch_gemm(e.W, e.ggml_type, e.n_rows, e.k, e.row_stride_bytes, e.X, x_f16, e.n_tokens, e.Y, s);
      if (err != hipSuccess) return QMM_ERR_HIP;
    }
  }
  if (trace_on()) fprintf(stderr, "qmm: batch of %d (%zu decode-sized, %d merged gemm launches)\n", count, gemv.size(), merged);
  if (gemv.empty()) return QMM_OK;
  return status_of(qmm::launch_gemv_batch(gemv.data(), static_cast<int>(gemv.size()), s));
}

}  // namespace

int qmm_matmul_batch(const qmm_matmul_desc *descs, int count, void *stream) {
  const int st = check_batch(descs, count);
  if (st != QMM_OK || count == 0) return st;
  return run_batch(descs, count, nullptr, 0, static_cast<hipStream_t>(stream));
}

int64_t qmm_matmul_batch_workspace_bytes(const qmm_matmul_desc *descs, int count) {
  const int st = check_batch(descs, count);
  if (st != QMM_OK) return st;
  int64_t most = 0;
  for (const GemmGroup &g : gemm_groups(descs, count)) most = std::max(most, group_bytes(descs, g));
  return most;
}

int qmm_matmul_batch_ws(const qmm_matmul_desc *descs, int count, void *workspace, int64_t workspace_bytes,
                        void *stream) {
  const int64_t need = qmm_matmul_batch_workspace_bytes(descs, count);
  if (need < 0) return static_cast<int>(need);
  if (count == 0) return QMM_OK;
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return QMM_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return QMM_ERR_ALIGN;
  }
  return run_batch(descs, count, need > 0 ? workspace : nullptr, workspace_bytes, static_cast<hipStream_t>(stream));
}

int qmm_dequantize(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes, float *out,
                   void *stream) {
  if (out == nullptr) return QMM_ERR_NULL;
  int st = check_weights(W, ggml_type, n_rows, k, row_stride_bytes);
  if (st != QMM_OK) return st;
  if (!product_within(n_rows, k, kMaxElems)) return QMM_ERR_SHAPE;
  if (!aligned(out, 4)) return QMM_ERR_ALIGN;
  if (n_rows == 0) return QMM_OK;
  if (trace_on())
    fprintf(stderr, "qmm: dequant %s rows=%lld k=%lld nb1=%lld\n", type_name(ggml_type), (long long)n_rows,
            (long long)k, (long long)row_stride_bytes);
  return status_of(qmm::launch_dequant(W, ggml_type, n_rows, k, row_stride_bytes, out, static_cast<hipStream_t>(stream)));
}

int qmm_get_rows(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
                 const int32_t *ids, int64_t n_ids, float *out, void *stream) {
  if (ids == nullptr || out == nullptr) return QMM_ERR_NULL;
  int st = check_weights(W, ggml_type, n_rows, k, row_stride_bytes);
  if (st != QMM_OK) return st;
  if (n_ids < 0 || n_ids > kMaxDim || !product_within(n_ids, k, kMaxElems)) return QMM_ERR_SHAPE;
  if (!aligned(ids, 4) || !aligned(out, 4)) return QMM_ERR_ALIGN;
  if (n_ids == 0) return QMM_OK;
  if (trace_on())
    fprintf(stderr, "qmm: get_rows %s rows=%lld k=%lld nb1=%lld ids=%lld\n", type_name(ggml_type), (long long)n_rows,
            (long long)k, (long long)row_stride_bytes, (long long)n_ids);
  return status_of(qmm::launch_get_rows(W, ggml_type, n_rows, k, row_stride_bytes, ids, n_ids, out,
                                        static_cast<hipStream_t>(stream)));
}

// MUL_MAT_ID routes, chosen from the sizes alone (ids are device data):
//  * per pair: every (token, slot) pair is a single-token product on the
//    decode kernels (one token, or about one pair per selected expert);
//  * tiles: pairs bucketed by expert, the streaming decode kernel runs
//    tiles of 2, 4 or 8 pairs of one expert as token slots (the tile size
//    is the average pairs per expert, rounded up to a slot count);
//  * gemm: more tokens than the decode kernels take and at least 4 pairs
//    per expert on average: 128-pair tiles on the matrix cores (a selected
//    expert costs about as much as 3 to 4 single-token passes over its
//    weights whatever its pair count up to 128).
// The grouped routes need the workspace and count experts in LDS.
struct IdPlan {
  enum Route { kPerPair, kTiles, kGemm } route;
  int tile;
};
static IdPlan id_plan(int64_t n_experts, int64_t n_ids, int64_t n_tokens) {
  const int64_t pairs = n_ids * n_tokens;
  const int64_t used = n_experts < pairs ? n_experts : pairs;
  if (n_experts > qmm::kRouteMaxExperts || n_tokens < 2 || used == 0) return {IdPlan::kPerPair, 0};
  if (n_tokens > QMM_GEMV_MAX_TOKENS && pairs >= 4 * used) return {IdPlan::kGemm, qmm::kTileTokens};
  const int64_t avg = (pairs + used - 1) / used;
  if (avg < 2) return {IdPlan::kPerPair, 0};
  return {IdPlan::kTiles, avg <= 2 ? 2 : avg <= 4 ? 4 : 8};
}

int64_t qmm_matmul_id_workspace_bytes(int64_t n_experts, int64_t n_ids, int64_t n_tokens) {
  if (n_experts < 0 || n_experts > kMaxDim || n_ids < 0 || n_tokens < 0) return QMM_ERR_SHAPE;
  if (n_ids > 0 && n_tokens > kMaxDim / n_ids) return QMM_ERR_SHAPE;
  if (n_ids == 0) return 0;
  const IdPlan plan = id_plan(n_experts, n_ids, n_tokens);
  if (plan.route == IdPlan::kPerPair) return 0;
  return qmm::route_workspace_bytes(n_experts, n_ids * n_tokens, plan.tile);
}

int64_t qmm_matmul_id_workspace_bytes_x16(int64_t n_experts, int64_t n_ids, int64_t n_tokens, int64_t k,
                                          int64_t x_slots) {
  const int64_t base = qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens);
  if (base < 0) return base;
  if (k <= 0 || k > kMaxDim || (x_slots != 1 && x_slots != n_ids)) return QMM_ERR_SHAPE;
  const IdPlan plan = id_plan(n_experts, n_ids, n_tokens);
  if (plan.route != IdPlan::kGemm) return base;
  if (n_tokens > kMaxDim / (x_slots * k)) return QMM_ERR_SHAPE;
  return base + qmm::route_x16_bytes(n_tokens, x_slots, k);
}

// Checks of a MUL_MAT_ID call, all on the host, except those of the
// workspace; fills in the route and the workspace the sizes call for.
static int check_matmul_id(const void *W, int ggml_type, int64_t n_experts, int64_t n_rows, int64_t k,
                           int64_t row_stride_bytes, int64_t expert_stride_bytes, const float *X, int64_t x_slots,
                           const int32_t *ids, int64_t n_ids, int64_t n_tokens, const float *Y, IdPlan *plan,
                           int64_t *need) {
  if (X == nullptr || ids == nullptr || Y == nullptr) return QMM_ERR_NULL;
  int st = check_weights(W, ggml_type, n_rows, k, row_stride_bytes);
  if (st != QMM_OK) return st;
  *need = qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens);
  if (*need < 0) return static_cast<int>(*need);
  if (x_slots != 1 && x_slots != n_ids) return QMM_ERR_SHAPE;
  if (expert_stride_bytes % 2 != 0 || expert_stride_bytes < n_rows * row_stride_bytes) return QMM_ERR_STRIDE;
  if (!product_within(n_experts, expert_stride_bytes, kMaxBytes) ||
      !product_within(n_tokens * x_slots, k, kMaxElems) || !product_within(n_tokens * n_ids, n_rows, kMaxElems))
    return QMM_ERR_SHAPE;
  if (ggml_type == QMM_TYPE_Q4_K && expert_stride_bytes % 16 != 0) return QMM_ERR_STRIDE;
  if (!aligned(X, 4) || !aligned(ids, 4) || !aligned(Y, 4)) return QMM_ERR_ALIGN;
  *plan = id_plan(n_experts, n_ids, n_tokens);
  const bool streamable = qmm::id_streamable(W, n_rows, k, row_stride_bytes, expert_stride_bytes);
  // the tile form reads X through one 32-bit buffer and needs the streaming layout
  if (plan->route == IdPlan::kTiles && (!streamable || n_tokens * x_slots > ((int64_t{1} << 32) - 1) / (4 * k)))
    *plan = {IdPlan::kPerPair, 0};
  if (plan->route != IdPlan::kPerPair) {
    const int64_t row_tiles = plan->route == IdPlan::kGemm ? (n_rows + 127) / 128 : 1;
    if (row_tiles * qmm::route_max_tiles(n_experts, n_ids * n_tokens, plan->tile) > kMaxDim) return QMM_ERR_SHAPE;
  }
  return QMM_OK;
}

// Enqueue a checked MUL_MAT_ID call; `workspace` holds at least the bytes
// check_matmul_id reported when the route is a grouped one.
static int run_matmul_id(const void *W, int ggml_type, int64_t n_experts, int64_t n_rows, int64_t k,
                         int64_t row_stride_bytes, int64_t expert_stride_bytes, const float *X, int64_t x_slots,
                         const int32_t *ids, int64_t n_ids, int64_t n_tokens, float *Y, void *workspace,
                         int64_t workspace_bytes, const IdPlan &plan, hipStream_t s) {
  const bool grouped = plan.route != IdPlan::kPerPair;
  const bool streaming = !grouped && qmm::id_streamable(W, n_rows, k, row_stride_bytes, expert_stride_bytes);
  if (trace_on())
    fprintf(stderr, "qmm: matmul_id %s %s experts=%lld rows=%lld k=%lld nb1=%lld nb2=%lld ids=%lld tokens=%lld\n",
            plan.route == IdPlan::kGemm ? "grouped-gemm" : plan.route == IdPlan::kTiles ? "grouped-decode"
            : streaming ? "stream" : "general", type_name(ggml_type), (long long)n_experts,
            (long long)n_rows, (long long)k, (long long)row_stride_bytes, (long long)expert_stride_bytes,
            (long long)n_ids, (long long)n_tokens);
  if (grouped)
    return status_of(qmm::launch_matmul_id_grouped(W, ggml_type, n_experts, n_rows, k, row_stride_bytes,
                                                   expert_stride_bytes, X, x_slots, ids, n_ids, n_tokens, Y,
                                                   workspace, workspace_bytes, plan.tile, s));
  if (streaming)
    return status_of(qmm::launch_gemv_id_stream(W, ggml_type, n_experts, n_rows, k, row_stride_bytes,
                                                expert_stride_bytes, X, x_slots, ids, n_ids, n_tokens, Y, s));
  return status_of(qmm::launch_gemv_id_general(W, ggml_type, n_experts, n_rows, k, row_stride_bytes,
                                              expert_stride_bytes, X, x_slots, ids, n_ids, n_tokens, Y, s));
}

int qmm_matmul_id(const void *W, int ggml_type, int64_t n_experts, int64_t n_rows, int64_t k,
                  int64_t row_stride_bytes, int64_t expert_stride_bytes, const float *X, int64_t x_slots,
                  const int32_t *ids, int64_t n_ids, int64_t n_tokens, float *Y, void *workspace,
                  int64_t workspace_bytes, void *stream) {
  IdPlan plan{IdPlan::kPerPair, 0};
  int64_t need = 0;
  const int st = check_matmul_id(W, ggml_type, n_experts, n_rows, k, row_stride_bytes, expert_stride_bytes, X,
                                 x_slots, ids, n_ids, n_tokens, Y, &plan, &need);
  if (st != QMM_OK) return st;
  if (n_rows == 0 || n_ids == 0 || n_tokens == 0) return QMM_OK;
  if (plan.route != IdPlan::kPerPair) {
    if (workspace == nullptr || workspace_bytes < need) return QMM_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return QMM_ERR_ALIGN;
  }
  return run_matmul_id(W, ggml_type, n_experts, n_rows, k, row_stride_bytes, expert_stride_bytes, X, x_slots, ids,
                       n_ids, n_tokens, Y, workspace, workspace_bytes, plan, static_cast<hipStream_t>(stream));
}

int qmm_matmul_id_noalloc(const void *W, int ggml_type, int64_t n_experts, int64_t n_rows, int64_t k,
                          int64_t row_stride_bytes, int64_t expert_stride_bytes, const float *X, int64_t x_slots,
                          const int32_t *ids, int64_t n_ids, int64_t n_tokens, float *Y, void *stream) {
  IdPlan plan{IdPlan::kPerPair, 0};
  int64_t need = 0;
  const int st = check_matmul_id(W, ggml_type, n_experts, n_rows, k, row_stride_bytes, expert_stride_bytes, X,
                                 x_slots, ids, n_ids, n_tokens, Y, &plan, &need);
  if (st != QMM_OK) return st;
  if (need > QMM_NOALLOC_SCRATCH_BYTES) return QMM_ERR_SCRATCH;
  if (n_rows == 0 || n_ids == 0 || n_tokens == 0) return QMM_OK;
  void *ws = nullptr;
  if (plan.route != IdPlan::kPerPair) {
    ws = device_scratch();
    if (ws == nullptr) return QMM_ERR_HIP;
  }
  return run_matmul_id(W, ggml_type, n_experts, n_rows, k, row_stride_bytes, expert_stride_bytes, X, x_slots, ids,
                       n_ids, n_tokens, Y, ws, ws ? QMM_NOALLOC_SCRATCH_BYTES : 0, plan,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"
