// Internal launch interface between the C ABI (qmm_api.hip) and the kernel
// translation units. Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <tuple>
#include <utility>

namespace qmm {

// hipLaunchKernel returns its status directly, so a launch error is reported
// without touching (or clearing) any earlier sticky error of the caller.
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                  Args &&...args) {
  std::tuple<KArgs...> values(std::forward<Args>(args)...);
  return std::apply(
      [&](auto &...v) {
        void *argv[] = {static_cast<void *>(&v)...};
        return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, shmem, stream);
      },
      values);
}

// CUs of the current device (read once per device; 0 if HIP cannot tell).
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (v > 0) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

hipError_t launch_dequant(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, float *out,
                          hipStream_t stream);
hipError_t launch_get_rows(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const int32_t *ids,
                           int64_t n_ids, float *out, hipStream_t stream);

// One MUL_MAT of a (possibly batched) call.
struct MatmulDesc {
  const void *W;
  int qtype;
  int64_t n_rows, k, nb1;
  const void *X;
  bool x_f16;
  int64_t n_tokens;
  float *Y;
};

// Decode kernels, 1 <= n_tokens <= QMM_GEMV_MAX_TOKENS. launch_gemv_batch runs
// `count` independent MUL_MATs, grouping those the streaming kernel can take
// into shared launches; the rest go one by one to the general kernel.
hipError_t launch_gemv_batch(const MatmulDesc *d, int count, hipStream_t stream);
hipError_t launch_gemv_general(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const void *X,
                               bool x_f16, int64_t n_tokens, float *Y, hipStream_t stream);

// Expert-routed decode (MUL_MAT_ID): one single-token product per
// (token, slot) pair, against expert ids[pair] of a stack of n_experts
// matrices expert_stride bytes apart. The streaming kernel takes stacks that
// id_streamable accepts, the general kernel any valid layout.
bool id_streamable(const void *W, int64_t n_rows, int64_t k, int64_t nb1, int64_t nb2);
hipError_t launch_gemv_id_stream(const void *W, int qtype, int64_t n_experts, int64_t n_rows, int64_t k, int64_t nb1,
                                 int64_t nb2, const float *X, int64_t x_slots, const int32_t *ids, int64_t n_ids,
                                 int64_t n_tokens, float *Y, hipStream_t stream);
hipError_t launch_gemv_id_general(const void *W, int qtype, int64_t n_experts, int64_t n_rows, int64_t k, int64_t nb1,
                                  int64_t nb2, const float *X, int64_t x_slots, const int32_t *ids, int64_t n_ids,
                                  int64_t n_tokens, float *Y, hipStream_t stream);

// Grouped expert-routed product for many tokens: a routing kernel buckets the
// pairs by expert into the workspace (route_workspace_bytes of it), then the
// matrix-core kernel runs tiles of kTileTokens pairs of one expert. Experts
// are counted in LDS, so n_experts <= kRouteMaxExperts.
constexpr int kTileTokens = 128;
constexpr int kRouteMaxExperts = 4096;
// Tiles hold up to `tile` pairs of one expert: kTileTokens for the
// matrix-core kernel, 2, 4 or 8 for the decode kernel's tile form.
int64_t route_max_tiles(int64_t n_experts, int64_t n_pairs, int tile);
int64_t route_workspace_bytes(int64_t n_experts, int64_t n_pairs, int tile);
// With the matrix-core tiles, a workspace of at least route_workspace_bytes
// + route_x16_bytes also holds an fp16 copy of X (after the routing table),
// which lets the two-group kernel run; results are the same bits.
int64_t route_x16_bytes(int64_t n_tokens, int64_t x_slots, int64_t k);
hipError_t launch_matmul_id_grouped(const void *W, int qtype, int64_t n_experts, int64_t n_rows, int64_t k,
                                    int64_t nb1, int64_t nb2, const float *X, int64_t x_slots, const int32_t *ids,
                                    int64_t n_ids, int64_t n_tokens, float *Y, void *workspace,
                                    int64_t workspace_bytes, int tile, hipStream_t stream);
hipError_t launch_gemv_id_tiles(const void *W, int qtype, int64_t n_experts, int64_t n_rows, int64_t k, int64_t nb1,
                                int64_t nb2, const float *X, int64_t x_slots, int64_t n_ids, int64_t n_tokens,
                                const int32_t *list, const int32_t *tiles, int64_t max_tiles, int nt, float *Y,
                                hipStream_t stream);
// The routed matrix-core product. Without Xh, the one-group kernel on fp32 X
// over tiles of at most kTileTokens pairs. With Xh (an fp16 copy of X), the
// two-group kernel, two tiles per workgroup, over tiles of at most
// kTileTokensTwoGroup pairs; the caller routes with that tile size when
// routed_two_group (given the larger tile's max_tiles) holds.
constexpr int kTileTokensTwoGroup = 160;
bool routed_two_group(int qtype, int64_t k, int64_t n_rows, int64_t max_tiles, int64_t cus);
hipError_t launch_gemm_routed(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, int64_t nb2,
                              const float *X, const _Float16 *Xh, int64_t x_slots, int64_t n_ids,
                              const int32_t *list, const int32_t *tiles, int64_t max_tiles, float *Y,
                              hipStream_t stream);

// Matrix-core kernel, any n_tokens >= 1.
hipError_t launch_gemm(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const void *X, bool x_f16,
                       int64_t n_tokens, float *Y, hipStream_t stream);
// The two-group kernel with k split across workgroups, for launches of few
// tiles with long k: gemm_split_bytes is the workspace it needs (per-tile
// counters, zero between calls, then partial tiles), 0 for shapes it does
// not take (then launch_gemm's choice holds).
int64_t gemm_split_bytes(int qtype, int64_t n_rows, int64_t k, int64_t n_tokens, bool x_f16);
hipError_t launch_gemm_split(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const _Float16 *X,
                             int64_t n_tokens, float *Y, void *workspace, int64_t workspace_bytes,
                             hipStream_t stream);
// Up to kGemmMaxItems MUL_MATs of one type and shape (rows, k, row stride,
// tokens; fp16 activations) in one two-group launch, their row tiles one
// after another. gemm_items_merge: the launch is worth making (its tiles
// suit the two-group kernel, or its last round splits).
// gemm_items_split_bytes: the workspace that lets the launch split its last
// round's tiles in k (0 if it does not). launch_gemm_items splits only with a
// workspace of at least that size; whole tiles give the same bits as the
// MUL_MATs launched one by one.
constexpr int kGemmMaxItems = 4;
bool gemm_items_merge(int qtype, int n_items, int64_t n_rows, int64_t k, int64_t n_tokens);
int64_t gemm_items_split_bytes(int qtype, int n_items, int64_t n_rows, int64_t k, int64_t n_tokens);
hipError_t launch_gemm_items(const void *const *W, int qtype, int n_items, int64_t n_rows, int64_t k, int64_t nb1,
                             const _Float16 *const *X, int64_t n_tokens, float *const *Y, void *workspace,
                             int64_t workspace_bytes, hipStream_t stream);

}  // namespace qmm
