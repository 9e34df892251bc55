// Grouped MUL_MAT_ID: the (token, slot) pairs are bucketed by expert on the
// GPU, then either the matrix-core kernel runs one tile per (weight row tile,
// 128 pairs of one expert) or, for decode-sized calls, the streaming decode
// kernel runs tiles of 2, 4 or 8 pairs of one expert as token slots; each
// selected expert's weights are read once per tile instead of once per pair.
//
// What is computed: the expert-routed MUL_MAT of [Load] "llama.cpp 源码完全拆解
// (三)：GGUF 装载、mmap 与张量放置", section "第六步：能力校验" (the probe's
// GGML_OP_MUL_MAT_ID case: activations F32 [k, n_ids, 512], ids I32
// [n_ids, 512]); the 512-token batch is what makes grouping pay.
//
// Routing (one 1024-thread workgroup, or one wavefront for up to 64 experts
// and 1024 pairs; ids are device data): count the pairs
// per expert in LDS, scan the counts into list offsets and token-tile
// offsets, write the tile table (expert, first list entry, count <= tile,
// number of tiles in the table) padded with empty tiles up to the host's
// bound, then place every pair in its
// expert's bucket. Pairs whose id names no expert go after the valid ones
// and get rows of NaN. Within a bucket the order depends on LDS atomics; a
// pair's result does not, because every output element is the same
// fixed-order sum whichever column of a tile its pair occupies.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace qmm {

namespace {

// fp32 -> fp16 copy of the activations for the two-group routed kernel
// (round to nearest even, the conversion the one-group kernel applies while
// staging), four values per step, by the routing launch's workgroups after
// the first, grid-stride over them: the copy runs beside the routing.
__device__ __forceinline__ void x16_convert(const float *__restrict__ X, _Float16 *__restrict__ Xh, int64_t n4) {
  const int64_t stride = static_cast<int64_t>(gridDim.x - 1) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x - 1) * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4_t f = reinterpret_cast<const float4_a4 *>(X)[i];
    const half2_t a = cvt_half2(f.x, f.y), b = cvt_half2(f.z, f.w);
    reinterpret_cast<u32x2_a4 *>(Xh)[i] = u32x2_a4{as_u32(a), as_u32(b)};
  }
}

constexpr int kRouteThreads = 1024;
constexpr int kPerThread = kRouteMaxExperts / kRouteThreads;
static_assert(kRouteMaxExperts % kRouteThreads == 0, "experts split evenly over the threads");

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t *__restrict__ ids, int n_pairs,
                                                              int n_experts, int max_tiles, int tile,
                                                              int32_t *__restrict__ list, int32_t *__restrict__ tiles,
                                                              float *__restrict__ Y, int n_rows, const float *X,
                                                              _Float16 *Xh, int64_t n4) {
  if (blockIdx.x > 0) {  // the activation copy's workgroups
    x16_convert(X, Xh, n4);
    return;
  }
  __shared__ int cnt[kRouteMaxExperts];
  __shared__ int cur[kRouteMaxExperts];
  __shared__ int scan_c[2][kRouteThreads];
  __shared__ int scan_t[2][kRouteThreads];
  __shared__ int bad_cur;
  const int tid = threadIdx.x;
  for (int e = tid; e < kRouteMaxExperts; e += kRouteThreads) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < n_pairs; p += kRouteThreads) {
    const int e = ids[p];
    if (e >= 0 && e < n_experts) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();

  // Thread tid owns experts [kPerThread tid, kPerThread (tid + 1)): its pair
  // and tile sums, then an inclusive scan over the threads (Hillis-Steele).
  int c_own = 0, t_own = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int c = cnt[kPerThread * tid + i];
    c_own += c;
    t_own += (c + tile - 1) / tile;
  }
  scan_c[0][tid] = c_own;
  scan_t[0][tid] = t_own;
  __syncthreads();
  int src = 0;
  for (int d = 1; d < kRouteThreads; d *= 2) {
    const int dst = src ^ 1;
    scan_c[dst][tid] = scan_c[src][tid] + (tid >= d ? scan_c[src][tid - d] : 0);
    scan_t[dst][tid] = scan_t[src][tid] + (tid >= d ? scan_t[src][tid - d] : 0);
    __syncthreads();
    src = dst;
  }
  int off = scan_c[src][tid] - c_own, toff = scan_t[src][tid] - t_own;
  const int n_valid = scan_c[src][kRouteThreads - 1], n_tiles = scan_t[src][kRouteThreads - 1];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int e = kPerThread * tid + i, c = cnt[e];
    cur[e] = off;
    for (int j = 0; j * tile < c; ++j, ++toff) {
      int32_t *t = tiles + 4 * static_cast<int64_t>(toff);
      t[0] = e;
      t[1] = off + j * tile;
      t[2] = min(tile, c - j * tile);
      t[3] = n_tiles;
    }
    off += c;
  }
  for (int i = n_tiles + tid; i < max_tiles; i += kRouteThreads) {
    int32_t *t = tiles + 4 * static_cast<int64_t>(i);
    t[0] = 0, t[1] = 0, t[2] = 0, t[3] = n_tiles;  // empty: its workgroups exit at once
  }
  if (tid == 0) bad_cur = n_valid;
  __syncthreads();

  for (int p = tid; p < n_pairs; p += kRouteThreads) {
    const int e = ids[p];
    const int pos = (e >= 0 && e < n_experts) ? atomicAdd(&cur[e], 1) : atomicAdd(&bad_cur, 1);
    list[pos] = p;
  }
  __syncthreads();  // the bucket writes above are visible to the whole workgroup
  for (int i = n_valid; i < n_pairs; ++i) {
    float *y = Y + static_cast<int64_t>(list[i]) * n_rows;
    for (int r = tid; r < n_rows; r += kRouteThreads) y[r] = __builtin_bit_cast(float, 0x7FC00000u);
  }
}

// The same routing for calls with few experts and pairs (a decode step of a
// small-expert MoE): one wavefront, every id held in registers, the scan done
// with cross-lane shuffles, so the kernel runs no workgroup-wide scans and
// only three barriers. Expert e is lane e's.
constexpr int kSmallExperts = 64;
constexpr int kSmallPairsPerLane = 16;
constexpr int kSmallPairs = 64 * kSmallPairsPerLane;

__global__ __launch_bounds__(64) void route_small_kernel(const int32_t *__restrict__ ids, int n_pairs, int n_experts,
                                                         int max_tiles, int tile, int32_t *__restrict__ list,
                                                         int32_t *__restrict__ tiles, float *__restrict__ Y,
                                                         int n_rows, const float *X, _Float16 *Xh, int64_t n4) {
  if (blockIdx.x > 0) {  // the activation copy's workgroups
    x16_convert(X, Xh, n4);
    return;
  }
  __shared__ int cnt[kSmallExperts];
  __shared__ int cur[kSmallExperts];
  __shared__ int bad_cur;
  const int lane = threadIdx.x;
  int e[kSmallPairsPerLane];
#pragma unroll
  for (int i = 0; i < kSmallPairsPerLane; ++i) {
    const int p = lane + 64 * i;
    e[i] = p < n_pairs ? ids[p] : -1;
  }
  cnt[lane] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSmallPairsPerLane; ++i)
    if (e[i] >= 0 && e[i] < n_experts) atomicAdd(&cnt[e[i]], 1);
  __syncthreads();

  const int c = lane < n_experts ? cnt[lane] : 0;
  const int t = (c + tile - 1) / tile;
  int ci = c, ti = t;  // inclusive scans over the lanes
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int cu = __shfl_up(ci, d), tu = __shfl_up(ti, d);
    if (lane >= d) ci += cu, ti += tu;
  }
  const int off = ci - c, toff = ti - t;
  const int n_valid = __shfl(ci, 63), n_tiles = __shfl(ti, 63);
  cur[lane] = off;
  for (int j = 0; j < t; ++j) {
    int32_t *q = tiles + 4 * static_cast<int64_t>(toff + j);
    q[0] = lane;
    q[1] = off + j * tile;
    q[2] = min(tile, c - j * tile);
    q[3] = n_tiles;
  }
  for (int i = n_tiles + lane; i < max_tiles; i += 64) {
    int32_t *q = tiles + 4 * static_cast<int64_t>(i);
    q[0] = 0, q[1] = 0, q[2] = 0, q[3] = n_tiles;  // empty: its workgroups exit at once
  }
  if (lane == 0) bad_cur = n_valid;
  __syncthreads();

#pragma unroll
  for (int i = 0; i < kSmallPairsPerLane; ++i) {
    const int p = lane + 64 * i;
    if (p < n_pairs) {
      const bool ok = e[i] >= 0 && e[i] < n_experts;
      list[ok ? atomicAdd(&cur[e[i]], 1) : atomicAdd(&bad_cur, 1)] = p;
    }
  }
  __syncthreads();  // the bucket writes above are visible to the whole wavefront
  for (int i = n_valid; i < n_pairs; ++i) {
    float *y = Y + static_cast<int64_t>(list[i]) * n_rows;
    for (int r = lane; r < n_rows; r += 64) y[r] = __builtin_bit_cast(float, 0x7FC00000u);
  }
}

}  // namespace

int64_t route_x16_bytes(int64_t n_tokens, int64_t x_slots, int64_t k) { return n_tokens * x_slots * k * 2; }

int64_t route_max_tiles(int64_t n_experts, int64_t n_pairs, int tile) {
  // sum over experts of ceil(count / tile) <= n_pairs / tile + (experts used)
  return (n_pairs + tile - 1) / tile + (n_experts < n_pairs ? n_experts : n_pairs);
}

int64_t route_workspace_bytes(int64_t n_experts, int64_t n_pairs, int tile) {
  return (n_pairs * 4 + 15) / 16 * 16 + 16 * route_max_tiles(n_experts, n_pairs, tile);
}

hipError_t launch_matmul_id_grouped(const void *W, int qtype, int64_t n_experts, int64_t n_rows, int64_t k,
                                    int64_t nb1, int64_t nb2, const float *X, int64_t x_slots, const int32_t *ids,
                                    int64_t n_ids, int64_t n_tokens, float *Y, void *workspace,
                                    int64_t workspace_bytes, int tile, hipStream_t stream) {
  const int64_t n_pairs = n_tokens * n_ids;
  // The matrix-core route runs the two-group kernel, on wider tiles, when
  // the workspace also holds the fp16 copy of X (after the routing table,
  // whose size for kTileTokens bounds the wider tiles' table too) and the
  // tile pairs fill the GPU.
  _Float16 *Xh = nullptr;
  if (tile == kTileTokens) {
    const int64_t route_bytes = route_workspace_bytes(n_experts, n_pairs, tile);
    const int64_t x16 = route_x16_bytes(n_tokens, x_slots, k);
    if (workspace_bytes >= route_bytes + x16 &&
        routed_two_group(qtype, k, n_rows, route_max_tiles(n_experts, n_pairs, kTileTokensTwoGroup), device_cus())) {
      Xh = reinterpret_cast<_Float16 *>(static_cast<char *>(workspace) + route_bytes);
      tile = kTileTokensTwoGroup;
    }
  }
  const int64_t max_tiles = route_max_tiles(n_experts, n_pairs, tile);
  int32_t *list = static_cast<int32_t *>(workspace);
  int32_t *tiles = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + (n_pairs * 4 + 15) / 16 * 16);
  const bool small = n_experts <= kSmallExperts && n_pairs <= kSmallPairs;
  // workgroup 0 routes; with Xh, workgroups 1.. make the fp16 copy of X,
  // about four float4 per thread
  const int block = small ? 64 : kRouteThreads;
  const int64_t n4 = Xh != nullptr ? n_tokens * x_slots * k / 4 : 0;
  const int64_t conv = std::min<int64_t>((n4 + 4 * block - 1) / (4 * block), 4096);
  const dim3 grid(static_cast<unsigned>(1 + conv));
  hipError_t e = small ? launch(route_small_kernel, grid, dim3(64), 0, stream, ids, static_cast<int>(n_pairs),
                                static_cast<int>(n_experts), static_cast<int>(max_tiles), tile, list, tiles, Y,
                                static_cast<int>(n_rows), X, Xh, n4)
                       : launch(route_kernel, grid, dim3(kRouteThreads), 0, stream, ids, static_cast<int>(n_pairs),
                                static_cast<int>(n_experts), static_cast<int>(max_tiles), tile, list, tiles, Y,
                                static_cast<int>(n_rows), X, Xh, n4);
  if (e != hipSuccess) return e;
  if (tile == kTileTokens || tile == kTileTokensTwoGroup)
    return launch_gemm_routed(W, qtype, n_rows, k, nb1, nb2, X, Xh, x_slots, n_ids, list, tiles, max_tiles, Y,
                              stream);
  return launch_gemv_id_tiles(W, qtype, n_experts, n_rows, k, nb1, nb2, X, x_slots, n_ids, n_tokens, list, tiles,
                              max_tiles, tile, Y, stream);
}

}  // namespace qmm
