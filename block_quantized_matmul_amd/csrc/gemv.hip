// Decode MUL_MAT (1 <= n_tokens <= 8), general layouts: any even row stride and
// 2-byte-aligned W. (16-byte-aligned layouts take the streaming kernel in
// gemv_stream.hip.) y[t][r] = sum_b d_rb * sum_i (q - z) x[t][32 b + i].
//
// What is computed: [Bind] "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section
// 2.3 (blocks are dequantised inside MUL_MAT, then multiplied) and [Arch]
// "llama.cpp 源码完全拆解(一)：整体架构与模块全景", section "权重装载：GGUF、mmap
// 与 4 bit 块" (w = s (q - z); the GPU kernels decode scale and integer weights
// per block and multiply-add them with activations in registers).
//
// Design (MI355X, gfx950). The kernel is bound by HBM: every weight byte is
// read exactly once. One workgroup owns 16 rows; its 8 or 16 wavefronts split the
// row's blocks into contiguous ranges and meet in LDS at the end, in a fixed
// order (no atomics, so results are bitwise reproducible).
//
// Latency hiding: each wavefront keeps kRing units of weights in flight on the
// vector-memory counter. The activations are staged once per workgroup into
// LDS as fp16, already in MFMA operand order, so reading them never waits on
// (and never drains) the weight stream. Activations that do not fit the LDS
// budget are staged in chunks of k.
//
// The dot products run on the matrix cores: one v_mfma_f32_16x16x32_f16 per
// block covers 16 rows x 32 weights x 16 token slots. The B operand holds the
// integer codes (q - z), exact in fp16; the A operand holds the activations
// rounded to fp16; each lane then applies its row's block scale d in fp32
// (acc += d * partial), so the weights enter the sum exactly. Lane l of the B
// operand serves row l % 16 and 8 elements of block-slice l / 16; the A
// operand uses the same element order, so each MFMA is exactly that block's
// partial dot product. D holds token 4 (l / 16) + e, row l % 16 in element e
// of lane l.
//
// Weight access (row start 4-byte aligned): a unit is a pair of blocks (36
// bytes Q4_0, 40 Q4_1, 44 Q5_0, 48 Q5_1, 68 Q8_0). The four lanes of a row load overlapping dword
// windows that together cover the pair once; the two scales are forwarded
// from the lanes that loaded them with ds_bpermute. Rows whose start is only
// 2-byte aligned take 16-bit loads, one block per unit.
#include "common.h"
#include "gemv_common.h"
#include "launch.h"

namespace qmm {

constexpr int kRing = 8;                  // weight units in flight per wavefront
constexpr int kXLdsBudget = 64 * 1024;    // bytes of LDS for staged activations

template <int QT, bool ALIGN4> struct GemvRaw;
// Q4_0 pair: dwords g, g + 1 (even block, codes start 2 bytes in) and 5 + g (odd block).
template <> struct GemvRaw<QMM_TYPE_Q4_0, true> { u32x2_t a; uint32_t b; };
// Q8_0 pair: dwords 2g .. 2g + 2 (even block) and 9 + 2g .. 10 + 2g (odd block).
template <> struct GemvRaw<QMM_TYPE_Q8_0, true> { uint32_t a0, a1, a2; u32x2_t b; };
// Q4_1 pair (40 bytes, both blocks dword-aligned): dwords g, g + 1 (even
// block: d|m in dword 0, codes in dwords 1..4) and 5 + g, 6 + g (odd block).
template <> struct GemvRaw<QMM_TYPE_Q4_1, true> { u32x2_t a, b; };
// Q5_0 pair (44 bytes; block 1 at byte 22): dwords 0-1 (d, fifth bits of
// block 0), 1 + g, 2 + g (its codes start at byte 6), 5-6 (d in the high
// half of dword 5, fifth bits in dword 6) and 7 + g (block 1's codes).
template <> struct GemvRaw<QMM_TYPE_Q5_0, true> { u32x2_t h0, c0, h1; uint32_t c1; };
// Q5_1 pair (48 bytes): dwords 0-1 (d|m, fifth bits), 2 + g, 6-7, 8 + g.
template <> struct GemvRaw<QMM_TYPE_Q5_1, true> { u32x2_t h0, h1; uint32_t c0, c1; };
// Single block, 16-bit loads: scale bits and the lane's code dwords.
template <> struct GemvRaw<QMM_TYPE_Q4_0, false> { uint32_t d, q; };
template <> struct GemvRaw<QMM_TYPE_Q8_0, false> { uint32_t d, q0, q1; };
template <> struct GemvRaw<QMM_TYPE_Q4_1, false> { uint32_t d, q; };  // d = d | m << 16
template <> struct GemvRaw<QMM_TYPE_Q5_0, false> { uint32_t d, h, q; };
template <> struct GemvRaw<QMM_TYPE_Q5_1, false> { uint32_t d, h, q; };  // d = d | m << 16

template <int QT, bool ALIGN4>
__device__ __forceinline__ GemvRaw<QT, ALIGN4> gemv_load(const uint8_t *rp, int u, int g) {
  GemvRaw<QT, ALIGN4> r;
  if constexpr (ALIGN4) {
    const uint8_t *p = rp + static_cast<int64_t>(u) * (2 * Block<QT>::bytes);
    if constexpr (QT == QMM_TYPE_Q4_0) {
      r.a = ld_u32x2(p + 4 * g);
      r.b = ld_u32(p + 20 + 4 * g);
    } else if constexpr (QT == QMM_TYPE_Q4_1) {
      r.a = ld_u32x2(p + 4 * g);
      r.b = ld_u32x2(p + 20 + 4 * g);
    } else if constexpr (QT == QMM_TYPE_Q5_0) {
      r.h0 = ld_u32x2(p);
      r.c0 = ld_u32x2(p + 4 + 4 * g);
      r.h1 = ld_u32x2(p + 20);
      r.c1 = ld_u32(p + 28 + 4 * g);
    } else if constexpr (QT == QMM_TYPE_Q5_1) {
      r.h0 = ld_u32x2(p);
      r.c0 = ld_u32(p + 8 + 4 * g);
      r.h1 = ld_u32x2(p + 24);
      r.c1 = ld_u32(p + 32 + 4 * g);
    } else {
      const u32x3_a4 a = *reinterpret_cast<const u32x3_a4 *>(p + 8 * g);
      r.a0 = a.x;
      r.a1 = a.y;
      r.a2 = a.z;
      r.b = ld_u32x2(p + 36 + 8 * g);
    }
  } else {
    const uint8_t *p = rp + static_cast<int64_t>(u) * Block<QT>::bytes;
    r.d = ld_u16(p);
    if constexpr (QT == QMM_TYPE_Q4_0) {
      r.q = ld_u16(p + 2 + 4 * g) | (ld_u16(p + 4 + 4 * g) << 16);
    } else if constexpr (QT == QMM_TYPE_Q4_1) {
      r.d |= ld_u16(p + 2) << 16;
      r.q = ld_u16(p + 4 + 4 * g) | (ld_u16(p + 6 + 4 * g) << 16);
    } else if constexpr (QTraits<QT>::has_qh) {
      constexpr int o = QTraits<QT>::qh, c = QTraits<QT>::codes;
      if constexpr (QTraits<QT>::has_min) r.d |= ld_u16(p + 2) << 16;
      r.h = ld_u16(p + o) | (ld_u16(p + o + 2) << 16);
      r.q = ld_u16(p + c + 4 * g) | (ld_u16(p + c + 2 + 4 * g) << 16);
    } else {
      r.q0 = ld_u16(p + 2 + 8 * g) | (ld_u16(p + 4 + 8 * g) << 16);
      r.q1 = ld_u16(p + 6 + 8 * g) | (ld_u16(p + 8 + 8 * g) << 16);
    }
  }
  return r;
}

// One unit: blocks 2u, 2u + 1 (pairs) or block u (single), global indices;
// xs is the staged chunk starting at block b_lo.
template <int QT, int NT, bool ALIGN4>
__device__ __forceinline__ void gemv_unit(float acc[4], const GemvRaw<QT, ALIGN4> &r, const half8_t *xs, int u,
                                          int b_lo, int g, int r16, int xslot) {
  if constexpr (ALIGN4) {
    const half8_t xe = xs[(4 * (2 * u - b_lo) + g) * NT + xslot];
    const half8_t xo = xs[(4 * (2 * u + 1 - b_lo) + g) * NT + xslot];
    if constexpr (QT == QMM_TYPE_Q4_0) {
      // Even block: scale = low half of dword 0 (lane g = 0's a.x); odd block:
      // scale = high half of dword 4 (lane g = 3's a.y).
      const uint32_t de = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * r16, static_cast<int>(r.a.x)));
      const uint32_t dd = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * (r16 + 48), static_cast<int>(r.a.y)));
      gemv_block<NT>(acc, xe, gemv_codes<QT>(shift16(r.a.x, r.a.y), 0), de & 0xFFFFu);
      gemv_block<NT>(acc, xo, gemv_codes<QT>(r.b, 0), dd >> 16);
    } else if constexpr (QT == QMM_TYPE_Q4_1) {
      // d|m of each block: dword 0 / dword 5 of the pair, held by lane g = 0
      // of the row (a.x / b.x).
      const uint32_t de = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * r16, static_cast<int>(r.a.x)));
      const uint32_t dd = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * r16, static_cast<int>(r.b.x)));
      gemv_block_min<NT>(acc, xe, gemv_codes<QT>(r.a.y, 0), de);
      gemv_block_min<NT>(acc, xo, gemv_codes<QT>(r.b.y, 0), dd);
    } else if constexpr (QT == QMM_TYPE_Q5_0) {
      gemv_block<NT>(acc, xe, gemv_codes5<QT>(shift16(r.c0.x, r.c0.y), shift16(r.h0.x, r.h0.y), 4 * g),
                     r.h0.x & 0xFFFFu);
      gemv_block<NT>(acc, xo, gemv_codes5<QT>(r.c1, r.h1.y, 4 * g), r.h1.x >> 16);
    } else if constexpr (QT == QMM_TYPE_Q5_1) {
      gemv_block_min<NT>(acc, xe, gemv_codes5<QT>(r.c0, r.h0.y, 4 * g), r.h0.x);
      gemv_block_min<NT>(acc, xo, gemv_codes5<QT>(r.c1, r.h1.y, 4 * g), r.h1.x);
    } else {
      // Even block: scale = low half of dword 0 (lane g = 0's a0); odd block
      // starts at byte 34: scale = high half of dword 8 (lane g = 3's a2).
      const uint32_t de = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * r16, static_cast<int>(r.a0)));
      const uint32_t dd = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * (r16 + 48), static_cast<int>(r.a2)));
      gemv_block<NT>(acc, xe, gemv_codes<QT>(shift16(r.a0, r.a1), shift16(r.a1, r.a2)), de & 0xFFFFu);
      gemv_block<NT>(acc, xo, gemv_codes<QT>(r.b.x, r.b.y), dd >> 16);
    }
  } else {
    const half8_t x = xs[(4 * (u - b_lo) + g) * NT + xslot];
    if constexpr (QT == QMM_TYPE_Q4_0)
      gemv_block<NT>(acc, x, gemv_codes<QT>(r.q, 0), r.d);
    else if constexpr (QT == QMM_TYPE_Q4_1)
      gemv_block_min<NT>(acc, x, gemv_codes<QT>(r.q, 0), r.d);
    else if constexpr (QTraits<QT>::has_qh)
      gemv_any_block<QT, NT>(acc, x, gemv_codes5<QT>(r.q, r.h, 4 * g), r.d);
    else
      gemv_block<NT>(acc, x, gemv_codes<QT>(r.q0, r.q1), r.d);
  }
}

// Dynamic LDS: the staged activations of one chunk, chunk_blocks * 64 * NT bytes.
// Expert routing (MUL_MAT_ID) when ids is not null: workgroup row y serves
// pair p = pair0 + blockIdx.y = (token p / n_ids, slot p % n_ids), whose
// matrix is expert ids[p] of the stack (stride nb2), activation row
// X[token][slot] (X[token][0] when x_slots == 1, fp32) and output Y[p]; an
// id outside [0, n_experts) gives a row of NaNs.
struct GemvRoute {
  const int32_t *ids;
  int64_t nb2;
  int n_experts, n_ids, x_slots, pair0;
};

template <int QT, int NT, bool XF16, bool ALIGN4, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void gemv_kernel(const uint8_t *__restrict__ W, int n_rows, int nblk,
                                                            int64_t nb1, const void *__restrict__ X, int n_tokens,
                                                            int k, float *__restrict__ Y, int chunk_blocks,
                                                            GemvRoute route) {
  extern __shared__ __attribute__((aligned(16))) half8_t xs[];
  __shared__ float red[WAVES][NT > 4 ? 32 : 16][4];
  if (route.ids != nullptr) {
    const int p = route.pair0 + static_cast<int>(blockIdx.y);
    const int e = __builtin_amdgcn_readfirstlane(route.ids[p]);
    const int t = p / route.n_ids, slot = p - t * route.n_ids;
    Y += static_cast<int64_t>(p) * n_rows;
    if (e < 0 || e >= route.n_experts) {
      const int row = static_cast<int>(blockIdx.x) * 16 + static_cast<int>(threadIdx.x);
      if (threadIdx.x < 16 && row < n_rows) Y[row] = __builtin_bit_cast(float, 0x7FC00000u);
      return;
    }
    W += static_cast<int64_t>(e) * route.nb2;
    X = static_cast<const float *>(X) + (static_cast<int64_t>(t) * route.x_slots + (route.x_slots > 1 ? slot : 0)) * k;
    n_tokens = 1;
  }

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar control flow
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  // Rows past the end read the last row (valid memory); their results are
  // dropped at the store. Token slots past n_tokens read the last staged
  // token; their D entries are never stored.
  const int row = min(row0 + r16, n_rows - 1);
  const uint8_t *rp = W + static_cast<int64_t>(row) * nb1;
  const int xslot = min(r16, n_tokens - 1);

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int b_lo = 0; b_lo < nblk; b_lo += chunk_blocks) {
    const int b_hi = min(nblk, b_lo + chunk_blocks);
    const int nu = ALIGN4 ? ((b_hi - b_lo) >> 1) : (b_hi - b_lo);
    const int ubase = ALIGN4 ? (b_lo >> 1) : b_lo;
    // Waves take contiguous ranges of 8-block groups when the chunk has
    // whole groups (as the streaming kernel does, so both kernels sum in
    // the same order and agree bitwise), else of units.
    const int upg = ALIGN4 ? 4 : 8;  // units per 8-block group
    const int span = ((b_hi - b_lo) & 7) == 0 ? upg : 1;
    const int ng = nu / span;
    const int u0 = ubase + span * static_cast<int>((static_cast<int64_t>(wave) * ng) / WAVES);
    const int u1 = ubase + span * static_cast<int>((static_cast<int64_t>(wave + 1) * ng) / WAVES);
    const bool has_units = u0 < u1;

    // Weight loads go out first, so the activation staging below overlaps
    // their latency. Ring indices are clamped to the wave's last unit so all
    // loads are in bounds.
    GemvRaw<QT, ALIGN4> ring[kRing];
    if (has_units) {
#pragma unroll
      for (int i = 0; i < kRing; ++i) ring[i] = gemv_load<QT, ALIGN4>(rp, min(u0 + i, u1 - 1), g);
    }
    if (b_lo > 0) __syncthreads();  // previous chunk's activations no longer read
    gemv_stage_x<QT, NT, XF16, 64 * WAVES>(xs, X, n_tokens, k, b_lo, b_hi);
    __syncthreads();

    if (has_units) {
      for (int base = u0; base < u1; base += kRing) {
#pragma unroll
        for (int i = 0; i < kRing; ++i) {
          const int u = base + i;
          if (u < u1) {
            gemv_unit<QT, NT, ALIGN4>(acc, ring[i], xs, u, b_lo, g, r16, xslot);
            ring[i] = gemv_load<QT, ALIGN4>(rp, min(u + kRing, u1 - 1), g);
          }
        }
      }
    }
    if (ALIGN4 && ((b_hi - b_lo) & 1) && wave == WAVES - 1) {
      // Odd block count in this chunk (only the last one): the final block
      // starts 4-byte aligned; 16-bit loads.
      const GemvRaw<QT, false> t = gemv_load<QT, false>(rp, b_hi - 1, g);
      gemv_unit<QT, NT, false>(acc, t, xs, b_hi - 1, b_lo, g, r16, xslot);
    }
  }

  constexpr int kRedLanes = NT > 4 ? 32 : 16;
  if (lane < kRedLanes) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][lane][e] = acc[e];
  }
  __syncthreads();
  if (threadIdx.x < 16 * NT) {
    const int r = threadIdx.x & 15;
    const int t = threadIdx.x >> 4;
    const int src = r + 16 * (t >> 2);
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[w][src][t & 3];
    const int orow = row0 + r;
    if (t < n_tokens && orow < n_rows) Y[static_cast<int64_t>(t) * n_rows + orow] = s;
  }
}

struct GemvLaunch {
  dim3 grid;
  size_t lds;
  hipStream_t s;
  const uint8_t *w;
  int n_rows, nblk;
  int64_t nb1;
  const void *X;
  int n_tokens, k;
  float *Y;
  int chunk_blocks;
  GemvRoute route;
};

// Allow the kernel more than the default dynamic LDS (once per instantiation).
template <typename K> static hipError_t allow_lds(K kernel) {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize, kXLdsBudget);
  return e;
}

template <int QT, int NT, bool XF16, int WAVES>
static hipError_t gemv_go_w(bool align4, const GemvLaunch &a) {
  hipError_t e = allow_lds(align4 ? gemv_kernel<QT, NT, XF16, true, WAVES> : gemv_kernel<QT, NT, XF16, false, WAVES>);
  if (e != hipSuccess) return e;
  if (align4)
    return launch(gemv_kernel<QT, NT, XF16, true, WAVES>, a.grid, dim3(64 * WAVES), a.lds, a.s, a.w, a.n_rows, a.nblk,
                  a.nb1, a.X, a.n_tokens, a.k, a.Y, a.chunk_blocks, a.route);
  return launch(gemv_kernel<QT, NT, XF16, false, WAVES>, a.grid, dim3(64 * WAVES), a.lds, a.s, a.w, a.n_rows, a.nblk,
                a.nb1, a.X, a.n_tokens, a.k, a.Y, a.chunk_blocks, a.route);
}

template <int QT, int NT, bool XF16>
static hipError_t gemv_go(bool align4, const GemvLaunch &a) {
  const int64_t groups = static_cast<int64_t>(a.grid.x) * (a.route.ids ? a.grid.y : 1);
  return k_split_for(groups, device_cus()) == kKSplitSmall ? gemv_go_w<QT, NT, XF16, kKSplitSmall>(align4, a)
                                                           : gemv_go_w<QT, NT, XF16, kKSplitLarge>(align4, a);
}

template <int QT, bool XF16>
static hipError_t gemv_nt(int nt, bool align4, GemvLaunch a) {
  // chunk_blocks: a multiple of 8, as many blocks as fit the LDS budget for NT slots.
  auto chunk = [&](int NT) {
    int cb = kXLdsBudget / (64 * NT);
    cb -= cb & 7;  // chunks hold whole 8-block groups
    a.chunk_blocks = a.nblk <= cb ? a.nblk : cb;
    a.lds = static_cast<size_t>(a.chunk_blocks) * 64 * NT;
  };
  if (nt <= 1) { chunk(1); return gemv_go<QT, 1, XF16>(align4, a); }
  if (nt <= 2) { chunk(2); return gemv_go<QT, 2, XF16>(align4, a); }
  if (nt <= 4) { chunk(4); return gemv_go<QT, 4, XF16>(align4, a); }
  chunk(8);
  return gemv_go<QT, 8, XF16>(align4, a);
}

hipError_t launch_gemv_id_general(const void *W, int qtype, int64_t n_experts, int64_t n_rows, int64_t k, int64_t nb1,
                                  int64_t nb2, const float *X, int64_t x_slots, const int32_t *ids, int64_t n_ids,
                                  int64_t n_tokens, float *Y, hipStream_t stream) {
  // Q4_K has no general-layout path: the entry points admit only layouts the
  // streaming kernel takes (16-byte-aligned rows)
  if (qtype == QMM_TYPE_Q4_K) return hipErrorInvalidValue;
  const int64_t pairs = n_tokens * n_ids;
  constexpr int64_t kMaxY = 65535;  // grid rows per launch
  const bool align4 = (reinterpret_cast<uintptr_t>(W) % 4 == 0) && (nb1 % 4 == 0) && (nb2 % 4 == 0);
  for (int64_t p0 = 0; p0 < pairs; p0 += kMaxY) {
    GemvLaunch a;
    const unsigned count = static_cast<unsigned>(pairs - p0 < kMaxY ? pairs - p0 : kMaxY);
    a.grid = dim3(static_cast<unsigned>((n_rows + 15) / 16), count);
    a.lds = 0;
    a.s = stream;
    a.w = static_cast<const uint8_t *>(W);
    a.n_rows = static_cast<int>(n_rows);
    a.nblk = static_cast<int>(k / 32);
    a.nb1 = nb1;
    a.X = X;
    a.n_tokens = 1;
    a.k = static_cast<int>(k);
    a.Y = Y;
    a.chunk_blocks = a.nblk;
    a.route = GemvRoute{ids, nb2, static_cast<int>(n_experts), static_cast<int>(n_ids), static_cast<int>(x_slots),
                        static_cast<int>(p0)};
    hipError_t e = by_qtype(qtype, [&](auto qt) { return gemv_nt<decltype(qt)::value, false>(1, align4, a); });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gemv_general(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const void *X,
                               bool x_f16, int64_t n_tokens, float *Y, hipStream_t stream) {
  // Q4_K has no general-layout path: the entry points admit only layouts the
  // streaming kernel takes (16-byte-aligned rows)
  if (qtype == QMM_TYPE_Q4_K) return hipErrorInvalidValue;
  GemvLaunch a;
  a.grid = dim3(static_cast<unsigned>((n_rows + 15) / 16));
  a.lds = 0;
  a.s = stream;
  a.w = static_cast<const uint8_t *>(W);
  a.n_rows = static_cast<int>(n_rows);
  a.nblk = static_cast<int>(k / 32);
  a.nb1 = nb1;
  a.X = X;
  a.n_tokens = static_cast<int>(n_tokens);
  a.k = static_cast<int>(k);
  a.Y = Y;
  a.chunk_blocks = a.nblk;
  a.route = GemvRoute{nullptr, 0, 0, 0, 0, 0};
  const bool align4 = (reinterpret_cast<uintptr_t>(W) % 4 == 0) && (nb1 % 4 == 0);
  const int nt = a.n_tokens;
  return by_qtype(qtype, [&](auto qt) {
    constexpr int QT = decltype(qt)::value;
    return x_f16 ? gemv_nt<QT, true>(nt, align4, a) : gemv_nt<QT, false>(nt, align4, a);
  });
}

}  // namespace qmm
