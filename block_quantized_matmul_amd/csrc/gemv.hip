// Decode MUL_MAT (1 <= n_tokens <= 8): y[t][r] = sum_b d_rb * sum_i (q - z) x[t][32 b + i].
//
// What is computed: [Bind] "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section
// 2.3 (blocks are dequantised inside MUL_MAT, then multiplied) and [Arch]
// "llama.cpp 源码完全拆解(一)：整体架构与模块全景", section "权重装载：GGUF、mmap
// 与 4 bit 块" (w = s (q - z); the GPU kernels decode scale and integer weights
// per block and multiply-add them with activations in registers).
//
// Design (MI355X, gfx950). The kernel is bound by HBM: every weight byte is
// read exactly once, with dword-aligned vector loads that together cover each
// row contiguously. One workgroup owns 16 rows; its 8 wavefronts split the
// row's blocks into contiguous ranges and meet in LDS at the end, in a fixed
// order (no atomics, so results are bitwise reproducible).
//
// The dot products run on the matrix cores: one v_mfma_f32_16x16x32_f16 per
// block covers 16 rows x 32 weights x 16 token slots. The B operand holds the
// integer codes (q - z), which are exact in fp16; the A operand holds the
// activations rounded to fp16; each lane then applies its row's block scale d
// in fp32 (acc += d * partial), so the weights enter the sum exactly. Lane l
// of the B operand serves row l % 16 and the 8 elements of block-slice
// l / 16; the A operand uses the same element order, so each MFMA is exactly
// that block's partial dot product. D holds token 4 (l / 16) + e, row l % 16
// in element e of lane l.
//
// Memory access for the common case (row starts 4-byte aligned): a unit is a
// pair of blocks (36 bytes Q4_0, 68 bytes Q8_0). The four lanes of a row load
// overlapping dword windows that together cover the pair once; the two
// scales are forwarded from the lanes that loaded them with ds_bpermute. Rows
// whose start is only 2-byte aligned (odd block count with dense rows, or a
// 2-byte-aligned W) take 16-bit loads, one block per unit.
#include "common.h"
#include "launch.h"

namespace qmm {

constexpr int kGemvWaves = 8;
constexpr int kGemvThreads = 64 * kGemvWaves;
constexpr int kPrefetch = 2;  // units in flight ahead of the one being computed

template <int QT, bool ALIGN4> struct GemvRaw;
// Q4_0 pair: dwords g, g + 1 (even block, codes start 2 bytes in) and 5 + g (odd block).
template <> struct GemvRaw<QMM_TYPE_Q4_0, true> { u32x2_t a; uint32_t b; };
// Q8_0 pair: dwords 2g .. 2g + 2 (even block) and 9 + 2g .. 10 + 2g (odd block).
template <> struct GemvRaw<QMM_TYPE_Q8_0, true> { uint32_t a0, a1, a2; u32x2_t b; };
// Single block, 16-bit loads: scale bits and the lane's code dwords.
template <> struct GemvRaw<QMM_TYPE_Q4_0, false> { uint32_t d, q; };
template <> struct GemvRaw<QMM_TYPE_Q8_0, false> { uint32_t d, q0, q1; };

template <int QT, bool ALIGN4>
__device__ __forceinline__ GemvRaw<QT, ALIGN4> gemv_load(const uint8_t *rp, int u, int g) {
  GemvRaw<QT, ALIGN4> r;
  if constexpr (ALIGN4) {
    const uint8_t *p = rp + static_cast<int64_t>(u) * (2 * Block<QT>::bytes);
    if constexpr (QT == QMM_TYPE_Q4_0) {
      r.a = ld_u32x2(p + 4 * g);
      r.b = ld_u32(p + 20 + 4 * g);
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
    } else {
      r.q0 = ld_u16(p + 2 + 8 * g) | (ld_u16(p + 4 + 8 * g) << 16);
      r.q1 = ld_u16(p + 6 + 8 * g) | (ld_u16(p + 8 + 8 * g) << 16);
    }
  }
  return r;
}

// A-operand (activations) for block `blk`, in the element order of the
// B-operand built by gemv_codes(). Token rows beyond n_tokens were clamped to
// a valid row by the caller; their D entries are never stored.
template <int QT, bool XF16>
__device__ __forceinline__ half8_t gemv_x(const void *xrow, int blk, int g) {
  if constexpr (QT == QMM_TYPE_Q4_0) {
    const int o = 32 * blk + 4 * g;  // elements o..o+3 and o+16..o+19
    if constexpr (XF16) {
      const half4_t a = *reinterpret_cast<const half4_t *>(static_cast<const _Float16 *>(xrow) + o);
      const half4_t b = *reinterpret_cast<const half4_t *>(static_cast<const _Float16 *>(xrow) + o + 16);
      return half8_t{a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    } else {
      const float4_t a = *reinterpret_cast<const float4_t *>(static_cast<const float *>(xrow) + o);
      const float4_t b = *reinterpret_cast<const float4_t *>(static_cast<const float *>(xrow) + o + 16);
      return make_half8(cvt_half2(a.x, a.y), cvt_half2(a.z, a.w), cvt_half2(b.x, b.y), cvt_half2(b.z, b.w));
    }
  } else {
    const int o = 32 * blk + 8 * g;  // elements o..o+7
    if constexpr (XF16) {
      return *reinterpret_cast<const half8_t *>(static_cast<const _Float16 *>(xrow) + o);
    } else {
      const float4_t a = *reinterpret_cast<const float4_t *>(static_cast<const float *>(xrow) + o);
      const float4_t b = *reinterpret_cast<const float4_t *>(static_cast<const float *>(xrow) + o + 4);
      return make_half8(cvt_half2(a.x, a.y), cvt_half2(a.z, a.w), cvt_half2(b.x, b.y), cvt_half2(b.z, b.w));
    }
  }
}

// B-operand: this lane's 8 exact codes (q - z) of one block.
template <int QT> __device__ __forceinline__ half8_t gemv_codes(uint32_t q0, uint32_t q1);
template <> __device__ __forceinline__ half8_t gemv_codes<QMM_TYPE_Q4_0>(uint32_t q0, uint32_t) {
  half2_t h[4];
  q4_unpack(q0, h);
  return make_half8(h[0], h[1], h[2], h[3]);
}
template <> __device__ __forceinline__ half8_t gemv_codes<QMM_TYPE_Q8_0>(uint32_t q0, uint32_t q1) {
  half2_t lo[2], hi[2];
  q8_unpack(q0, lo);
  q8_unpack(q1, hi);
  return make_half8(lo[0], lo[1], hi[0], hi[1]);
}

template <int NT>
__device__ __forceinline__ void gemv_block(float acc[4], half8_t xop, half8_t wop, uint32_t d_bits) {
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};
  const float4_t part = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, wop, zero, 0, 0, 0);
  const float d = half_bits_to_float(d_bits);
  constexpr int E = NT < 4 ? NT : 4;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(d, part[e], acc[e]);
}

template <int QT, int NT, bool XF16, bool ALIGN4>
__device__ __forceinline__ void gemv_unit(float acc[4], const GemvRaw<QT, ALIGN4> &r, const void *xrow, int u, int g,
                                          int r16) {
  if constexpr (ALIGN4) {
    if constexpr (QT == QMM_TYPE_Q4_0) {
      // Even block: scale = low half of dword 0 (lane g = 0's a.x); odd block:
      // scale = high half of dword 4 (lane g = 3's a.y).
      const uint32_t de = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * r16, static_cast<int>(r.a.x)));
      const uint32_t dd = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * (r16 + 48), static_cast<int>(r.a.y)));
      gemv_block<NT>(acc, gemv_x<QT, XF16>(xrow, 2 * u, g), gemv_codes<QT>(shift16(r.a.x, r.a.y), 0), de & 0xFFFFu);
      gemv_block<NT>(acc, gemv_x<QT, XF16>(xrow, 2 * u + 1, g), gemv_codes<QT>(r.b, 0), dd >> 16);
    } else {
      // Even block: scale = low half of dword 0 (lane g = 0's a0); odd block
      // starts at byte 34: scale = high half of dword 8 (lane g = 3's a2).
      const uint32_t de = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * r16, static_cast<int>(r.a0)));
      const uint32_t dd = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(4 * (r16 + 48), static_cast<int>(r.a2)));
      gemv_block<NT>(acc, gemv_x<QT, XF16>(xrow, 2 * u, g),
                     gemv_codes<QT>(shift16(r.a0, r.a1), shift16(r.a1, r.a2)), de & 0xFFFFu);
      gemv_block<NT>(acc, gemv_x<QT, XF16>(xrow, 2 * u + 1, g), gemv_codes<QT>(r.b.x, r.b.y), dd >> 16);
    }
  } else {
    if constexpr (QT == QMM_TYPE_Q4_0)
      gemv_block<NT>(acc, gemv_x<QT, XF16>(xrow, u, g), gemv_codes<QT>(r.q, 0), r.d);
    else
      gemv_block<NT>(acc, gemv_x<QT, XF16>(xrow, u, g), gemv_codes<QT>(r.q0, r.q1), r.d);
  }
}

template <int QT, int NT, bool XF16, bool ALIGN4>
__global__ __launch_bounds__(kGemvThreads) void gemv_kernel(const uint8_t *__restrict__ W, int n_rows, int nblk,
                                                            int64_t nb1, const void *__restrict__ X, int n_tokens,
                                                            int k, float *__restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  // Rows past the end and token slots past n_tokens read valid memory (the
  // last row / token) and their results are dropped at the store.
  const int row = min(row0 + r16, n_rows - 1);
  const uint8_t *rp = W + static_cast<int64_t>(row) * nb1;
  const int tok = min(r16, n_tokens - 1);
  const void *xrow = XF16 ? static_cast<const void *>(static_cast<const _Float16 *>(X) + static_cast<int64_t>(tok) * k)
                          : static_cast<const void *>(static_cast<const float *>(X) + static_cast<int64_t>(tok) * k);

  const int n_units = ALIGN4 ? (nblk >> 1) : nblk;
  const int u0 = static_cast<int>((static_cast<int64_t>(wave) * n_units) / kGemvWaves);
  const int u1 = static_cast<int>((static_cast<int64_t>(wave + 1) * n_units) / kGemvWaves);

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (u0 < u1) {
    // Software pipeline: kPrefetch units of weights are in flight while one
    // is computed. Prefetch indices are clamped to the wave's last unit so
    // every load is unconditional and in bounds.
    GemvRaw<QT, ALIGN4> ring[kPrefetch];
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) ring[i] = gemv_load<QT, ALIGN4>(rp, min(u0 + i, u1 - 1), g);
    for (int u = u0; u < u1; ++u) {
      const GemvRaw<QT, ALIGN4> cur = ring[0];
#pragma unroll
      for (int i = 0; i + 1 < kPrefetch; ++i) ring[i] = ring[i + 1];
      ring[kPrefetch - 1] = gemv_load<QT, ALIGN4>(rp, min(u + kPrefetch, u1 - 1), g);
      gemv_unit<QT, NT, XF16, ALIGN4>(acc, cur, xrow, u, g, r16);
    }
  }
  if (ALIGN4 && (nblk & 1) && wave == kGemvWaves - 1) {
    // Odd block count: the last block starts 4-byte aligned; 16-bit loads.
    const GemvRaw<QT, false> t = gemv_load<QT, false>(rp, nblk - 1, g);
    gemv_unit<QT, NT, XF16, false>(acc, t, xrow, nblk - 1, g, r16);
  }

  constexpr int kRedLanes = NT > 4 ? 32 : 16;
  __shared__ float red[kGemvWaves][kRedLanes][4];
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
    for (int w = 0; w < kGemvWaves; ++w) s += red[w][src][t & 3];
    const int orow = row0 + r;
    if (t < n_tokens && orow < n_rows) Y[static_cast<int64_t>(t) * n_rows + orow] = s;
  }
}

template <int QT, int NT, bool XF16>
static hipError_t gemv_dispatch_align(bool align4, dim3 grid, hipStream_t s, const uint8_t *w, int n_rows, int nblk,
                                      int64_t nb1, const void *X, int n_tokens, int k, float *Y) {
  if (align4)
    return launch(gemv_kernel<QT, NT, XF16, true>, grid, dim3(kGemvThreads), 0, s, w, n_rows, nblk, nb1, X, n_tokens, k, Y);
  return launch(gemv_kernel<QT, NT, XF16, false>, grid, dim3(kGemvThreads), 0, s, w, n_rows, nblk, nb1, X, n_tokens, k, Y);
}

template <int QT, bool XF16>
static hipError_t gemv_dispatch_nt(int nt, bool align4, dim3 grid, hipStream_t s, const uint8_t *w, int n_rows,
                                   int nblk, int64_t nb1, const void *X, int n_tokens, int k, float *Y) {
  if (nt <= 1) return gemv_dispatch_align<QT, 1, XF16>(align4, grid, s, w, n_rows, nblk, nb1, X, n_tokens, k, Y);
  if (nt <= 2) return gemv_dispatch_align<QT, 2, XF16>(align4, grid, s, w, n_rows, nblk, nb1, X, n_tokens, k, Y);
  if (nt <= 4) return gemv_dispatch_align<QT, 4, XF16>(align4, grid, s, w, n_rows, nblk, nb1, X, n_tokens, k, Y);
  return gemv_dispatch_align<QT, 8, XF16>(align4, grid, s, w, n_rows, nblk, nb1, X, n_tokens, k, Y);
}

hipError_t launch_gemv(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const void *X, bool x_f16,
                       int64_t n_tokens, float *Y, hipStream_t stream) {
  const uint8_t *w = static_cast<const uint8_t *>(W);
  const bool align4 = (reinterpret_cast<uintptr_t>(W) % 4 == 0) && (nb1 % 4 == 0);
  const dim3 grid(static_cast<unsigned>((n_rows + 15) / 16));
  const int nblk = static_cast<int>(k / 32), nr = static_cast<int>(n_rows), nt = static_cast<int>(n_tokens),
            kk = static_cast<int>(k);
  if (qtype == QMM_TYPE_Q4_0) {
    if (x_f16) return gemv_dispatch_nt<QMM_TYPE_Q4_0, true>(nt, align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y);
    return gemv_dispatch_nt<QMM_TYPE_Q4_0, false>(nt, align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y);
  }
  if (x_f16) return gemv_dispatch_nt<QMM_TYPE_Q8_0, true>(nt, align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y);
  return gemv_dispatch_nt<QMM_TYPE_Q8_0, false>(nt, align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y);
}

}  // namespace qmm
