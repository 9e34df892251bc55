// Prefill MUL_MAT (any n_tokens, used above 8): Y = X * dequant(W)^T on the
// matrix cores.
//
// What is computed: [Bind] "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section
// 2.3 (MUL_MAT reads the blocks and dequantises them to fp16/fp32 on the spot,
// then multiplies) with the reconstruction w = d (q - z) of [Arch]
// "llama.cpp 源码完全拆解(一)：整体架构与模块全景", section "权重装载：GGUF、mmap
// 与 4 bit 块". The 512-token shape of the prefill workload is the batch the
// capability probe of [Load] "llama.cpp 源码完全拆解(三)：GGUF 装载、mmap 与张量
// 放置", section "第六步：能力校验" uses to reach a backend's batched kernel.
//
// Design (MI355X, gfx950). The path is a dense contraction, so it runs on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation. A 256-thread workgroup owns
// a 128-row x 128-token output tile and walks k in stages of 128 (four
// blocks). Each stage: the quantised blocks of 128 rows (9 KiB for Q4_0) and
// the activation tile are fetched into registers while the previous stage is
// on the matrix cores; then the blocks are decoded to fp16 d * (q - z) (exact
// integer code, one fp16 rounding of the product) and written with the fp16
// activations into padded LDS tiles; four wavefronts each run a 64 x 64
// sub-tile as 4 x 4 MFMA tiles. Weights never exist in dequantised form
// outside LDS.
#include "common.h"
#include "launch.h"

namespace qmm {

constexpr int kBM = 128;  // weight rows per tile
constexpr int kBN = 128;  // tokens per tile
constexpr int kBK = 128;  // k per stage (4 blocks)
constexpr int kLdsStride = kBK + 8;  // halves; 16-byte pad breaks LDS bank conflicts
constexpr int kGemmThreads = 256;

// Decoded pair of blocks (the codes of block j as dwords, its scale bits).
template <int QT> struct PairCodes;
template <> struct PairCodes<QMM_TYPE_Q4_0> { uint32_t d[2]; uint32_t q[2][4]; };
template <> struct PairCodes<QMM_TYPE_Q8_0> { uint32_t d[2]; uint32_t q[2][8]; };

template <int QT>
__device__ __forceinline__ void load_block_u16(const uint8_t *p, uint32_t &d, uint32_t *q) {
  constexpr int nq = QT == QMM_TYPE_Q4_0 ? 4 : 8;
  d = ld_u16(p);
#pragma unroll
  for (int i = 0; i < nq; ++i) q[i] = ld_u16(p + 2 + 4 * i) | (ld_u16(p + 4 + 4 * i) << 16);
}

// Blocks blk0 and blk0 + 1 of the row at rp; blocks at or past nblk read as
// zero codes with zero scale.
template <int QT, bool ALIGN4>
__device__ __forceinline__ PairCodes<QT> load_pair(const uint8_t *rp, int blk0, int nblk) {
  constexpr int BB = Block<QT>::bytes;
  constexpr int nq = QT == QMM_TYPE_Q4_0 ? 4 : 8;
  PairCodes<QT> c;
  const uint8_t *p = rp + static_cast<int64_t>(blk0) * BB;
  if (ALIGN4 && blk0 + 1 < nblk) {
    // 2 * BB bytes from a 4-byte-aligned address: block 0 = dwords 0.., its
    // codes start 2 bytes in; block 1 starts at byte BB (2 mod 4), its codes
    // at BB + 2 (aligned).
    constexpr int ndw = 2 * BB / 4;  // 9 (Q4_0) or 17 (Q8_0)
    uint32_t w[ndw];
#pragma unroll
    for (int i = 0; i + 4 <= ndw; i += 4) {
      const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(p + 4 * i);
      w[i] = v.x; w[i + 1] = v.y; w[i + 2] = v.z; w[i + 3] = v.w;
    }
    w[ndw - 1] = ld_u32(p + 4 * (ndw - 1));
    c.d[0] = w[0] & 0xFFFFu;
#pragma unroll
    for (int i = 0; i < nq; ++i) c.q[0][i] = shift16(w[i], w[i + 1]);
    c.d[1] = w[nq] >> 16;
#pragma unroll
    for (int i = 0; i < nq; ++i) c.q[1][i] = w[nq + 1 + i];
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (blk0 + j < nblk) {
        load_block_u16<QT>(p + j * BB, c.d[j], c.q[j]);
      } else {
        c.d[j] = 0;
#pragma unroll
        for (int i = 0; i < nq; ++i) c.q[j][i] = 0;
      }
    }
  }
  return c;
}

// Decode one block to 32 fp16 weights fl16(d * (q - z)) in element order and
// store them at dst (16-byte aligned LDS).
template <int QT>
__device__ __forceinline__ void store_block_f16(_Float16 *dst, uint32_t d_bits, const uint32_t *q) {
  const _Float16 dh = __builtin_bit_cast(_Float16, static_cast<uint16_t>(d_bits));
  const half2_t d2 = {dh, dh};
  half2_t h[16];
  if constexpr (QT == QMM_TYPE_Q4_0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t u[4];
      q4_unpack(q[i], u);
      h[2 * i] = u[0] * d2;      // elements 4i, 4i+1
      h[2 * i + 1] = u[1] * d2;  // 4i+2, 4i+3
      h[8 + 2 * i] = u[2] * d2;  // 16+4i, 17+4i
      h[9 + 2 * i] = u[3] * d2;  // 18+4i, 19+4i
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      half2_t u[2];
      q8_unpack(q[i], u);
      h[2 * i] = u[0] * d2;
      h[2 * i + 1] = u[1] * d2;
    }
  }
  u32x4_t *o = reinterpret_cast<u32x4_t *>(dst);
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = u32x4_t{as_u32(h[4 * i]), as_u32(h[4 * i + 1]), as_u32(h[4 * i + 2]), as_u32(h[4 * i + 3])};
}

// Activation slice of one thread: 64 consecutive k values of one token.
template <bool XF16> struct XRaw;
template <> struct XRaw<true> { u32x4_t v[8]; };
template <> struct XRaw<false> { float4_t v[16]; };

template <bool XF16>
__device__ __forceinline__ XRaw<XF16> load_x(const void *X, int tok, bool tok_ok, int k, int k0) {
  XRaw<XF16> r;
  constexpr int per32 = XF16 ? 4 : 8;  // vectors per 32 elements
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const bool ok = tok_ok && (k0 + 32 * c < k);
#pragma unroll
    for (int i = 0; i < per32; ++i) {
      if constexpr (XF16) {
        const u32x4_t *p = reinterpret_cast<const u32x4_t *>(static_cast<const _Float16 *>(X) +
                                                             static_cast<int64_t>(tok) * k + k0 + 32 * c) + i;
        r.v[c * per32 + i] = ok ? *p : u32x4_t{0u, 0u, 0u, 0u};
      } else {
        const float4_t *p = reinterpret_cast<const float4_t *>(static_cast<const float *>(X) +
                                                               static_cast<int64_t>(tok) * k + k0 + 32 * c) + i;
        r.v[c * per32 + i] = ok ? *p : float4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  return r;
}

template <bool XF16>
__device__ __forceinline__ void store_x(_Float16 *dst, const XRaw<XF16> &r) {
  u32x4_t *o = reinterpret_cast<u32x4_t *>(dst);
  if constexpr (XF16) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = r.v[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4_t a = r.v[2 * i], b = r.v[2 * i + 1];
      o[i] = u32x4_t{as_u32(cvt_half2(a.x, a.y)), as_u32(cvt_half2(a.z, a.w)), as_u32(cvt_half2(b.x, b.y)),
                     as_u32(cvt_half2(b.z, b.w))};
    }
  }
}

template <int QT, bool XF16, bool ALIGN4>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(const uint8_t *__restrict__ W, int n_rows, int nblk,
                                                            int64_t nb1, const void *__restrict__ X, int n_tokens,
                                                            int k, float *__restrict__ Y, bool y_vec4, int row_tiles) {
  __shared__ __attribute__((aligned(16))) _Float16 Ws[kBM * kLdsStride];
  __shared__ __attribute__((aligned(16))) _Float16 Xs[kBN * kLdsStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  // 1-D grid: consecutive workgroups walk the row tiles of one token tile.
  const int row0 = static_cast<int>(blockIdx.x % row_tiles) * kBM;
  const int tok0 = static_cast<int>(blockIdx.x / row_tiles) * kBN;

  // Staging roles: thread -> (row, pair of blocks) and (token, 64-wide half of the stage).
  const int srow = tid >> 1, spair = tid & 1;
  const uint8_t *rp = W + static_cast<int64_t>(min(row0 + srow, n_rows - 1)) * nb1;
  const int stok = tid >> 1, shalf = tid & 1;
  const bool stok_ok = tok0 + stok < n_tokens;
  const int stok_c = min(tok0 + stok, n_tokens - 1);

  float4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int n_stages = (nblk + 3) / 4;
  PairCodes<QT> wraw = load_pair<QT, ALIGN4>(rp, 2 * spair, nblk);
  XRaw<XF16> xraw = load_x<XF16>(X, stok_c, stok_ok, k, 64 * shalf);

  for (int s = 0; s < n_stages; ++s) {
    __syncthreads();  // everyone is done reading the previous stage
    store_block_f16<QT>(Ws + srow * kLdsStride + 64 * spair, wraw.d[0], wraw.q[0]);
    store_block_f16<QT>(Ws + srow * kLdsStride + 64 * spair + 32, wraw.d[1], wraw.q[1]);
    store_x<XF16>(Xs + stok * kLdsStride + 64 * shalf, xraw);
    __syncthreads();
    if (s + 1 < n_stages) {
      wraw = load_pair<QT, ALIGN4>(rp, 4 * (s + 1) + 2 * spair, nblk);
      xraw = load_x<XF16>(X, stok_c, stok_ok, k, kBK * (s + 1) + 64 * shalf);
    }
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      half8_t a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const half8_t *>(Ws + (64 * wm + 16 * i + (lane & 15)) * kLdsStride + kk + 8 * (lane >> 4));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const half8_t *>(Xs + (64 * wn + 16 * j + (lane & 15)) * kLdsStride + kk + 8 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // D element e of lane l in tile (i, j): row 64 wm + 16 i + 4 (l / 16) + e,
  // token 64 wn + 16 j + l % 16.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = tok0 + 64 * wn + 16 * j + (lane & 15);
    if (tok >= n_tokens) continue;
    float *yrow = Y + static_cast<int64_t>(tok) * n_rows;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + 64 * wm + 16 * i + 4 * (lane >> 4);
      if (y_vec4 && r + 3 < n_rows) {
        *reinterpret_cast<float4_t *>(yrow + r) = acc[i][j];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (r + e < n_rows) yrow[r + e] = acc[i][j][e];
      }
    }
  }
}

template <int QT, bool XF16>
static hipError_t gemm_dispatch(bool align4, dim3 grid, hipStream_t s, const uint8_t *w, int n_rows, int nblk,
                                int64_t nb1, const void *X, int n_tokens, int k, float *Y, bool y_vec4, int row_tiles) {
  if (align4)
    return launch(gemm_kernel<QT, XF16, true>, grid, dim3(kGemmThreads), 0, s, w, n_rows, nblk, nb1, X, n_tokens, k, Y,
                  y_vec4, row_tiles);
  return launch(gemm_kernel<QT, XF16, false>, grid, dim3(kGemmThreads), 0, s, w, n_rows, nblk, nb1, X, n_tokens, k, Y,
                y_vec4, row_tiles);
}

hipError_t launch_gemm(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const void *X, bool x_f16,
                       int64_t n_tokens, float *Y, hipStream_t stream) {
  const uint8_t *w = static_cast<const uint8_t *>(W);
  const bool align4 = (reinterpret_cast<uintptr_t>(W) % 4 == 0) && (nb1 % 4 == 0);
  const bool y_vec4 = (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && (n_rows % 4 == 0);
  const int64_t row_tiles = (n_rows + kBM - 1) / kBM, tok_tiles = (n_tokens + kBN - 1) / kBN;
  if (row_tiles * tok_tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(row_tiles * tok_tiles));
  const int rt = static_cast<int>(row_tiles);
  const int nblk = static_cast<int>(k / 32), nr = static_cast<int>(n_rows), nt = static_cast<int>(n_tokens),
            kk = static_cast<int>(k);
  if (qtype == QMM_TYPE_Q4_0) {
    if (x_f16) return gemm_dispatch<QMM_TYPE_Q4_0, true>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
    return gemm_dispatch<QMM_TYPE_Q4_0, false>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
  }
  if (x_f16) return gemm_dispatch<QMM_TYPE_Q8_0, true>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
  return gemm_dispatch<QMM_TYPE_Q8_0, false>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
}

}  // namespace qmm
