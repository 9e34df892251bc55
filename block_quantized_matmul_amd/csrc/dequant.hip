// Block decoder: out[r][i] = fp32(d) * fp32(q - z) (Q4_1, Q5_1: fp32(d) * q
// + m, one rounding), bit-exact, for every row of W or for the rows an index
// vector selects (GET_ROWS).
//
// [Bind] "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section 2.3 (block
// layout); [Arch] "llama.cpp 源码完全拆解(一)：整体架构与模块全景", section
// "权重装载：GGUF、mmap 与 4 bit 块" (w_hat = s (q - z)); GET_ROWS on a quantised
// weight with an I32 index vector: [Load] "llama.cpp 源码完全拆解(三)：GGUF 装载、
// mmap 与张量放置", section "第六步：能力校验" (the op the capability probe
// builds for token-embedding tensors).
//
// One thread writes eight consecutive outputs (one quarter of a block), so a
// wavefront stores 2 KiB of contiguous fp32 with 16-byte stores. HBM-bound:
// 18 to 34 bytes read and 128 bytes written per block.
#include "common.h"
#include "launch.h"

namespace qmm {

// Output row r is W's row ids[r] (or r when ids is null); an index outside
// [0, n_rows) gives a row of quiet NaNs and reads nothing.
template <int QT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ W, int64_t n_quarters, int nblk,
                                                      int64_t nb1, const int32_t *__restrict__ ids, int64_t n_rows,
                                                      float *__restrict__ out) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < n_quarters; t += stride) {
    const int part = static_cast<int>(t & 3);  // elements [8 part, 8 part + 8)
    const int64_t blk = t >> 2;
    const int64_t orow = blk / nblk;
    const int b = static_cast<int>(blk - orow * nblk);
    float4_a4 *o = reinterpret_cast<float4_a4 *>(out + blk * 32 + 8 * part);
    const int64_t row = ids ? static_cast<int64_t>(ids[orow]) : orow;
    if (row < 0 || row >= n_rows) {
      const float nan = __builtin_bit_cast(float, 0x7FC00000u);
      o[0] = float4_t{nan, nan, nan, nan};
      o[1] = float4_t{nan, nan, nan, nan};
      continue;
    }
    const uint8_t *p = W + row * nb1 + static_cast<int64_t>(b) * Block<QT>::bytes;
    const float d = half_bits_to_float(ld_u16(p));
    float v[8];
    if constexpr (QTraits<QT>::nibbles) {
      // part 0/1: low nibbles of qs[0..7] / qs[8..15]; part 2/3: high nibbles.
      constexpr int Z = QTraits<QT>::zero;
      const uint8_t *q = p + QTraits<QT>::codes + 8 * (part & 1);
      const int shift = (part & 2) ? 4 : 0;
      // fifth bits of this part's elements 8 part .. 8 part + 7 (5-bit types)
      uint32_t h5 = 0;
      if constexpr (QTraits<QT>::has_qh) {
        const uint8_t *qh = p + QTraits<QT>::qh;
        h5 = ((ld_u16(qh) | (ld_u16(qh + 2) << 16)) >> (8 * part)) & 0xFFu;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t two = ld_u16(q + 2 * j);
        const int c0 = static_cast<int>(((two >> shift) & 0xF) | (((h5 >> (2 * j)) & 1) << 4));
        const int c1 = static_cast<int>(((two >> (8 + shift)) & 0xF) | (((h5 >> (2 * j + 1)) & 1) << 4));
        v[2 * j] = d * static_cast<float>(c0 - Z);
        v[2 * j + 1] = d * static_cast<float>(c1 - Z);
      }
      if constexpr (QTraits<QT>::has_min) {
        // d * q is exact, so adding m rounds once, as one fma would
        const float m = half_bits_to_float(ld_u16(p + 2));
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = __fadd_rn(v[j], m);
      }
    } else {
      const uint8_t *q = p + 2 + 8 * part;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t two = ld_u16(q + 2 * j);
        v[2 * j] = d * static_cast<float>(static_cast<int8_t>(two & 0xFF));
        v[2 * j + 1] = d * static_cast<float>(static_cast<int8_t>(two >> 8));
      }
    }
    o[0] = float4_t{v[0], v[1], v[2], v[3]};
    o[1] = float4_t{v[4], v[5], v[6], v[7]};
  }
}

static hipError_t decode_rows(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const int32_t *ids,
                              int64_t n_out, float *out, hipStream_t stream) {
  const int nblk = static_cast<int>(k / 32);
  const int64_t quarters = n_out * nblk * 4;
  const int64_t want = (quarters + 255) / 256;
  const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
  const uint8_t *w = static_cast<const uint8_t *>(W);
  return by_qtype(qtype, [&](auto qt) {
    return launch(dequant_kernel<decltype(qt)::value>, dim3(grid), dim3(256), 0, stream, w, quarters, nblk, nb1, ids,
                  n_rows, out);
  });
}

hipError_t launch_dequant(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, float *out,
                          hipStream_t stream) {
  return decode_rows(W, qtype, n_rows, k, nb1, nullptr, n_rows, out, stream);
}

hipError_t launch_get_rows(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const int32_t *ids,
                           int64_t n_ids, float *out, hipStream_t stream) {
  return decode_rows(W, qtype, n_rows, k, nb1, ids, n_ids, out, stream);
}

}  // namespace qmm
