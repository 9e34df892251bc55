// Block decoder: out[r][i] = fp32(d) * fp32(q - z) (Q4_1, Q5_1: fp32(d) * q
// + m, one rounding; Q4_K: fp32(d sc_j) q - fp32(dmin m_j), one rounding),
// bit-exact, for every row of W or for the rows an index vector selects
// (GET_ROWS).
//
// [Bind] "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section 2.3 (block
// layout); [Arch] "llama.cpp 源码完全拆解(一)：整体架构与模块全景", section
// "权重装载：GGUF、mmap 与 4 bit 块" (w_hat = s (q - z)); GET_ROWS on a quantised
// weight with an I32 index vector: [Load] "llama.cpp 源码完全拆解(三)：GGUF 装载、
// mmap 与张量放置", section "第六步：能力校验" (the op the capability probe
// builds for token-embedding tensors).
//
// A wavefront writes 2 KiB of output (16 blocks) with two 16-byte stores per
// lane that each cover 1 KiB contiguously: lane l of store s writes outputs
// 4 (l % 8) .. +3 of block 16 w + 8 s + l / 8 (w: the wavefront's index in
// the grid-stride loop). HBM-bound: 18 to 34 bytes read and 128 bytes written
// per block. The stores are non-temporal (the output is written once and not
// read back by this kernel): 2048 rows of 32000x4096 Q4_0 take 7.9 instead of
// 9.6 us, and the contiguous 1 KiB stores gain another 15 % over 32-byte
// pieces per lane.
#include "common.h"
#include "launch.h"

namespace qmm {

// Output row r is W's row ids[r] (or r when ids is null); an index outside
// [0, n_rows) gives a row of quiet NaNs and reads nothing.
template <int QT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ W, int64_t n_blocks, int nblk,
                                                      int64_t nb1, const int32_t *__restrict__ ids, int64_t n_rows,
                                                      float *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int e0 = 4 * (lane & 7);  // this lane's first element of its block
  const int64_t n_waves = static_cast<int64_t>(gridDim.x) * (blockDim.x >> 6);
  for (int64_t w = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6; 16 * w < n_blocks;
       w += n_waves) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t blk = 16 * w + 8 * s + (lane >> 3);
      if (blk >= n_blocks) break;
      const int64_t orow = blk / nblk;
      const int b = static_cast<int>(blk - orow * nblk);
      float4_a4 *o = reinterpret_cast<float4_a4 *>(out + blk * 32 + e0);
      const int64_t row = ids ? static_cast<int64_t>(ids[orow]) : orow;
      if (row < 0 || row >= n_rows) {
        const float nan = __builtin_bit_cast(float, 0x7FC00000u);
        __builtin_nontemporal_store(float4_a4{nan, nan, nan, nan}, o);
        continue;
      }
      float v[4];
      if constexpr (QTraits<QT>::kquant) {
        // 32-weight sub-block j of super-block b / 8 (16-byte-aligned rows):
        // elements e0..e0+3 are the low (j even) or high nibbles of code
        // bytes 16 + 32 (j / 2) + e0 .. +3; w = fp32(d sc) q - fp32(dmin m),
        // both products exact, rounded once by the fma
        const int j = b & 7;
        const uint8_t *sb = W + row * nb1 + static_cast<int64_t>(b >> 3) * 144;
        const u32x4_t hdr = *reinterpret_cast<const u32x4_t *>(sb);
        const uint32_t four = ld_u32(sb + 16 + 32 * (j >> 1) + e0) >> (4 * (j & 1));
        uint32_t sc, mn;
        q4k_scale_min(hdr.y, hdr.z, hdr.w, j, sc, mn);
        const float dsc = half_bits_to_float(hdr.x & 0xFFFFu) * static_cast<float>(sc);
        const float dmm = half_bits_to_float(hdr.x >> 16) * static_cast<float>(mn);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_fmaf(static_cast<float>((four >> (8 * i)) & 0xF), dsc, -dmm);
        __builtin_nontemporal_store(float4_a4{v[0], v[1], v[2], v[3]}, o);
        continue;
      }
      const uint8_t *p = W + row * nb1 + static_cast<int64_t>(b) * Block<QT>::bytes;
      const float d = half_bits_to_float(ld_u16(p));
      if constexpr (QTraits<QT>::nibbles) {
        // elements e0..e0+3: the low (e0 < 16) or high nibbles of code bytes
        // e0 % 16 .. +3, with their fifth bits (5-bit types) from bits e0..e0+3
        constexpr int Z = QTraits<QT>::zero;
        const uint8_t *q = p + QTraits<QT>::codes + (e0 & 15);
        const uint32_t four = ld_u16(q) | (ld_u16(q + 2) << 16);
        const int shift = e0 >= 16 ? 4 : 0;
        uint32_t h4 = 0;
        if constexpr (QTraits<QT>::has_qh) {
          const uint8_t *qh = p + QTraits<QT>::qh;
          h4 = ((ld_u16(qh) | (ld_u16(qh + 2) << 16)) >> e0) & 0xFu;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = static_cast<int>(((four >> (8 * j + shift)) & 0xF) | (((h4 >> j) & 1) << 4));
          v[j] = d * static_cast<float>(c - Z);
        }
        if constexpr (QTraits<QT>::has_min) {
          // d * q is exact, so adding m rounds once, as one fma would
          const float m = half_bits_to_float(ld_u16(p + 2));
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = __fadd_rn(v[j], m);
        }
      } else {
        const uint8_t *q = p + 2 + e0;
        const uint32_t four = ld_u16(q) | (ld_u16(q + 2) << 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = d * static_cast<float>(static_cast<int8_t>((four >> (8 * j)) & 0xFF));
      }
      __builtin_nontemporal_store(float4_a4{v[0], v[1], v[2], v[3]}, o);
    }
  }
}

static hipError_t decode_rows(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const int32_t *ids,
                              int64_t n_out, float *out, hipStream_t stream) {
  const int nblk = static_cast<int>(k / 32);
  const int64_t blocks = n_out * nblk;
  const int64_t want = (blocks + 63) / 64;  // 4 wavefronts of 16 blocks per workgroup
  const unsigned grid = static_cast<unsigned>(want < 65536 ? want : 65536);
  const uint8_t *w = static_cast<const uint8_t *>(W);
  return by_qtype_k(qtype, [&](auto qt) {
    return launch(dequant_kernel<decltype(qt)::value>, dim3(grid), dim3(256), 0, stream, w, blocks, nblk, nb1, ids,
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
