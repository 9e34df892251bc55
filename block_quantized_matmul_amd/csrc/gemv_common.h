// Helpers shared by the decode kernels (gemv.hip, gemv_stream.hip): the
// B operand of exact integer codes, the A operand of staged activations, and
// one block's MFMA with its fp32 scale.
#pragma once

#include "common.h"

namespace qmm {

// Both decode kernels give a 16-row group to one workgroup whose wavefronts
// split k into contiguous ranges of 8-block groups and add their partial sums
// in wavefront order. A launch with no more row groups than the GPU has CUs
// (one workgroup per CU) uses 16 wavefronts, halving each one's share and so
// the compute left after its data arrives; larger launches use 8, which lets
// two workgroups share a CU and overlap. Both kernels take the same split for
// the same launch size, so their results are bitwise identical wherever both
// apply.
constexpr int kKSplitSmall = 16;
constexpr int kKSplitLarge = 8;
__host__ inline int k_split_for(int64_t row_groups, int cus) {
  return cus > 0 && row_groups <= cus ? kKSplitSmall : kKSplitLarge;
}

// B-operand: this lane's 8 exact codes (q - z) of one block.
template <int QT> __device__ __forceinline__ half8_t gemv_codes(uint32_t q0, uint32_t q1);
template <> __device__ __forceinline__ half8_t gemv_codes<QMM_TYPE_Q4_0>(uint32_t q0, uint32_t) {
  half2_t h[4];
  q4_unpack<8>(q0, h);
  return make_half8(h[0], h[1], h[2], h[3]);
}
template <> __device__ __forceinline__ half8_t gemv_codes<QMM_TYPE_Q4_1>(uint32_t q0, uint32_t) {
  half2_t h[4];
  q4_unpack<0>(q0, h);
  return make_half8(h[0], h[1], h[2], h[3]);
}
// B-operand of a 5-bit type: the lane's code bytes qs[j0..j0+3] (elements
// j0..j0+3 and j0+16..j0+19) with their fifth bits from qh.
template <int QT> __device__ __forceinline__ half8_t gemv_codes5(uint32_t qs, uint32_t qh, int j0) {
  half2_t h[4];
  q5_unpack<QTraits<QT>::zero>(qs, qh, j0, h);
  return make_half8(h[0], h[1], h[2], h[3]);
}
template <> __device__ __forceinline__ half8_t gemv_codes<QMM_TYPE_Q8_0>(uint32_t q0, uint32_t q1) {
  half2_t lo[2], hi[2];
  q8_unpack(q0, lo);
  q8_unpack(q1, hi);
  return make_half8(lo[0], lo[1], hi[0], hi[1]);
}

// Staged activations: for chunk-relative block bb, lane group g and token t,
// the 8 fp16 values of the A operand live at xs[(4 bb + g) * NT + t], in the
// element order the B operand uses:
//   Q4_0, Q4_1, Q5_0, Q5_1: elements 4g..4g+3 then 16+4g..16+4g+3;
//   Q8_0: elements 8g..8g+7.
template <int QT, int NT, bool XF16, int THREADS>
__device__ __forceinline__ void gemv_stage_x(half8_t *xs, const void *X, int n_tokens, int k, int b_lo, int b_hi) {
  const int nb = b_hi - b_lo;
  const int n4 = n_tokens * nb * 8;  // 4-element pieces to stage
  for (int i = threadIdx.x; i < n4; i += THREADS) {
    const int t = i / (nb * 8);
    const int rem = i - t * nb * 8;
    const int bb = rem >> 3, j = rem & 7;  // piece j holds elements 4j..4j+3 of block bb
    const int64_t src = static_cast<int64_t>(t) * k + 32 * (b_lo + bb) + 4 * j;
    half4_t h;
    if constexpr (XF16) {
      h = *reinterpret_cast<const half4_a4 *>(static_cast<const _Float16 *>(X) + src);
    } else {
      const float4_t f = *reinterpret_cast<const float4_a4 *>(static_cast<const float *>(X) + src);
      const half2_t a = cvt_half2(f.x, f.y), b = cvt_half2(f.z, f.w);
      h = half4_t{a.x, a.y, b.x, b.y};
    }
    const int g = QTraits<QT>::nibbles ? (j & 3) : (j >> 1);
    const int half_off = QTraits<QT>::nibbles ? 4 * (j >> 2) : 4 * (j & 1);
    *reinterpret_cast<half4_t *>(reinterpret_cast<_Float16 *>(xs + (4 * bb + g) * NT + t) + half_off) = h;
  }
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

// A block with a minimum offset (Q4_1): sum_i (d q_i + m) x_i =
// d * sum_i q_i x_i + m * sum_i x_i. The second sum comes from one more MFMA
// with an all-ones B operand (every column then holds the block's sum of the
// fp16 activations of each token slot); dm_bits = d | m << 16.
template <int NT>
__device__ __forceinline__ void gemv_block_min(float acc[4], half8_t xop, half8_t wop, uint32_t dm_bits) {
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};
  const _Float16 one = static_cast<_Float16>(1.0f);
  const half8_t ones = {one, one, one, one, one, one, one, one};
  const float4_t part = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, wop, zero, 0, 0, 0);
  const float4_t sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, ones, zero, 0, 0, 0);
  const float d = half_bits_to_float(dm_bits & 0xFFFFu), m = half_bits_to_float(dm_bits >> 16);
  constexpr int E = NT < 4 ? NT : 4;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(m, sx[e], __builtin_fmaf(d, part[e], acc[e]));
}

// A Q4_K sub-block: sum_i (dsc q_i - dmm) x_i = dsc * sum_i q_i x_i - dmm *
// sum_i x_i, with dsc = d sc_j and dmm = dmin m_j exact in fp32; the second
// sum comes from an MFMA with an all-ones B operand, as for Q4_1.
template <int NT>
__device__ __forceinline__ void gemv_block_k(float acc[4], half8_t xop, half8_t wop, float dsc, float dmm) {
  const float4_t zero = {0.f, 0.f, 0.f, 0.f};
  const _Float16 one = static_cast<_Float16>(1.0f);
  const half8_t ones = {one, one, one, one, one, one, one, one};
  const float4_t part = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, wop, zero, 0, 0, 0);
  const float4_t sx = __builtin_amdgcn_mfma_f32_16x16x32_f16(xop, ones, zero, 0, 0, 0);
  constexpr int E = NT < 4 ? NT : 4;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(dsc, part[e], __builtin_fmaf(-dmm, sx[e], acc[e]));
}

// One block's contribution for any type: dm_bits = d (low half) and, for a
// type with a minimum, m (high half).
template <int QT, int NT>
__device__ __forceinline__ void gemv_any_block(float acc[4], half8_t xop, half8_t wop, uint32_t dm_bits) {
  if constexpr (QTraits<QT>::has_min)
    gemv_block_min<NT>(acc, xop, wop, dm_bits);
  else
    gemv_block<NT>(acc, xop, wop, dm_bits & 0xFFFFu);
}

}  // namespace qmm
