// Device-side helpers shared by the kernels: vector types, binary16 handling
// and in-register unpacking of GGUF block codes into exact fp16 integers.
//
// Block layout ([Bind] = "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section
// 2.3): Q4_0 = binary16 d + 16 bytes of nibbles (element j in the low nibble
// of byte j, element j + 16 in the high nibble); Q8_0 = binary16 d + 32 int8.
// Reconstruction ([Arch] = "llama.cpp 源码完全拆解(一)：整体架构与模块全景",
// section "权重装载：GGUF、mmap 与 4 bit 块"): w = d * (q - z), z = 8 for Q4_0
// and 0 for Q8_0. Q4_1, the legacy type with a minimum offset (same page,
// the paragraph on the three quantisation families): binary16 d, binary16 m,
// then Q4_0's 16 nibble bytes; w = d * q + m with unsigned codes 0..15.
// Q5_0 / Q5_1 (the other legacy types; their packing is this library's
// reading): d (and m for Q5_1), a 32-bit word whose bit j is the fifth bit
// of element j, then 16 nibble bytes with the low four bits; codes 0..31,
// w = d * (q - 16) for Q5_0 and d * q + m for Q5_1.
// Q4_K (a k-quant; the same page says k-quants use 256-weight blocks whose
// scales and minimums are stored in two levels; the bit layout is this
// library's reading, the GGUF one): a 144-byte super-block of 256 weights =
// binary16 d, binary16 dmin, 12 bytes of eight 6-bit sub-block scales sc_j
// and minimums m_j, 128 code bytes (byte 32 c + l: element 64 c + l in the
// low nibble, element 64 c + 32 + l in the high one); w = d sc_j q - dmin m_j.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qmm.h"

namespace qmm {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// Multi-dword global loads need only dword alignment on CDNA, so these types
// let the compiler emit dwordx2/x3/x4 loads from 4-byte-aligned addresses.
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float float4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef _Float16 half4_a4 __attribute__((ext_vector_type(4), aligned(4)));

template <int QT> struct Block;
template <> struct Block<QMM_TYPE_Q4_0> { static constexpr int bytes = 18; };
template <> struct Block<QMM_TYPE_Q4_1> { static constexpr int bytes = 20; };
template <> struct Block<QMM_TYPE_Q5_0> { static constexpr int bytes = 22; };
template <> struct Block<QMM_TYPE_Q5_1> { static constexpr int bytes = 24; };
template <> struct Block<QMM_TYPE_Q8_0> { static constexpr int bytes = 34; };
// Q4_K: bytes per 32 weights (a 256-weight super-block is 144 bytes), so that
// the decode kernel's 8-block quads are exactly one super-block
template <> struct Block<QMM_TYPE_Q4_K> { static constexpr int bytes = 18; };

// nibbles: (low) 4-bit codes in Q4_0's byte order; has_min: a binary16 m
// follows d; has_qh: a 32-bit word of fifth bits follows (at byte qh);
// codes: byte offset of the code bytes; zero: the zero point z.
template <int QT> struct QTraits {
  static constexpr bool nibbles = QT != QMM_TYPE_Q8_0;
  static constexpr bool has_min = QT == QMM_TYPE_Q4_1 || QT == QMM_TYPE_Q5_1;
  static constexpr bool has_qh = QT == QMM_TYPE_Q5_0 || QT == QMM_TYPE_Q5_1;
  static constexpr int qh = has_min ? 4 : 2;
  static constexpr int codes = 2 + (has_min ? 2 : 0) + (has_qh ? 4 : 0);
  static constexpr int zero = QT == QMM_TYPE_Q4_0 ? 8 : QT == QMM_TYPE_Q5_0 ? 16 : 0;
  // 256-weight super-blocks with 6-bit sub-block scales and minimums
  static constexpr bool kquant = QT == QMM_TYPE_Q4_K;
};

// Calls f(std::integral_constant<int, QT>) for the run-time type id (one of
// the three the library accepts; the entry points validate it first).
// by_qtype covers the 32-weight block types; by_qtype_k also Q4_K (for the
// kernels that take it: the decoder, the streaming decode kernel, the GEMM).
template <class F> __host__ inline auto by_qtype(int qtype, F f) {
  if (qtype == QMM_TYPE_Q4_0) return f(std::integral_constant<int, QMM_TYPE_Q4_0>{});
  if (qtype == QMM_TYPE_Q4_1) return f(std::integral_constant<int, QMM_TYPE_Q4_1>{});
  if (qtype == QMM_TYPE_Q5_0) return f(std::integral_constant<int, QMM_TYPE_Q5_0>{});
  if (qtype == QMM_TYPE_Q5_1) return f(std::integral_constant<int, QMM_TYPE_Q5_1>{});
  return f(std::integral_constant<int, QMM_TYPE_Q8_0>{});
}
template <class F> __host__ inline auto by_qtype_k(int qtype, F f) {
  if (qtype == QMM_TYPE_Q4_K) return f(std::integral_constant<int, QMM_TYPE_Q4_K>{});
  return by_qtype(qtype, f);
}

__device__ __forceinline__ uint32_t ld_u16(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }
__device__ __forceinline__ uint32_t ld_u32(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
__device__ __forceinline__ u32x2_t ld_u32x2(const uint8_t *p) {
  u32x2_a4 v = *reinterpret_cast<const u32x2_a4 *>(p);
  return u32x2_t{v.x, v.y};
}

// Exact binary16 -> fp32 widening of a scale (hardware conversion; every
// binary16 value, subnormals included, is representable in fp32).
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}
__device__ __forceinline__ half2_t as_half2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Bytes [2, 6) of the 8-byte window (lo, hi): a dword that starts 2 bytes
// into `lo`.
__device__ __forceinline__ uint32_t shift16(uint32_t lo, uint32_t hi) { return __builtin_amdgcn_alignbit(hi, lo, 16); }

// v_perm_b32 selectors: destination bytes take source bytes 4..7 (the first
// operand) or 0x64 from the magic second operand. Half (lo) = 0x64bb where
// bb is the selected byte, i.e. the fp16 value 1024 + bb.
constexpr uint32_t kMagic64 = 0x64646464u;
constexpr uint32_t kSelB01 = 0x00050004u;  // halves (1024 + byte0, 1024 + byte1)
constexpr uint32_t kSelB23 = 0x00070006u;  // halves (1024 + byte2, 1024 + byte3)

__device__ __forceinline__ half2_t bytes01_plus_1024(uint32_t v) { return as_half2(__builtin_amdgcn_perm(v, kMagic64, kSelB01)); }
__device__ __forceinline__ half2_t bytes23_plus_1024(uint32_t v) { return as_half2(__builtin_amdgcn_perm(v, kMagic64, kSelB23)); }

// Four nibble code bytes qs[j..j+3] -> eight exact fp16 values (q - Z):
//   out[0] = (e_j, e_j+1), out[1] = (e_j+2, e_j+3)          (low nibbles)
//   out[2] = (e_j+16, e_j+17), out[3] = (e_j+18, e_j+19)    (high nibbles)
// Low nibble n: 1024 + n - (1024 + Z) = n - Z. High nibble m (kept in place,
// so the byte is 16 m): (1024 + 16 m) / 16 - (64 + Z) = m - Z. Both steps
// are exact. Z = 8 for Q4_0, 0 for Q4_1.
template <int Z = 8>
__device__ __forceinline__ void q4_unpack(uint32_t qs, half2_t out[4]) {
  const half2_t mlo = {(_Float16)(-1024.0f - Z), (_Float16)(-1024.0f - Z)};
  const half2_t s16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t mhi = {(_Float16)(-64.0f - Z), (_Float16)(-64.0f - Z)};
  const uint32_t lo = qs & 0x0F0F0F0Fu;
  const uint32_t hi = qs & 0xF0F0F0F0u;
  out[0] = bytes01_plus_1024(lo) + mlo;
  out[1] = bytes23_plus_1024(lo) + mlo;
  out[2] = bytes01_plus_1024(hi) * s16 + mhi;
  out[3] = bytes23_plus_1024(hi) * s16 + mhi;
}

// Four bits h (bit i for byte i) moved to bit 4 of each byte of a dword: the
// multiply by 1 + 2^7 + 2^14 + 2^21 puts bit i at bit 8 i (among others that
// the mask drops).
__device__ __forceinline__ uint32_t spread4_to_bit4(uint32_t h) {
  return ((__umul24(h, 0x00204081u)) & 0x01010101u) << 4;
}

// Four 5-bit code bytes qs[j0..j0+3] with their fifth bits from qh (bit j
// for element j) -> eight exact fp16 values (q - Z), in q4_unpack's order:
//   out[0..1] = elements j0..j0+3, out[2..3] = elements j0+16..j0+19.
template <int Z>
__device__ __forceinline__ void q5_unpack(uint32_t qs, uint32_t qh, int j0, half2_t out[4]) {
  const half2_t mz = {(_Float16)(-1024.0f - Z), (_Float16)(-1024.0f - Z)};
  const uint32_t lo = (qs & 0x0F0F0F0Fu) | spread4_to_bit4(__builtin_amdgcn_ubfe(qh, j0, 4));
  const uint32_t hi = ((qs >> 4) & 0x0F0F0F0Fu) | spread4_to_bit4(__builtin_amdgcn_ubfe(qh, j0 + 16, 4));
  out[0] = bytes01_plus_1024(lo) + mz;
  out[1] = bytes23_plus_1024(lo) + mz;
  out[2] = bytes01_plus_1024(hi) + mz;
  out[3] = bytes23_plus_1024(hi) + mz;
}

// Four Q8_0 int8 codes -> four exact fp16 values: (c ^ 0x80) = c + 128 as an
// unsigned byte u; 1024 + u - 1152 = c.
__device__ __forceinline__ void q8_unpack(uint32_t qs, half2_t out[2]) {
  const half2_t m1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const uint32_t u = qs ^ 0x80808080u;
  out[0] = bytes01_plus_1024(u) + m1152;
  out[1] = bytes23_plus_1024(u) + m1152;
}

__device__ __forceinline__ half8_t make_half8(half2_t a, half2_t b, half2_t c, half2_t d) {
  return half8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Q4_K: sub-block j's 6-bit scale and minimum from the 12 scale bytes held
// as three little-endian dwords (s0 = bytes 0-3, s1 = 4-7, s2 = 8-11). For
// j < 4 they are the low 6 bits of bytes j and j + 4; for j >= 4 the low 4
// bits come from the nibbles of byte j + 4 and the high 2 from the top bits
// of bytes j - 4 (scale) and j (minimum).
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j, uint32_t &sc,
                                              uint32_t &m) {
  if (j < 4) {
    sc = (s0 >> (8 * j)) & 63u;
    m = (s1 >> (8 * j)) & 63u;
  } else {
    const int i = 8 * (j - 4);
    const uint32_t b = s2 >> i;
    sc = (b & 15u) | (((s0 >> (i + 6)) & 3u) << 4);
    m = ((b >> 4) & 15u) | (((s1 >> (i + 6)) & 3u) << 4);
  }
}

// fp32 -> fp16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ half2_t cvt_half2(float a, float b) { return __builtin_convertvector(float2_t{a, b}, half2_t); }

}  // namespace qmm
