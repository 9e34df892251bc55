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
// a 128-row x 128-token output tile; its four wavefronts each compute 64 x 64
// as 4 x 4 MFMA tiles. k advances in stages of 64 (two blocks):
//  * staging: each thread loads half of one row's two blocks (5, 6 or 9
//    dwords inside the pair) and half of one token's 64 activations, two
//    stages ahead of their use, decodes the blocks to fp16 d * (q - z) or
//    d * q + m (exact integer code, one fp16 rounding) and stores weights and
//    activations into LDS;
//  * LDS is double-buffered, so the stores of stage s + 1 (and their decode
//    arithmetic) overlap the MFMAs of stage s, with one LDS-only barrier per
//    stage; rows of 128 bytes with their 16-byte chunks permuted by
//    row (lds_at) keep the stores and the MFMA operand reads free of bank
//    conflicts;
//  * within a stage the MFMAs are interleaved with the decode, the LDS
//    stores and the loads of the next stages (interleave_stage);
//  * two workgroups fit a CU (64 KiB of LDS each), so one's loads and
//    barriers overlap the other's matrix work; launches with few tiles use
//    64-row tiles (three workgroups per CU).
// Weights never exist in dequantised form outside LDS.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace qmm {

constexpr int kBM = 128;  // weight rows per tile
constexpr int kBN = kTileTokens;  // tokens per tile (128)
constexpr int kBK = 64;   // k per stage (2 blocks)
// LDS tiles are 128 rows x 64 halves, 128 bytes per row without padding;
// 16-byte chunk c of row r sits at chunk position c ^ (r % 8). On gfx950 this
// keeps the MFMA operand reads (row lane % 16, chunk lane / 16 + 4 h) and
// both staging stores free of LDS bank conflicts, which a padded 144-byte
// pitch does not for the reads (measured: twice the LDS cycles per read).
__device__ __forceinline__ int lds_at(int row, int chunk) { return row * kBK + 8 * (chunk ^ (row & 7)); }
constexpr int kGemmThreads = 256;
constexpr int kXcds = 8;       // XCDs of the GPU; workgroups are dealt to them round-robin
constexpr int kGroupRows = 8;  // row tiles per group of the tile order
static_assert(kGemmThreads == 2 * kBM && kGemmThreads == 2 * kBN, "two staging threads per row and per token");

// d (and m, in the high half, for a type with a minimum) and the code dwords
// of one block, with 16-bit loads.
// (and the fifth-bit word, for a 5-bit type, in q[0] before the codes)
template <int QT>
__device__ __forceinline__ void load_block_u16(const uint8_t *p, uint32_t &d, uint32_t *q) {
  constexpr int nq = QTraits<QT>::nibbles ? 4 : 8;
  constexpr int c = QTraits<QT>::codes;
  constexpr int h = QTraits<QT>::has_qh ? 1 : 0;
  d = ld_u16(p);
  if constexpr (QTraits<QT>::has_min) d |= ld_u16(p + 2) << 16;
  if constexpr (QTraits<QT>::has_qh) q[0] = ld_u16(p + QTraits<QT>::qh) | (ld_u16(p + QTraits<QT>::qh + 2) << 16);
#pragma unroll
  for (int i = 0; i < nq; ++i) q[h + i] = ld_u16(p + c + 4 * i) | (ld_u16(p + c + 2 + 4 * i) << 16);
}

// Decode one block to 32 fp16 weights fl16(d * (q - z)) (Q4_1: fl16(d q + m),
// one fp16 fma, a single rounding of the exact value) in element order and
// store them as chunks c0 .. c0 + 3 of LDS tile row `row`. d_bits holds d in
// its low half and, for Q4_1, m in its high half.
template <int QT>
__device__ __forceinline__ void store_block_f16(_Float16 *tile, int row, int c0, uint32_t d_bits, const uint32_t *q,
                                                uint32_t qh = 0) {
  const _Float16 dh = __builtin_bit_cast(_Float16, static_cast<uint16_t>(d_bits));
  const half2_t d2 = {dh, dh};
  half2_t h[16];
  if constexpr (QT == QMM_TYPE_Q4_0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t u[4];
      q4_unpack<8>(q[i], u);
      h[2 * i] = u[0] * d2;      // elements 4i, 4i+1
      h[2 * i + 1] = u[1] * d2;  // 4i+2, 4i+3
      h[8 + 2 * i] = u[2] * d2;  // 16+4i, 17+4i
      h[9 + 2 * i] = u[3] * d2;  // 18+4i, 19+4i
    }
  } else if constexpr (QTraits<QT>::has_qh) {
    // 5-bit codes: fl16(d (q - z)), or fl16(d q + m) with one fp16 fma
    const _Float16 mh = __builtin_bit_cast(_Float16, static_cast<uint16_t>(d_bits >> 16));
    const half2_t m2 = {mh, mh};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t u[4];
      q5_unpack<QTraits<QT>::zero>(q[i], qh, 4 * i, u);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int at = e < 2 ? 2 * i + e : 8 + 2 * i + (e - 2);
        if constexpr (QTraits<QT>::has_min)
          h[at] = __builtin_elementwise_fma(u[e], d2, m2);
        else
          h[at] = u[e] * d2;
      }
    }
  } else if constexpr (QT == QMM_TYPE_Q4_1) {
    const _Float16 mh = __builtin_bit_cast(_Float16, static_cast<uint16_t>(d_bits >> 16));
    const half2_t m2 = {mh, mh};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t u[4];
      q4_unpack<0>(q[i], u);
      h[2 * i] = __builtin_elementwise_fma(u[0], d2, m2);
      h[2 * i + 1] = __builtin_elementwise_fma(u[1], d2, m2);
      h[8 + 2 * i] = __builtin_elementwise_fma(u[2], d2, m2);
      h[9 + 2 * i] = __builtin_elementwise_fma(u[3], d2, m2);
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
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<u32x4_t *>(tile + lds_at(row, c0 + i)) =
        u32x4_t{as_u32(h[4 * i]), as_u32(h[4 * i + 1]), as_u32(h[4 * i + 2]), as_u32(h[4 * i + 3])};
}

// One staging thread's half of a stage's pair of blocks (h = 0: block 2 s,
// h = 1: block 2 s + 1), as raw dwords. With 4-byte-aligned rows and a whole
// pair, half 0 is the pair's first nq + 1 dwords (scale = low half of w[0],
// codes = bytes 2.. = w shifted by 16 bits) and half 1 its last nq + 1 dwords
// (scale = high half of w[0], codes = w[1..]); all lie inside the pair. The
// loaded dwords are not touched until the stage is stored, so the loads stay
// in flight (any arithmetic on them right after the load would wait for it).
// Blocks whose size is a multiple of 4 (Q4_1, Q5_1) are dword-aligned in a
// pair: both halves are one whole block, d|m in w[0] and the rest after it.
// The 5-bit types add the fifth-bit word before the codes: w[1] (Q5_0 half
// 0: shifted by 16 bits like everything else), codes in w[2..5].
template <int QT> struct HalfRaw {
  static constexpr int nq = (QTraits<QT>::nibbles ? 4 : 8) + (QTraits<QT>::has_qh ? 1 : 0);
  uint32_t w[nq + 1];
};

template <int QT>
__device__ __forceinline__ HalfRaw<QT> load_half_pair_blocks(const uint8_t *rp, int st, int h);

// Q4_K: a stage (64 weights) is code chunk st % 4 of super-block st / 4,
// whose low nibbles are sub-block 2 (st % 4) and high nibbles sub-block
// 2 (st % 4) + 1; half h keeps the 16-byte header (d | dmin, scale bytes)
// and the chunk's 32 code bytes, and j = its sub-block. Rows are 16-byte
// aligned (the entry points require it for this type).
template <> struct HalfRaw<QMM_TYPE_Q4_K> {
  static constexpr int nq = 11;
  uint32_t w[12];
  int j;
};

template <int QT>
__device__ __forceinline__ HalfRaw<QT> load_half_pair(const uint8_t *rp, int st, int h) {
  if constexpr (QTraits<QT>::kquant) {
    const uint8_t *sb = rp + static_cast<int64_t>(st >> 2) * 144;
    const u32x4_t a = *reinterpret_cast<const u32x4_t *>(sb);
    const u32x4_t b = *reinterpret_cast<const u32x4_t *>(sb + 16 + 32 * (st & 3));
    const u32x4_t c = *reinterpret_cast<const u32x4_t *>(sb + 32 + 32 * (st & 3));
    HalfRaw<QT> r;
    r.w[0] = a.x, r.w[1] = a.y, r.w[2] = a.z, r.w[3] = a.w;
    r.w[4] = b.x, r.w[5] = b.y, r.w[6] = b.z, r.w[7] = b.w;
    r.w[8] = c.x, r.w[9] = c.y, r.w[10] = c.z, r.w[11] = c.w;
    r.j = 2 * (st & 3) + h;
    return r;
  } else {
    return load_half_pair_blocks<QT>(rp, st, h);
  }
}

template <int QT>
__device__ __forceinline__ HalfRaw<QT> load_half_pair_blocks(const uint8_t *rp, int st, int h) {
  constexpr int nq = HalfRaw<QT>::nq;
  constexpr int BB = Block<QT>::bytes;
  constexpr int h1 = BB % 4 == 0 ? BB : BB - 2;  // half 1 starts here, 4-byte aligned
  const uint8_t *p = rp + static_cast<int64_t>(st) * (2 * BB) + (h ? h1 : 0);
  HalfRaw<QT> r;
  constexpr int NW = nq + 1;
#pragma unroll
  for (int i = 0; i + 4 <= NW; i += 4) {
    const u32x4_a4 v = *reinterpret_cast<const u32x4_a4 *>(p + 4 * i);
    r.w[i] = v.x; r.w[i + 1] = v.y; r.w[i + 2] = v.z; r.w[i + 3] = v.w;
  }
  if constexpr (NW % 4 == 2) {
    const u32x2_t v = ld_u32x2(p + 4 * (NW - 2));
    r.w[NW - 2] = v.x; r.w[NW - 1] = v.y;
  } else if constexpr (NW % 4 == 1) {
    r.w[NW - 1] = ld_u32(p + 4 * (NW - 1));
  }
  return r;
}

// Block blk of the row with 16-bit loads (any even row stride), in the
// layout of half 1 (scale in the high half of w[0], codes in w[1..]); a block
// at or past nblk reads as zero codes with a zero scale.
template <int QT>
__device__ __forceinline__ HalfRaw<QT> load_half_u16(const uint8_t *rp, int blk, int nblk) {
  constexpr int nq = HalfRaw<QT>::nq;
  if constexpr (QTraits<QT>::kquant) {
    // Q4_K rows are always 16-byte aligned and hold whole stages
    return load_half_pair<QT>(rp, blk >> 1, blk & 1);
  }
  HalfRaw<QT> r;
  if (blk < nblk) {
    uint32_t d;
    load_block_u16<QT>(rp + static_cast<int64_t>(blk) * Block<QT>::bytes, d, r.w + 1);
    r.w[0] = QTraits<QT>::has_min ? d : d << 16;  // the layout of half 1
  } else {
#pragma unroll
    for (int i = 0; i <= nq; ++i) r.w[i] = 0;
  }
  return r;
}

// Decode a half (layout of half 0 if first_layout, else of half 1) and
// store its 32 fp16 weights as chunks c0 .. c0 + 3 of tile row `row`.
// first_layout may differ between lanes.
template <int QT>
__device__ __forceinline__ void store_half(_Float16 *tile, int row, int c0, const HalfRaw<QT> &r, bool first_layout) {
  constexpr int nq = HalfRaw<QT>::nq;
  if constexpr (QTraits<QT>::kquant) {
    // sub-block j: fp32 fma(q, d sc_j, -dmin m_j) (both products exact, one
    // rounding), then fp16; element 4 i + b is byte b of code dword i
    uint32_t sc, mn;
    q4k_scale_min(r.w[1], r.w[2], r.w[3], r.j, sc, mn);
    const float dsc = half_bits_to_float(r.w[0] & 0xFFFFu) * static_cast<float>(sc);
    const float dmm = half_bits_to_float(r.w[0] >> 16) * static_cast<float>(mn);
    const int shift = 4 * (r.j & 1);
    uint32_t h[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t v = (r.w[4 + i] >> shift) & 0x0F0F0F0Fu;
      const float f0 = __builtin_fmaf(static_cast<float>(v & 0xFFu), dsc, -dmm);
      const float f1 = __builtin_fmaf(static_cast<float>((v >> 8) & 0xFFu), dsc, -dmm);
      const float f2 = __builtin_fmaf(static_cast<float>((v >> 16) & 0xFFu), dsc, -dmm);
      const float f3 = __builtin_fmaf(static_cast<float>(v >> 24), dsc, -dmm);
      h[2 * i] = as_u32(cvt_half2(f0, f1));
      h[2 * i + 1] = as_u32(cvt_half2(f2, f3));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4_t *>(tile + lds_at(row, c0 + i)) = u32x4_t{h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]};
    (void)first_layout;
    return;
  }
  uint32_t q[nq];
  if constexpr (QTraits<QT>::has_min) {  // one layout for both halves
#pragma unroll
    for (int i = 0; i < nq; ++i) q[i] = r.w[i + 1];
    if constexpr (QTraits<QT>::has_qh)
      store_block_f16<QT>(tile, row, c0, r.w[0], q + 1, q[0]);
    else
      store_block_f16<QT>(tile, row, c0, r.w[0], q);
    return;
  }
  const uint32_t d = first_layout ? (r.w[0] & 0xFFFFu) : (r.w[0] >> 16);
#pragma unroll
  for (int i = 0; i < nq; ++i) q[i] = first_layout ? shift16(r.w[i], r.w[i + 1]) : r.w[i + 1];
  if constexpr (QTraits<QT>::has_qh)
    store_block_f16<QT>(tile, row, c0, d, q + 1, q[0]);
  else
    store_block_f16<QT>(tile, row, c0, d, q);
}

// Activations of one stage (128 tokens x 64 k) as 16-byte pieces spread so
// that consecutive lanes read consecutive pieces of one token's row: a
// wavefront's load covers whole 128-byte runs of a few rows instead of one
// piece of 64 different rows (which costs the address unit a cache line per
// lane). fp16: piece c = 256 i + tid (i < 4) is token c / 8, elements
// 8 (c % 8) .. +7; fp32: piece c = 256 i + tid (i < 8) is token c / 16,
// elements 4 (c % 16) .. +3.
template <bool XF16> struct XPieces;
template <> struct XPieces<true> { u32x4_t v[4]; };
template <> struct XPieces<false> { float4_t v[8]; };

template <bool XF16> struct XMap {
  static constexpr int n = XF16 ? 4 : 8;         // pieces per thread
  static constexpr int per_tok = XF16 ? 8 : 16;  // pieces per token row of a stage
  static constexpr int elems = XF16 ? 8 : 4;     // elements per piece
};

// Token rows are clamped to the last token; k0 + elements past k (the
// missing second block of an odd count) read as zeros when `tail`.
template <bool XF16>
__device__ __forceinline__ XPieces<XF16> load_x_pieces(const void *X, int tok0, int n_tokens, int k, int k0, int tid,
                                                       bool tail) {
  using M = XMap<XF16>;
  XPieces<XF16> r;
#pragma unroll
  for (int i = 0; i < M::n; ++i) {
    const int c = 256 * i + tid;
    const int tok = min(tok0 + c / M::per_tok, n_tokens - 1);
    const int e = k0 + M::elems * (c % M::per_tok);
    const int64_t off = static_cast<int64_t>(tok) * k + e;
    if (!tail || e < k) {
      if constexpr (XF16)
        r.v[i] = *reinterpret_cast<const u32x4_a4 *>(static_cast<const _Float16 *>(X) + off);
      else
        r.v[i] = *reinterpret_cast<const float4_a4 *>(static_cast<const float *>(X) + off);
    } else {
      if constexpr (XF16)
        r.v[i] = u32x4_t{0u, 0u, 0u, 0u};
      else
        r.v[i] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
  return r;
}

template <bool XF16>
__device__ __forceinline__ void store_x_pieces(_Float16 *xs, const XPieces<XF16> &r, int tid) {
  using M = XMap<XF16>;
#pragma unroll
  for (int i = 0; i < M::n; ++i) {
    const int c = 256 * i + tid;
    const int tok = c / M::per_tok, e = M::elems * (c % M::per_tok);
    _Float16 *dst = xs + lds_at(tok, e >> 3) + (e & 7);
    if constexpr (XF16) {
      *reinterpret_cast<u32x4_t *>(dst) = r.v[i];
    } else {
      const float4_t f = r.v[i];
      *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{as_u32(cvt_half2(f.x, f.y)), as_u32(cvt_half2(f.z, f.w))};
    }
  }
}

// The routed form: piece i of a thread belongs to token slot c / per_tok of
// the tile, whose activation row starts at xrow[i] (gathered once per tile).
template <bool XF16>
__device__ __forceinline__ XPieces<XF16> load_x_rows(const float *const *xrow, int k, int k0, int tid, bool tail) {
  static_assert(!XF16, "routed activations are fp32");
  using M = XMap<XF16>;
  XPieces<XF16> r;
#pragma unroll
  for (int i = 0; i < M::n; ++i) {
    const int e = k0 + M::elems * (tid % M::per_tok);
    if (!tail || e < k)
      r.v[i] = *reinterpret_cast<const float4_a4 *>(xrow[i] + e);
    else
      r.v[i] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  return r;
}

// Workgroup barrier that waits for LDS accesses only: __syncthreads() would
// also wait for the global loads of later stages, which are meant to stay in
// flight across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Instruction order for one pipelined stage (32 MFMAs, the next stage's
// decode and LDS stores, its global loads): the first operand reads, then
// each MFMA followed by two VALU instructions of the decode, with an LDS
// store, an operand read and a global load spread between them. A wavefront
// issues in order, so without this the 32 MFMAs go out back to back and the
// decode waits behind them; interleaved, the decode runs while the matrix
// cores work.
template <int NMFMA = 32>
__device__ __forceinline__ void interleave_stage() {
  constexpr int kDsRead = 0x100, kDsWrite = 0x200, kMfma = 0x008, kValu = 0x002, kVmemRead = 0x020;
#pragma unroll
  for (int i = 0; i < NMFMA / 4; ++i) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kValu, 2, 0);
    if ((i & 3) == 0) __builtin_amdgcn_sched_group_barrier(kDsWrite, 1, 0);
    if ((i & 3) == 2) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    if ((i & 7) == 5) __builtin_amdgcn_sched_group_barrier(kVmemRead, 1, 0);
  }
}

// Expert routing (MUL_MAT_ID): token tile t of the grid is tiles[t] =
// (expert, first entry, count) of `list`, the (token, slot) pairs grouped by
// expert; entry j of the tile is pair p = list[first + j], whose activation
// row is X[p / n_ids][x_slots > 1 ? p % n_ids : 0] and output row Y[p]. A
// tile with count 0 is empty.
struct GemmRoute {
  const int32_t *list;
  const int32_t *tiles;  // 4 ints per tile
  int64_t nb2;
  int n_ids, x_slots;
};

// BM = 128 rows per tile, or 64 for launches with few tiles: each
// wavefront then computes 32 x 64, only the first 128 threads stage
// weights, and (with fp16 activations) three workgroups fit a CU.
// KS = 2 (64-row tiles, a block count that is a multiple of 4): the
// workgroup holds two groups of four wavefronts, each taking half of k with
// LDS stages of its own; the second group's partial tile is added to the
// first's through LDS in a fixed order before the store. A launch that
// fills only one wavefront per SIMD then has two, with no memory beyond LDS.
template <int QT, bool XF16, bool ALIGN4, bool ROUTED = false, int BM = kBM, int KS = 1>
__global__ __launch_bounds__(kGemmThreads * KS, KS == 2 ? 1 : ((BM == kBM || !XF16) ? 2 : 3)) void gemm_kernel(
    const uint8_t *__restrict__ W, int n_rows, int nblk, int64_t nb1, const void *__restrict__ X, int n_tokens, int k,
    float *__restrict__ Y, bool y_vec4, int row_tiles, GemmRoute route) {
  static_assert(BM == kBM || (BM == kBM / 2 && !ROUTED), "128-row tiles, or 64 for the plain product");
  static_assert(KS == 1 || (KS == 2 && BM == kBM / 2 && !ROUTED), "the k split is for plain 64-row tiles");
  constexpr int MI = BM / 32;  // 16-row MFMA tiles per wavefront
  constexpr int kTileHalves = 2 * (BM + kBN) * kBK;  // one group's two stages of weights and activations
  __shared__ __attribute__((aligned(16))) _Float16 lds_static[KS == 1 ? kTileHalves : 8];
  extern __shared__ __attribute__((aligned(16))) _Float16 lds_dynamic[];
  const int kg = KS == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kGemmThreads);
  _Float16 *lds_group = (KS == 1 ? lds_static : lds_dynamic) + kg * kTileHalves;
  _Float16 *Ws[2] = {lds_group, lds_group + BM * kBK};
  _Float16 *Xs[2] = {lds_group + 2 * BM * kBK, lds_group + 2 * BM * kBK + kBN * kBK};

  const int tid = static_cast<int>(threadIdx.x) - kg * kGemmThreads;  // thread within the k group
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const bool wstage = BM == kBM || tid < 2 * BM;  // uniform per wavefront
  // Tile of this workgroup. Workgroups go to the 8 XCDs round-robin, so
  // XCD x = blockIdx % 8 takes a contiguous range of tile numbers (a plain
  // 1-D order for the remainder); within it, tiles run over groups of
  // kGroupRows row tiles, row tile fastest, so the workgroups of one XCD share
  // weight rows and activation tokens in its L2.
  const int n_tiles = static_cast<int>(gridDim.x);
  const int bid = static_cast<int>(blockIdx.x);
  const int per_xcd = n_tiles / kXcds;
  const int lin = bid < per_xcd * kXcds ? (bid % kXcds) * per_xcd + bid / kXcds : bid;
  const int tok_tiles = n_tiles / row_tiles;
  const int in_group = kGroupRows * tok_tiles;
  const int first_row = (lin / in_group) * kGroupRows;
  const int group_rows = min(row_tiles - first_row, kGroupRows);
  const int row0 = (first_row + (lin % in_group) % group_rows) * BM;
  int tok0 = ((lin % in_group) / group_rows) * kBN;

  int list0 = 0;
  const float *xrow[XMap<XF16>::n];
  if constexpr (ROUTED) {
    const int *td = route.tiles + 4 * (tok0 / kBN);
    const int e = __builtin_amdgcn_readfirstlane(td[0]);
    list0 = __builtin_amdgcn_readfirstlane(td[1]);
    n_tokens = __builtin_amdgcn_readfirstlane(td[2]);
    if (n_tokens == 0) return;  // whole workgroup: an unused tile
    W += static_cast<int64_t>(e) * route.nb2;
    tok0 = 0;
    using M = XMap<XF16>;
#pragma unroll
    for (int i = 0; i < M::n; ++i) {
      const int slot = min((256 * i + tid) / M::per_tok, n_tokens - 1);
      const int p = route.list[list0 + slot];
      const int t = p / route.n_ids;
      const int64_t xr = static_cast<int64_t>(t) * route.x_slots + (route.x_slots > 1 ? p - t * route.n_ids : 0);
      xrow[i] = static_cast<const float *>(X) + xr * k;
    }
  }

  // Weight staging: thread -> (row, half of the stage's block pair). The two
  // halves of a row sit in adjacent lanes, so each load instruction touches
  // 32 rows rather than 64. Rows past the end re-read the last one.
  const int srow = (tid >> 1) & (BM - 1), sh = tid & 1;
  const uint8_t *rp = W + static_cast<int64_t>(min(row0 + srow, n_rows - 1)) * nb1;

  float4_t acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    HalfRaw<QT> w;
    XPieces<XF16> x;
  };
  // Stages with a whole pair of blocks; an odd block count leaves one more.
  // With KS = 2 each group takes half of them (nblk % 4 == 0): group kg
  // computes stages st0 .. st0 + n_full - 1.
  const int n_full = nblk / (2 * KS);
  const int st0 = kg * n_full;
  auto load = [&](Stage &r, int st) {
    if (wstage) {
      if constexpr (ALIGN4)
        r.w = load_half_pair<QT>(rp, st0 + st, sh);
      else
        r.w = load_half_u16<QT>(rp, 2 * (st0 + st) + sh, nblk);
    }
    if constexpr (ROUTED)
      r.x = load_x_rows<XF16>(xrow, k, kBK * st, tid, false);
    else
      r.x = load_x_pieces<XF16>(X, tok0, n_tokens, k, kBK * (st0 + st), tid, false);
  };
  auto store = [&](int buf, const Stage &r) {
    if (wstage) store_half<QT>(Ws[buf], srow, 4 * sh, r.w, ALIGN4 && sh == 0);
    store_x_pieces<XF16>(Xs[buf], r.x, tid);
  };
  // operands: A (weights) row (BM / 2) wm + 16 i + lane % 16, B (activations)
  // token 64 wn + 16 j + lane % 16; elements 8 (lane / 16) .. +7 of k step
  // h (chunk lane / 16 + 4 h); rows 16 apart share the chunk swizzle.
  int aofs[2], bofs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    aofs[h] = lds_at((BM / 2) * wm + (lane & 15), (lane >> 4) + 4 * h);
    bofs[h] = lds_at(64 * wn + (lane & 15), (lane >> 4) + 4 * h);
  }
  auto compute = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      half8_t a[MI], b[4];
#pragma unroll
      for (int i = 0; i < MI; ++i) a[i] = *reinterpret_cast<const half8_t *>(Ws[buf] + aofs[h] + 16 * i * kBK);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const half8_t *>(Xs[buf] + bofs[h] + 16 * j * kBK);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  if (n_full > 0) {
    // Two register sets hold stages loaded two stages ahead of their use;
    // stage s + 1 is stored into the other LDS buffer while stage s is on the
    // matrix cores. Loads past the last whole stage re-read it (unconditional
    // loads keep the wait counts exact); such data is stored but never used.
    const int last = n_full - 1;
    Stage r0, r1;
    load(r0, 0);
    load(r1, min(1, last));
    store(0, r0);
    load(r0, min(2, last));
    lds_barrier();
    int s = 0;
    for (; s + 1 < n_full; s += 2) {
      compute(0);               // stage s
      store(1, r1);             // stage s + 1
      load(r1, min(s + 3, last));
      interleave_stage<8 * MI>();
      lds_barrier();
      compute(1);               // stage s + 1
      store(0, r0);             // stage s + 2 (a copy of the last stage at the end)
      load(r0, min(s + 4, last));
      interleave_stage<8 * MI>();
      lds_barrier();
    }
    if (s < n_full) compute(0);  // odd count of whole stages: the last one
  }
  if (KS == 1 && (nblk & 1)) {
    // the last, single block: half 0 loads it, half 1 stores zeros
    const int buf = n_full & 1;
    Stage t;
    if (wstage) t.w = load_half_u16<QT>(rp, 2 * n_full + sh, nblk);
    if constexpr (ROUTED)
      t.x = load_x_rows<XF16>(xrow, k, kBK * n_full, tid, true);
    else
      t.x = load_x_pieces<XF16>(X, tok0, n_tokens, k, kBK * n_full, tid, true);
    if (wstage) store_half<QT>(Ws[buf], srow, 4 * sh, t.w, false);
    store_x_pieces<XF16>(Xs[buf], t.x, tid);
    lds_barrier();
    compute(buf);
  }

  if constexpr (KS == 2) {
    // group 1's partial tile through LDS (its stage buffers are free once
    // every wavefront has passed this barrier), added to group 0's in a
    // fixed order; group 0 stores
    lds_barrier();
    float4_t *red = reinterpret_cast<float4_t *>(lds_dynamic) + (wave * 64 + lane) * (MI * 4);
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[i * 4 + j] = acc[i][j];
    }
    lds_barrier();
    if (kg == 1) return;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] += red[i * 4 + j];
  }
  // D element e of lane l in tile (i, j): row (BM / 2) wm + 16 i + 4 (l / 16) + e,
  // token 64 wn + 16 j + l % 16.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = tok0 + 64 * wn + 16 * j + (lane & 15);
    if (tok >= n_tokens) continue;
    const int64_t yr = ROUTED ? route.list[list0 + tok] : tok;
    float *yrow = Y + yr * n_rows;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = row0 + (BM / 2) * wm + 16 * i + 4 * (lane >> 4);
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

// Large launches with fp16 activations (at least one 128 x 256 tile per CU,
// an even block count): one workgroup of eight wavefronts per CU owns a
// 128-row x 256-token tile and runs as two groups of four that take turns
// ("ping-pong"). While one group issues the MFMAs of a stage from LDS, the
// other stages data for later stages; an LDS-only barrier ends each phase
// and the groups swap. Every SIMD holds one wavefront of each group, so its
// matrix core is fed by one of them while the other's staging runs beside
// it, instead of two wavefronts that reach their MFMAs and their decode at
// the same time. Each wavefront computes 64 x 64 (rows 64 (w % 2), tokens
// 128 g + 64 (w / 2)); a stage's weights are decoded once for 256 tokens,
// and the groups progress in lockstep, so neither finishes long after the
// other. The staging is split by kind so that every wavefront of a group
// has the same work: group 0 decodes the weights (one block of one row per
// thread, loaded from global memory two stages ahead into registers), group
// 1 copies the activations from global memory straight into LDS
// (global_load_lds: lane l's 16 bytes land at M0 + 16 l; no registers, VALU
// or LDS store instructions) three stages ahead, into four buffers (an L2
// hit under this load takes more than one stage to land).
constexpr int kPPThreads = 512;
constexpr int kPPBN = 256;                       // tokens per tile
constexpr int kPPWHalves = kBM * kBK;            // one weight stage (16 KiB)
constexpr int kPPXHalves = kPPBN * kBK;          // one activation stage (32 KiB)
constexpr int kPPXOps = kPPXHalves * 2 / (kGemmThreads * 16);  // copies per lane per stage (8)
constexpr int kPPXBufs = 4;
constexpr size_t kPPLds = (2 * kPPWHalves + kPPXBufs * kPPXHalves) * sizeof(_Float16);  // 160 KiB

__device__ __forceinline__ uint32_t lds_byte_addr(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}
// 16 bytes per lane from base + voff into LDS at m0 + 16 lane. M0 is written
// by a scalar move, and an LDS-DMA load must not follow it directly.
__device__ __forceinline__ void dma16(uint32_t voff, const void *base, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
               : "memory", "m0");
}
// The same with a per-lane 64-bit address (rows gathered through a list).
__device__ __forceinline__ void dma16(const void *p, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(p), "s"(lds) : "memory", "m0");
}
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// The k split of the workspace form, for launches of few tiles with long k:
// each of the t_sk tiles is computed by `parts` workgroups, part p (workgroup
// parts * tile + p) summing stages [n_st p / parts, n_st (p + 1) / parts).
// Each stores its partial sum into the workspace slot of (tile, p) and then
// counts it on the tile's counter with an agent-scope acquire-release add,
// which makes the stores visible to the workgroup that reads the count after
// it. The workgroup whose add completes the count adds the parts in k order,
// ((P0 + P1) + P2) + ..., and stores Y (with two parts, its own from
// registers: a sum of two terms is the same either way round), then sets the
// counter back to zero for the next call. No workgroup waits for another,
// and the order of the additions depends only on the shape and the CU
// count, so results repeat bit for bit.
// A launch may also run whole tiles before the split ones (t_whole of them,
// workgroups 0 .. t_whole - 1, the split tiles' workgroups after them): a
// launch of a few rounds of tiles whose last round would leave at least half
// of the CUs idle splits only that round's tiles in two, so it takes half a
// round.
struct PPSplit {
  int t_sk;        // split tiles
  int g_sk;        // workgroups (t_whole + t_sk * parts)
  int parts;       // parts per split tile
  int *cnt;        // t_sk counters, zero between calls
  float4_t *part;  // t_sk * parts partial tiles, kPPThreads * 16 float4 each
  int t_whole;     // tiles run whole, before the split ones
};

// The MUL_MATs of one launch: up to kPPMaxItems matrices of the same type and
// shape (rows, k, row stride, tokens), each with its own weights, fp16
// activations and output. Their row tiles follow one another in the tile
// order, as the row tiles of one matrix do, so independent MUL_MATs of a
// layer fill the rounds of a single launch together.
constexpr int kPPMaxItems = kGemmMaxItems;
struct PPItems {
  const uint8_t *W[kPPMaxItems];
  const _Float16 *X[kPPMaxItems];
  float *Y[kPPMaxItems];
  int n;
};

template <int QT, bool ALIGN4, bool SK>
__global__ __launch_bounds__(kPPThreads, 2) void gemm_pp_kernel(PPItems items, int n_rows, int nblk, int64_t nb1,
                                                                int n_tokens, int k, bool y_vec4, int row_tiles,
                                                                PPSplit sk) {
  extern __shared__ __attribute__((aligned(16))) _Float16 lds_dynamic[];
  _Float16 *const Wbuf = lds_dynamic;                   // 2 weight stages
  _Float16 *const Xbuf = lds_dynamic + 2 * kPPWHalves;  // kPPXBufs activation stages
  const int g = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kGemmThreads);
  const int tid = static_cast<int>(threadIdx.x) - g * kGemmThreads;  // thread within the group
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int n_st = nblk / 2;

  // tile order: as gemm_kernel (XCD-contiguous ranges, groups of row tiles)
  // over the tile's index: the workgroup's, or in the split form the tile's;
  // the row tiles are the items' row tiles one after another
  const int v_rows = items.n * row_tiles;
  const int n_tiles = SK ? sk.t_whole + sk.t_sk : static_cast<int>(gridDim.x);
  const int tok_tiles = n_tiles / v_rows;
  auto coords = [&](int bid, int &item, int &row0, int &tok0) {
    const int per_xcd = n_tiles / kXcds;
    const int lin = bid < per_xcd * kXcds ? (bid % kXcds) * per_xcd + bid / kXcds : bid;
    const int in_group = kGroupRows * tok_tiles;
    const int first_row = (lin / in_group) * kGroupRows;
    const int group_rows = min(v_rows - first_row, kGroupRows);
    const int vr = first_row + (lin % in_group) % group_rows;
    item = vr / row_tiles;
    row0 = (vr - item * row_tiles) * kBM;
    tok0 = ((lin % in_group) / group_rows) * kPPBN;
  };
  // the item's pointers, selected without indexing the argument array
  auto item_ptrs = [&](int item, const uint8_t *&w, const _Float16 *&x, float *&y) {
    w = items.W[0];
    x = items.X[0];
    y = items.Y[0];
#pragma unroll
    for (int i = 1; i < kPPMaxItems; ++i)
      if (item == i) {
        w = items.W[i];
        x = items.X[i];
        y = items.Y[i];
      }
  };

  // group 0: row tid / 2, block tid % 2 of the stage's pair
  const int srow = tid >> 1, sh = tid & 1;
  const uint32_t xlds0 = lds_byte_addr(Xbuf) + 8 * kPPXOps * wave * (kBK * 2);
  int aofs[2], bofs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    aofs[h] = lds_at(64 * wm + (lane & 15), (lane >> 4) + 4 * h);
    bofs[h] = lds_at((kPPBN / 2) * g + 64 * wn + (lane & 15), (lane >> 4) + 4 * h);
  }
  float4_t acc[4][4];

  // Stages [sb, sb + ns) of the tile at (row0, tok0) into acc.
  auto run = [&](const uint8_t *W, const _Float16 *X, int row0, int tok0, int sb, int ns) {
    const uint8_t *rp = W + static_cast<int64_t>(min(row0 + srow, n_rows - 1)) * nb1 +
                        static_cast<int64_t>(sb) * (2 * Block<QT>::bytes);
    const int nb = nblk - 2 * sb;  // blocks from rp on
    const _Float16 *xs0 = X + static_cast<int64_t>(kBK) * sb;
    // group 1: copy i of wavefront w fills LDS rows 8 (8 w + i) .. + 7 of the
    // activation tile; lane p writes position p % 8 of row p / 8, which holds
    // chunk (p % 8) ^ (row % 8) (the lds_at permutation). Token rows past the
    // end re-read the last token.
    uint32_t xoff[kPPXOps];
#pragma unroll
    for (int i = 0; i < kPPXOps; ++i) {
      const int row = 8 * (kPPXOps * wave + i) + (lane >> 3);
      const int c = (lane & 7) ^ (row & 7);
      const int tok = min(tok0 + row, n_tokens - 1);
      xoff[i] = static_cast<uint32_t>((tok * k + 8 * c) * 2);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

    const int last = ns - 1;
    auto load_w = [&](HalfRaw<QT> &r, int st) {
      if constexpr (ALIGN4)
        r = load_half_pair<QT>(rp, st, sh);
      else
        r = load_half_u16<QT>(rp, 2 * st + sh, nb);
    };
    auto store_w = [&](int buf, const HalfRaw<QT> &r) {
      store_half<QT>(Wbuf + buf * kPPWHalves, srow, 4 * sh, r, ALIGN4 && sh == 0);
    };
    auto copy_x = [&](int st) {
      const _Float16 *base = xs0 + static_cast<int64_t>(kBK) * st;
      const uint32_t lds = xlds0 + static_cast<uint32_t>((st % kPPXBufs) * kPPXHalves * 2);
#pragma unroll
      for (int i = 0; i < kPPXOps; ++i) dma16(xoff[i], base, lds + i * 1024);
    };
    // Operands of a stage in registers. A stage's activations are complete in
    // LDS one phase before its weights, and both are complete for group 1 one
    // phase before it computes the stage, so the reads are issued ahead:
    // group 1 reads all operands of stage s during its memory phase, group 0
    // the activations of stage s + 1 during its memory phase and the weights
    // at the start of its compute phase. The MFMAs then wait on LDS latency
    // once per stage at most.
    half8_t pa[2][4], pb[2][4];
    auto read_a = [&](int st) {
      const _Float16 *ws = Wbuf + (st & 1) * kPPWHalves;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) pa[h][i] = *reinterpret_cast<const half8_t *>(ws + aofs[h] + 16 * i * kBK);
    };
    auto read_b = [&](int st) {
      const _Float16 *xs = Xbuf + (st % kPPXBufs) * kPPXHalves;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) pb[h][j] = *reinterpret_cast<const half8_t *>(xs + bofs[h] + 16 * j * kBK);
    };
    auto mfmas = [&] {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[h][i], pb[h][j], acc[i][j], 0, 0, 0);
    };
    auto phase_end = [] {
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    // memory(s), group 0: the activation operands of stage s + 1 (complete
    // since the previous barrier; read first, so their latency passes under
    // the decode rather than at this phase's barrier), the weights of stage
    // s + 1 into buffer (s + 1) % 2 from registers loaded two stages earlier,
    // and the loads of stage s + 3 into those registers (past the last stage
    // they re-read it; what they bring is stored into the idle buffer and
    // never read). Group 1: the operands of stage s (complete since the
    // previous barrier), the copy of stage s + 3's activations and a wait that
    // leaves the copies of stages s + 2 and s + 3 in flight, so stage s + 1's
    // (issued two memory phases earlier) has landed before the barrier.
    HalfRaw<QT> r0, r1;
    auto memory = [&](int s, HalfRaw<QT> &r, int buf) {
      if (g == 0) {
        if (s < last) read_b(s + 1);
        store_w(buf, r);
        load_w(r, min(s + 3, last));
      } else {
        read_a(s);
        read_b(s);
        if (s + 3 <= last) {
          copy_x(s + 3);
          wait_vmcnt<2 * kPPXOps>();
        } else if (s + 2 <= last) {
          wait_vmcnt<kPPXOps>();
        } else {
          wait_vmcnt<0>();
        }
      }
    };
    auto compute = [&](int s) {
      if (g == 0) {
        read_a(s);
        mfmas();
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the reads first
#pragma unroll
        for (int i = 0; i < 32; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // then the MFMAs
      } else {
        mfmas();
      }
    };

    if (g == 0) {
      load_w(r0, 0);
      load_w(r1, min(1, last));
      store_w(0, r0);
      load_w(r0, min(2, last));
    } else {
      copy_x(0);
      if (last >= 1) copy_x(1);
      if (last >= 2) copy_x(2);
      if (last >= 2)
        wait_vmcnt<2 * kPPXOps>();
      else
        wait_vmcnt<0>();
    }
    phase_end();  // stage 0 is in LDS
    if (g == 0) read_b(0);
    // Group 0 runs compute(s), memory(s); group 1 memory(s), compute(s): both
    // pass the same barriers, and each phase pairs one group's MFMAs with the
    // other's staging.
    // The loops run whole pairs of stages (straight-line bodies, so the wait
    // for a register set's loads leaves the other set's loads in flight), then
    // an odd last stage. The last barrier orders every LDS access of the
    // range before whatever the workgroup stores into LDS next.
    int s = 0;
    if (g == 0) {
      for (; s + 1 < ns; s += 2) {
        compute(s);
        phase_end();
        memory(s, r1, 1);
        phase_end();
        compute(s + 1);
        phase_end();
        memory(s + 1, r0, 0);
        phase_end();
      }
      if (s < ns) {
        compute(s);
        phase_end();
        memory(s, r1, 1);
        phase_end();
      }
    } else {
      for (; s + 1 < ns; s += 2) {
        memory(s, r1, 1);
        phase_end();
        compute(s);
        phase_end();
        memory(s + 1, r0, 0);
        phase_end();
        compute(s + 1);
        phase_end();
      }
      if (s < ns) {
        memory(s, r1, 1);
        phase_end();
        compute(s);
        phase_end();
      }
    }
    wait_vmcnt<0>();  // no load outlives the range
  };

  // D element e of lane l in tile (i, j): row 64 wm + 16 i + 4 (l / 16) + e,
  // token 128 g + 64 wn + 16 j + l % 16.
  auto store_y = [&](float *Y, int row0, int tok0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tok = tok0 + (kPPBN / 2) * g + 64 * wn + 16 * j + (lane & 15);
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
  };

  const uint8_t *w;
  const _Float16 *x;
  float *y;
  if constexpr (!SK) {
    int item, row0, tok0;
    coords(static_cast<int>(blockIdx.x), item, row0, tok0);
    item_ptrs(item, w, x, y);
    run(w, x, row0, tok0, 0, n_st);
    store_y(y, row0, tok0);
  } else {
    // workgroups past the whole tiles take part `me` of split tile `t`
    const int b = static_cast<int>(blockIdx.x);
    const bool whole = b < sk.t_whole;
    const int t = whole ? b : (b - sk.t_whole) / sk.parts, me = whole ? 0 : (b - sk.t_whole) % sk.parts;
    const int sb = whole ? 0 : n_st * me / sk.parts, se = whole ? n_st : n_st * (me + 1) / sk.parts;
    int item, row0, tok0;
    coords(whole ? t : sk.t_whole + t, item, row0, tok0);
    item_ptrs(item, w, x, y);
    run(w, x, row0, tok0, sb, se - sb);
    if (whole) {
      store_y(y, row0, tok0);
      return;
    }
    // store the part, count it, and if it completes the count, add the parts
    // (with more than two, its own read back too, so the sum needs no second
    // register tile)
    const float4_t *slots = sk.part + static_cast<int64_t>(t) * sk.parts * (kPPThreads * 16) + threadIdx.x;
    float4_t *mine = sk.part + (static_cast<int64_t>(t) * sk.parts + me) * (kPPThreads * 16) + threadIdx.x;
#pragma unroll
    for (int f = 0; f < 16; ++f) mine[f * kPPThreads] = acc[f / 4][f % 4];
    int *flag = reinterpret_cast<int *>(lds_dynamic);
    __syncthreads();  // every part store is ordered before the count
    if (threadIdx.x == 0) *flag = __hip_atomic_fetch_add(sk.cnt + t, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*flag != sk.parts - 1) return;
    float4_t v[16];
    if (sk.parts == 2) {
      const float4_t *other = slots + static_cast<int64_t>(1 - me) * (kPPThreads * 16);
#pragma unroll
      for (int f = 0; f < 16; ++f) v[f] = other[f * kPPThreads];
#pragma unroll
      for (int f = 0; f < 16; ++f) acc[f / 4][f % 4] += v[f];
    } else {
#pragma unroll
      for (int f = 0; f < 16; ++f) acc[f / 4][f % 4] = slots[f * kPPThreads];
      for (int c = 1; c < sk.parts; ++c) {
        const float4_t *part = slots + static_cast<int64_t>(c) * (kPPThreads * 16);
#pragma unroll
        for (int f = 0; f < 16; ++f) v[f] = part[f * kPPThreads];
#pragma unroll
        for (int f = 0; f < 16; ++f) acc[f / 4][f % 4] += v[f];
      }
    }
    store_y(y, row0, tok0);
    if (threadIdx.x == 0) __hip_atomic_store(sk.cnt + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Expert-routed MUL_MAT_ID with many pairs, on the two-group structure: a
// workgroup takes two tiles of the routing table (tiles 2 p and 2 p + 1, up
// to kPPRTile pairs of one expert each) for one 128-row tile, one tile per
// group. The tile is 160 pairs wide, not 128, because under random top-k
// routing an expert's pair count scatters around its mean: at 512 tokens, 2
// of 8 experts, the counts are about 128 +- 10, and 128-pair tiles would give
// half the experts a second, nearly empty tile that costs a full weight
// decode. Each group has its own weight stage and activation stages in LDS
// (its expert's rows, its pairs' activation rows) and does all of its own
// staging in its memory phase: one block of one row per thread, decoded
// from registers loaded three memory phases ahead, and its activation rows
// copied two stages ahead from an fp16 copy of X (made by the caller's
// conversion kernel, the same rounding the one-group kernel applies)
// straight into LDS, gathered through the pair list. The phases alternate
// as in the dense kernel, so one group's MFMAs run beside the other's
// staging. A group's weight stage is single-buffered: group 0 (compute
// first) stores stage s + 1 in the memory phase after computing stage s,
// group 1 (memory first) stores stage s in the memory phase before
// computing it; either way the phase barrier separates the store from the
// group's own reads. Each output element gets the same MFMAs in the same k
// order as in the one-group routed kernel, so the two agree bit for bit. A
// group whose tile is empty (the second of an odd tile count) runs on
// placeholder entries and stores nothing.
constexpr int kPPRTile = kTileTokensTwoGroup;                     // pairs per tile (10 column blocks)
constexpr int kPPRJ = kPPRTile / 32;                              // column blocks per wavefront (5)
constexpr int kPPRXOps = kPPRTile * kBK * 2 / (kGemmThreads * 16);  // copies per lane per stage (5)
constexpr size_t kPPRoutedLds = (2 * kPPWHalves + 3 * 2 * kPPRTile * kBK) * sizeof(_Float16);  // 152 KiB
static_assert(kPPRTile % 32 == 0 && kPPRXOps * kGemmThreads * 16 == kPPRTile * kBK * 2, "whole copies");
static_assert(kPPRoutedLds <= 160 * 1024, "one workgroup per CU");

template <int QT, bool ALIGN4>
__global__ __launch_bounds__(kPPThreads, 2) void gemm_pp_routed_kernel(const uint8_t *__restrict__ W, int n_rows,
                                                                       int nblk, int64_t nb1,
                                                                       const _Float16 *__restrict__ Xh, int k,
                                                                       float *__restrict__ Y, bool y_vec4,
                                                                       int row_tiles, GemmRoute route,
                                                                       int n_tiles_all) {
  extern __shared__ __attribute__((aligned(16))) _Float16 lds_dynamic[];
  constexpr int kXH = kPPRTile * kBK;  // one group's activation stage
  const int g = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kGemmThreads);
  const int tid = static_cast<int>(threadIdx.x) - g * kGemmThreads;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // LDS: one weight tile per group, then [stage][group] activation tiles (3
  // stages)
  _Float16 *const wt = lds_dynamic + g * kPPWHalves;
  auto xtile = [&](int buf) { return lds_dynamic + 2 * kPPWHalves + (2 * buf + g) * kXH; };

  // Work items are (128-row tile, tile pair) over the tiles the routing
  // kernel made (their number is in every table entry), so no workgroup
  // waits for a dispatch slot only to find its tiles empty. The grid is at
  // most one workgroup per CU; workgroup w takes items v = w, w + grid, ..,
  // in the dense kernels' order (XCD-contiguous runs of v, then groups of
  // kGroupRows row tiles with all tile pairs).
  const int n_wg = static_cast<int>(gridDim.x);
  const int bid = static_cast<int>(blockIdx.x);
  const int per_xcd = n_wg / kXcds;
  const int lin0 = bid < per_xcd * kXcds ? (bid % kXcds) * per_xcd + bid / kXcds : bid;
  const int n_tiles = min(n_tiles_all, __builtin_amdgcn_readfirstlane(route.tiles[3]));
  const int pair_tiles = (n_tiles + 1) / 2;
  const int n_items = row_tiles * pair_tiles;
  const int in_group = kGroupRows * pair_tiles;
  for (int lin = lin0; lin < n_items; lin += n_wg) {
  const int first_row = (lin / in_group) * kGroupRows;
  const int group_rows = min(row_tiles - first_row, kGroupRows);
  const int row0 = (first_row + (lin % in_group) % group_rows) * kBM;
  const int tp = (lin % in_group) / group_rows;

  // the two tiles; the second of an odd count reads as empty
  int e2[2], f2[2], c2[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 2 * tp + h;
    const bool in = t < n_tiles;
    e2[h] = in ? __builtin_amdgcn_readfirstlane(route.tiles[4 * t]) : 0;
    f2[h] = in ? __builtin_amdgcn_readfirstlane(route.tiles[4 * t + 1]) : 0;
    c2[h] = in ? __builtin_amdgcn_readfirstlane(route.tiles[4 * t + 2]) : 0;
  }
  const int e = g ? e2[1] : e2[0], first = g ? f2[1] : f2[0], cnt = g ? c2[1] : c2[0];

  // weights of this group's expert: row tid / 2, block tid % 2 of the pair
  const int srow = tid >> 1, sh = tid & 1;
  const uint8_t *rp = W + static_cast<int64_t>(e) * route.nb2 + static_cast<int64_t>(min(row0 + srow, n_rows - 1)) * nb1;
  // activations: copy i of wavefront w fills LDS rows 8 (kPPRXOps w + i) ..
  // + 7 of the group's tile (token slots); lane p writes position p % 8 of
  // row p / 8, which holds chunk (p % 8) ^ (row % 8) (the lds_at
  // permutation); slots past the tile's count repeat its last pair
  const _Float16 *xsrc[kPPRXOps];
#pragma unroll
  for (int i = 0; i < kPPRXOps; ++i) {
    const int slot = 8 * (kPPRXOps * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ (slot & 7);
    const int p = route.list[first + min(slot, max(cnt, 1) - 1)];
    const int t = p / route.n_ids;
    const int64_t xr = static_cast<int64_t>(t) * route.x_slots + (route.x_slots > 1 ? p - t * route.n_ids : 0);
    xsrc[i] = Xh + xr * k + 8 * c;
  }
  const uint32_t xdst0 = lds_byte_addr(xtile(0)) + 8 * kPPRXOps * wave * (kBK * 2);

  float4_t acc[4][kPPRJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kPPRJ; ++j) acc[i][j] = float4_t{0.f, 0.f, 0.f, 0.f};

  const int n_st = nblk / 2;
  const int last = n_st - 1;
  auto load_w = [&](HalfRaw<QT> &r, int st) {
    if constexpr (ALIGN4)
      r = load_half_pair<QT>(rp, st, sh);
    else
      r = load_half_u16<QT>(rp, 2 * st + sh, nblk);
  };
  auto store_w = [&](const HalfRaw<QT> &r) { store_half<QT>(wt, srow, 4 * sh, r, ALIGN4 && sh == 0); };
  // the copy of stage st into activation buffer b % 3
  auto copy_x = [&](int st, int b) {
    const uint32_t dst = xdst0 + static_cast<uint32_t>((b % 3) * 2 * kXH * 2);
#pragma unroll
    for (int i = 0; i < kPPRXOps; ++i) dma16(xsrc[i] + kBK * st, dst + i * 1024);
  };
  // wavefront (wm, wn): rows 64 wm .. + 63 of the tile, token column blocks
  // wn, wn + 2, .., so a partly filled tile splits its columns evenly
  int aofs[2], bofs[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    aofs[h] = lds_at(64 * wm + (lane & 15), (lane >> 4) + 4 * h);
    bofs[h] = lds_at(16 * wn + (lane & 15), (lane >> 4) + 4 * h);
  }
  // Column blocks of this wavefront that hold pairs (wave-uniform): the
  // MFMAs of the last two run only when their block is in use, so a tile
  // of 128 pairs costs what it did on 128-pair tiles. Skipped blocks hold
  // no pair, and nothing of theirs is stored.
  const int nj = min(kPPRJ, max(0, (cnt - 16 * wn + 31) / 32));
  static_assert(kPPRJ == 5, "three unconditional column blocks, two conditional");
  auto compute = [&](int s) {
    const _Float16 *xs = xtile(s % 3);
    half8_t a[2][4], b[2][kPPRJ];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[h][i] = *reinterpret_cast<const half8_t *>(wt + aofs[h] + 16 * i * kBK);
#pragma unroll
      for (int j = 0; j < kPPRJ; ++j) b[h][j] = *reinterpret_cast<const half8_t *>(xs + bofs[h] + 32 * j * kBK);
    }
    auto block = [&](int j) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[h][i], b[h][j], acc[i][j], 0, 0, 0);
    };
    block(0);
    block(1);
    block(2);
#pragma unroll
    for (int i = 0; i < 8 + 2 * kPPRJ; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the reads first
#pragma unroll
    for (int i = 0; i < 24; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // then the MFMAs
    if (nj > 3) block(3);
    if (nj > 4) block(4);
  };
  auto phase_end = [] {
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  // memory(s, r): the weights in r into the group's weight tile (stage s + 1
  // for group 0, stage s for group 1), the copy of stage s + 2, then a wait
  // that leaves only that copy and the weight loads issued after stage
  // s + 1's copy in flight (so stage s + 1's copy, issued one memory phase
  // earlier, has landed before the barrier; the weight loads are counted as
  // two operations, at most their number, so the wait is at worst stricter),
  // then the weight loads of the stage stored three memory phases later
  // (s + 4 for group 0, s + 3 for group 1). The weights come from HBM, each
  // expert's rows being read by one or two workgroups, hence three register
  // sets. Past the last stage copies and loads re-read it into the free
  // buffer and the registers; nothing reads them.
  const int ahead = g == 0 ? 4 : 3;
  HalfRaw<QT> r0, r1, r2;
  auto memory = [&](int s, HalfRaw<QT> &r) {
    store_w(r);
    copy_x(min(s + 2, last), s + 2);
    wait_vmcnt<kPPRXOps + 2>();
    load_w(r, min(s + ahead, last));
  };

  // prologue: copies of stages 0 and 1, weights of stages 0 to 2; group 0
  // stores stage 0 (the wait for its weight registers covers its copy,
  // issued before them), waits for stage 0's copy and loads stage 3 into the
  // freed registers
  copy_x(0, 0);
  load_w(r0, 0);
  copy_x(min(1, last), 1);
  load_w(r1, min(1, last));
  load_w(r2, min(2, last));
  if (g == 0) {
    store_w(r0);
    wait_vmcnt<kPPRXOps + 4>();  // stage 0's copy has landed (stage 1's copy and two weight sets may not)
    load_w(r0, min(3, last));
  }
  phase_end();  // group 0's stage 0 is in LDS
  // Whole triples of stages (straight-line bodies, so the wait for one
  // register set leaves the others' loads in flight), then up to two.
  int s = 0;
  if (g == 0) {
    for (; s + 2 < n_st; s += 3) {
      compute(s);
      phase_end();
      memory(s, r1);
      phase_end();
      compute(s + 1);
      phase_end();
      memory(s + 1, r2);
      phase_end();
      compute(s + 2);
      phase_end();
      memory(s + 2, r0);
      phase_end();
    }
    if (s < n_st) {
      compute(s);
      phase_end();
      memory(s, r1);
      phase_end();
    }
    if (s + 1 < n_st) {
      compute(s + 1);
      phase_end();
      memory(s + 1, r2);
      phase_end();
    }
  } else {
    for (; s + 2 < n_st; s += 3) {
      memory(s, r0);
      phase_end();
      compute(s);
      phase_end();
      memory(s + 1, r1);
      phase_end();
      compute(s + 1);
      phase_end();
      memory(s + 2, r2);
      phase_end();
      compute(s + 2);
      phase_end();
    }
    if (s < n_st) {
      memory(s, r0);
      phase_end();
      compute(s);
      phase_end();
    }
    if (s + 1 < n_st) {
      memory(s + 1, r1);
      phase_end();
      compute(s + 1);
      phase_end();
    }
  }
  wait_vmcnt<0>();  // no copy outlives the workgroup

  // D element e of lane l in tile (i, j): row 64 wm + 16 i + 4 (l / 16) + e,
  // token slot 16 (2 j + wn) + l % 16 of this group's tile
#pragma unroll
  for (int j = 0; j < kPPRJ; ++j) {
    const int slot = 16 * (2 * j + wn) + (lane & 15);
    if (slot >= cnt) continue;
    float *yrow = Y + static_cast<int64_t>(route.list[first + slot]) * n_rows;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + 64 * wm + 16 * i + 4 * (lane >> 4);
      if (y_vec4 && r + 3 < n_rows) {
        *reinterpret_cast<float4_t *>(yrow + r) = acc[i][j];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (r + q < n_rows) yrow[r + q] = acc[i][j][q];
      }
    }
  }
  }  // work items (the last phase barrier has ordered every LDS read before the next item's stores)
}

template <int QT, bool XF16, int BM, int KS = 1>
static hipError_t gemm_dispatch(bool align4, dim3 grid, hipStream_t s, const uint8_t *w, int n_rows, int nblk,
                                int64_t nb1, const void *X, int n_tokens, int k, float *Y, bool y_vec4, int row_tiles) {
  const GemmRoute none{nullptr, nullptr, 0, 0, 0};
  // KS = 2: each k group's two stages of weights and activations in dynamic LDS
  const size_t lds = KS == 1 ? 0 : static_cast<size_t>(KS) * 2 * (BM + kBN) * kBK * sizeof(_Float16);
  const dim3 block(kGemmThreads * KS);
  if (align4)
    return launch(gemm_kernel<QT, XF16, true, false, BM, KS>, grid, block, lds, s, w, n_rows, nblk, nb1, X, n_tokens,
                  k, Y, y_vec4, row_tiles, none);
  return launch(gemm_kernel<QT, XF16, false, false, BM, KS>, grid, block, lds, s, w, n_rows, nblk, nb1, X, n_tokens, k,
                Y, y_vec4, row_tiles, none);
}

bool routed_two_group(int qtype, int64_t k, int64_t n_rows, int64_t max_tiles, int64_t cus) {
  const int64_t row_tiles = (n_rows + kBM - 1) / kBM;
  return qtype != QMM_TYPE_Q4_K && cus > 0 && row_tiles * ((max_tiles + 1) / 2) >= cus && (k / 32) % 2 == 0;
}

hipError_t launch_gemm_routed(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, int64_t nb2,
                              const float *X, const _Float16 *Xh, int64_t x_slots, int64_t n_ids,
                              const int32_t *list, const int32_t *tiles, int64_t max_tiles, float *Y,
                              hipStream_t stream) {
  const uint8_t *w = static_cast<const uint8_t *>(W);
  const bool align4 = (reinterpret_cast<uintptr_t>(W) % 4 == 0) && (nb1 % 4 == 0) && (nb2 % 4 == 0);
  const bool y_vec4 = (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && (n_rows % 4 == 0);
  const int64_t row_tiles = (n_rows + kBM - 1) / kBM;
  if (row_tiles * max_tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(row_tiles * max_tiles));
  const GemmRoute route{list, tiles, nb2, static_cast<int>(n_ids), static_cast<int>(x_slots)};
  const int rt = static_cast<int>(row_tiles), nblk = static_cast<int>(k / 32), nr = static_cast<int>(n_rows),
            kk = static_cast<int>(k);
  // With the fp16 copy of X (Xh), the caller has routed into the two-group
  // kernel's tiles (routed_two_group held): two tiles per workgroup.
  const int64_t pairs_of_tiles = (max_tiles + 1) / 2;
  if (Xh != nullptr) {
    const int64_t cus = device_cus();
    const int64_t items = row_tiles * pairs_of_tiles;  // the host's bound; the kernel reads the actual count
    const dim3 pgrid(static_cast<unsigned>(cus > 0 && cus < items ? cus : items));
    const int nt_all = static_cast<int>(max_tiles);
    return by_qtype(qtype, [&](auto qt) {
      constexpr int QT = decltype(qt)::value;
      auto go = [&](auto kern) {
        return launch(kern, pgrid, dim3(kPPThreads), kPPRoutedLds, stream, w, nr, nblk, nb1, Xh, kk, Y, y_vec4, rt,
                      route, nt_all);
      };
      return align4 ? go(gemm_pp_routed_kernel<QT, true>) : go(gemm_pp_routed_kernel<QT, false>);
    });
  }
  const dim3 block(kGemmThreads);
  return by_qtype_k(qtype, [&](auto qt) {
    constexpr int QT = decltype(qt)::value;
    return align4 ? launch(gemm_kernel<QT, false, true, true>, grid, block, 0, stream, w, nr, nblk, nb1,
                           static_cast<const void *>(X), 0, kk, Y, y_vec4, rt, route)
                  : launch(gemm_kernel<QT, false, false, true>, grid, block, 0, stream, w, nr, nblk, nb1,
                           static_cast<const void *>(X), 0, kk, Y, y_vec4, rt, route);
  });
}

hipError_t launch_gemm(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const void *X, bool x_f16,
                       int64_t n_tokens, float *Y, hipStream_t stream) {
  const uint8_t *w = static_cast<const uint8_t *>(W);
  const bool align4 = (reinterpret_cast<uintptr_t>(W) % 4 == 0) && (nb1 % 4 == 0);
  const bool y_vec4 = (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && (n_rows % 4 == 0);
  const int64_t tok_tiles = (n_tokens + kBN - 1) / kBN;
  // With 128-row tiles, a launch of no more tiles than CUs leaves CUs idle
  // (two tiles share a CU); 64-row tiles double the workgroups (measured:
  // +28 % on 4096 rows x 512 tokens, -3 % at 1.3 tiles per CU).
  const int64_t cus = device_cus();
  const bool small = cus > 0 && ((n_rows + kBM - 1) / kBM) * tok_tiles <= cus;
  const int bm = small ? kBM / 2 : kBM;
  const int64_t row_tiles = (n_rows + bm - 1) / bm;
  if (row_tiles * tok_tiles > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(row_tiles * tok_tiles));
  const int rt = static_cast<int>(row_tiles);
  const int nblk = static_cast<int>(k / 32), nr = static_cast<int>(n_rows), nt = static_cast<int>(n_tokens),
            kk = static_cast<int>(k);
  // Small launches whose block count splits into two equal halves of whole
  // stages also split k inside the workgroup (two wavefronts per SIMD).
  const bool ksplit = small && nblk % 4 == 0;
  // fp16 activations, 128 x 256 tiles for at least 2/3 of the CUs (one
  // round) or in rounds that keep at least 3/4 of the CUs busy, whole stages,
  // and activations whose byte offsets fit 32 bits: the ping-pong kernel.
  // (One round on 172 of 256 CUs still beats the one-group kernel on all of
  // them: 11008 x 4096 at 512 tokens 78.7 -> 65.0 us, 14336 x 4096 80.9 ->
  // 64.5 us. Q4_K, whose fp32 decode is the longest, takes it too: 4096 x
  // 4096 at 2048 tokens 105-115 -> 86 us, 11008 x 4096 306 -> 257 us.)
  const int64_t pp_tiles = ((n_rows + kBM - 1) / kBM) * ((n_tokens + kPPBN - 1) / kPPBN);
  const int64_t pp_rounds = cus > 0 ? (pp_tiles + cus - 1) / cus : 0;
  const bool pp = x_f16 && cus > 0 && 3 * pp_tiles >= 2 * cus &&
                  (pp_tiles < cus || 4 * pp_tiles >= 3 * pp_rounds * cus) && nblk % 2 == 0 &&
                  pp_tiles <= 0x7FFFFFFF && n_tokens * k * 2 < (int64_t{1} << 32);
  if (pp) {
    const dim3 ppgrid(static_cast<unsigned>(pp_tiles));
    const int prt = static_cast<int>((n_rows + kBM - 1) / kBM);
    const _Float16 *xh = static_cast<const _Float16 *>(X);
    return by_qtype_k(qtype, [&](auto qt) {
      constexpr int QT = decltype(qt)::value;
      const PPItems one{{w}, {xh}, {Y}, 1};
      auto go = [&](auto kern) {
        return launch(kern, ppgrid, dim3(kPPThreads), kPPLds, stream, one, nr, nblk, nb1, nt, kk, y_vec4, prt,
                      PPSplit{});
      };
      return align4 ? go(gemm_pp_kernel<QT, true, false>) : go(gemm_pp_kernel<QT, false, false>);
    });
  }
  return by_qtype_k(qtype, [&](auto qt) {
    constexpr int QT = decltype(qt)::value;
    if (ksplit) {
      if (x_f16)
        return gemm_dispatch<QT, true, kBM / 2, 2>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
      return gemm_dispatch<QT, false, kBM / 2, 2>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
    }
    if (small) {
      if (x_f16) return gemm_dispatch<QT, true, kBM / 2>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
      return gemm_dispatch<QT, false, kBM / 2>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
    }
    if (x_f16) return gemm_dispatch<QT, true, kBM>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
    return gemm_dispatch<QT, false, kBM>(align4, grid, stream, w, nr, nblk, nb1, X, nt, kk, Y, y_vec4, rt);
  });
}

// The split form of the two-group kernel (PPSplit): fp16 activations, a
// 32-weight block type, whole stages. Two plans:
//  * few tiles with long k (at most half as many 128 x 256 tiles as CUs):
//    each tile is split into P = min(4, CUs / tiles) parts of equal stage
//    ranges (one workgroup each, P * tiles workgroups), each at least
//    kPPMinUnits stages. Measured on the MI355X, a part costs its 128 KiB
//    partial tile twice (stored, then read by the workgroup that adds), and
//    with every CU storing at once that traffic takes several microseconds:
//    more tiles or shorter k (4096 x 4096 or 11008 x 4096 at 512 tokens)
//    ran slower split than whole, few tiles with long k (4096 x 14336 at 512
//    tokens, 4096 x 4096 at 1024) faster.
//  * more tiles than CUs whose last round would fill at most half of the
//    CUs: the tiles of whole rounds run whole, the last round's tiles in two
//    parts each (t_whole whole tiles, then 2 * tail workgroups), so the last
//    round takes about half the time. A last round fuller than half gains
//    nothing from two parts (they would need two rounds), and a stream-K
//    remainder spread over all CUs measured slower (its ranges cross tiles).
constexpr int kPPMinUnits = 32;
constexpr int kPPMaxParts = 4;
constexpr int64_t kPPPartBytes = int64_t{kPPThreads} * 16 * sizeof(float4_t);  // one partial tile (128 KiB)

struct PPPlan {
  PPSplit sk{};
  int64_t bytes = 0;  // workspace: t_sk counters (256-byte padded), then the partial tiles; 0: no split
};

static PPPlan pp_split_plan(int qtype, int64_t n_items, int64_t n_rows, int64_t k, int64_t n_tokens, bool x_f16) {
  PPPlan p;
  const int64_t cus = device_cus();
  const int64_t nblk = k / 32;
  if (!x_f16 || qtype == QMM_TYPE_Q4_K || cus <= 0 || n_rows <= 0 || n_items < 1 || n_items > kPPMaxItems ||
      nblk % 2 != 0 || n_tokens < kPPBN || n_tokens * k * 2 >= (int64_t{1} << 32))
    return p;
  const int64_t T = n_items * ((n_rows + kBM - 1) / kBM) * ((n_tokens + kPPBN - 1) / kPPBN);
  const int64_t n_st = nblk / 2;
  int64_t t_whole = 0, t_sk = 0, parts = 0;
  if (2 * T <= cus) {
    t_sk = T;
    parts = std::min<int64_t>(kPPMaxParts, cus / T);
    if (n_st < parts * kPPMinUnits) return p;
  } else {
    const int64_t tail = T % cus, rounds = (T + cus - 1) / cus;
    // the whole rounds must be ones the two-group kernel takes (launch_gemm's rule)
    if (T <= cus || tail == 0 || 2 * tail > cus || n_st < 2 * kPPMinUnits || 4 * T < 3 * rounds * cus) return p;
    t_whole = T - tail;
    t_sk = tail;
    parts = 2;
  }
  const int64_t groups = t_whole + t_sk * parts;
  if (groups > 0x7FFFFFFF || (t_sk * n_st + 1) * t_sk * parts > 0x7FFFFFFF) return p;
  p.sk = PPSplit{static_cast<int>(t_sk), static_cast<int>(groups), static_cast<int>(parts), nullptr, nullptr,
                 static_cast<int>(t_whole)};
  p.bytes = (t_sk * 4 + 255) / 256 * 256 + t_sk * parts * kPPPartBytes;
  return p;
}

int64_t gemm_split_bytes(int qtype, int64_t n_rows, int64_t k, int64_t n_tokens, bool x_f16) {
  return pp_split_plan(qtype, 1, n_rows, k, n_tokens, x_f16).bytes;
}

int64_t gemm_items_split_bytes(int qtype, int n_items, int64_t n_rows, int64_t k, int64_t n_tokens) {
  return pp_split_plan(qtype, n_items, n_rows, k, n_tokens, true).bytes;
}

bool gemm_items_merge(int qtype, int n_items, int64_t n_rows, int64_t k, int64_t n_tokens) {
  if (n_items < 2 || n_items > kPPMaxItems || n_rows <= 0 || n_tokens <= 0) return false;
  if (pp_split_plan(qtype, n_items, n_rows, k, n_tokens, true).bytes > 0) return true;
  // whole tiles only: the two-group kernel's rule on the launch's tiles
  const int64_t cus = device_cus(), nblk = k / 32;
  const int64_t T = n_items * ((n_rows + kBM - 1) / kBM) * ((n_tokens + kPPBN - 1) / kPPBN);
  const int64_t rounds = cus > 0 ? (T + cus - 1) / cus : 0;
  return cus > 0 && 3 * T >= 2 * cus && (T < cus || 4 * T >= 3 * rounds * cus) && nblk % 2 == 0 &&
         T <= 0x7FFFFFFF && n_tokens * k * 2 < (int64_t{1} << 32);
}

hipError_t launch_gemm_items(const void *const *W, int qtype, int n_items, int64_t n_rows, int64_t k, int64_t nb1,
                             const _Float16 *const *X, int64_t n_tokens, float *const *Y, void *workspace,
                             int64_t workspace_bytes, hipStream_t stream) {
  if (n_items < 1 || n_items > kPPMaxItems) return hipErrorInvalidValue;
  PPPlan p = pp_split_plan(qtype, n_items, n_rows, k, n_tokens, true);
  const bool split = p.bytes > 0 && workspace != nullptr && workspace_bytes >= p.bytes;
  PPItems items{};
  bool align4 = nb1 % 4 == 0, y_vec4 = n_rows % 4 == 0;
  for (int i = 0; i < n_items; ++i) {
    items.W[i] = static_cast<const uint8_t *>(W[i]);
    items.X[i] = X[i];
    items.Y[i] = Y[i];
    align4 = align4 && reinterpret_cast<uintptr_t>(W[i]) % 4 == 0;
    y_vec4 = y_vec4 && reinterpret_cast<uintptr_t>(Y[i]) % 16 == 0;
  }
  items.n = n_items;
  const int64_t T = n_items * ((n_rows + kBM - 1) / kBM) * ((n_tokens + kPPBN - 1) / kPPBN);
  if (T > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (split) {
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    p.sk.cnt = reinterpret_cast<int *>(ws);
    p.sk.part = reinterpret_cast<float4_t *>(ws + (static_cast<int64_t>(p.sk.t_sk) * 4 + 255) / 256 * 256);
  }
  const int prt = static_cast<int>((n_rows + kBM - 1) / kBM);
  const int nblk = static_cast<int>(k / 32), nr = static_cast<int>(n_rows), nt = static_cast<int>(n_tokens),
            kk = static_cast<int>(k);
  const dim3 grid(static_cast<unsigned>(split ? p.sk.g_sk : T));
  return by_qtype_k(qtype, [&](auto qt) {
    constexpr int QT = decltype(qt)::value;
    auto go = [&](auto kern, const PPSplit &sk) {
      return launch(kern, grid, dim3(kPPThreads), kPPLds, stream, items, nr, nblk, nb1, nt, kk, y_vec4, prt, sk);
    };
    if constexpr (QT != QMM_TYPE_Q4_K) {
      if (split)
        return align4 ? go(gemm_pp_kernel<QT, true, true>, p.sk) : go(gemm_pp_kernel<QT, false, true>, p.sk);
    }
    return align4 ? go(gemm_pp_kernel<QT, true, false>, PPSplit{}) : go(gemm_pp_kernel<QT, false, false>, PPSplit{});
  });
}

hipError_t launch_gemm_split(const void *W, int qtype, int64_t n_rows, int64_t k, int64_t nb1, const _Float16 *X,
                             int64_t n_tokens, float *Y, void *workspace, int64_t workspace_bytes,
                             hipStream_t stream) {
  const PPPlan p = pp_split_plan(qtype, 1, n_rows, k, n_tokens, true);
  if (p.bytes == 0 || workspace == nullptr || workspace_bytes < p.bytes) return hipErrorInvalidValue;
  const void *w[1] = {W};
  const _Float16 *x[1] = {X};
  float *y[1] = {Y};
  return launch_gemm_items(w, qtype, 1, n_rows, k, nb1, x, n_tokens, y, workspace, workspace_bytes, stream);
}

}  // namespace qmm
