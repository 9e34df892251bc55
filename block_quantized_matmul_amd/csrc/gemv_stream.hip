// Streaming decode MUL_MAT (1 <= n_tokens <= 8) for 16-byte-aligned layouts,
// one or several independent matrices per launch.
//
// What is computed: as in gemv.hip, y[t][r] = sum_b d_rb * sum_i (q - z) x[t][32 b + i]
// ([Bind] "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section 2.3; [Arch]
// "llama.cpp 源码完全拆解(一)：整体架构与模块全景", section "权重装载：GGUF、mmap
// 与 4 bit 块"), with the exact-code MFMA formulation and per-block fp32 scale
// of gemv_common.h.
//
// Design (MI355X, gfx950): the kernel is an HBM stream, so its structure
// copies that of a plain streaming read as closely as it can.
//  * A workgroup owns one 16-row group of one matrix; a launch's grid is
//    (row groups of its largest matrix) x (matrices), and the hardware
//    balances the workgroups across the CUs. Its 8 or 16 wavefronts (see
//    k_split_for) split k into
//    contiguous ranges of quads (8 blocks: 144 bytes Q4_0, 160 Q4_1, 176
//    Q5_0, 192 Q5_1, 272 Q8_0 per row, a whole number of 16-byte chunks) and
//    stream them
//    independently; they meet once, at the end, to add their partial sums in
//    a fixed order through LDS (no atomics: results are reproducible, and
//    identical to the general kernel's, which splits k the same way).
//  * A stage (one quad for all 16 rows) is fetched with fully coalesced
//    16-byte loads (consecutive lanes take consecutive chunks of a row)
//    together with the activation slice of the same 8 blocks, all into one
//    register set. A wavefront issues the loads of a round of stages at once
//    and then consumes them in order (the wait counter is exact).
//  * Consuming a stage copies it into the wavefront's private LDS area (the
//    activations converted to fp16 in MFMA operand order) and runs 8 MFMAs
//    (16 for Q4_1 and Q5_1, whose second MFMA per block sums the activations
//    for the minimum term).
// Several matrices per launch remove the fixed per-launch cost that
// dominates decode-sized matmuls (a launch plus its ramp costs about as much
// as streaming ten megabytes).
#include "common.h"
#include "gemv_common.h"
#include "launch.h"

#include <stddef.h>

#include <type_traits>

namespace qmm {

constexpr int kRMaxMats = 16;

template <int QT, int NT, int G = 1> struct RCfg {
  // 16-byte chunks per row per quad of 8 blocks (144, 160 or 272 bytes)
  static constexpr int quad_chunks = Block<QT>::bytes / 2;
  // LDS bytes per row of the stage copy. Unpadded (chunk c at 16 c, one
  // 16-byte store per chunk) for up to 2 tokens. With 4 or 8 tokens, whose
  // activation traffic makes LDS the tighter resource, rows are padded by 8
  // bytes (stride 38 or 70 dwords): the per-row dword reads of a half
  // wavefront then fall in distinct banks (at 36 or 68 they conflict 2-way on
  // gfx950), at the price of two 8-byte stores per chunk.
  static constexpr int row_stride = quad_chunks * 16 + (NT >= 4 ? 8 : 0);
  static constexpr int w_loads = (16 * G * quad_chunks + 63) / 64;   // loads per lane for the 16 G rows
  // stages per round, sized so a round's registers stay near 64 VGPRs (the
  // kernel then fits 4 wavefronts per SIMD, i.e. 2 workgroups per CU)
  static constexpr int stage_vgprs = 4 * w_loads + NT * 4;
  static constexpr int depth = (64 / stage_vgprs) < 1 ? 1 : (64 / stage_vgprs > 6 ? 6 : 64 / stage_vgprs);
  // With 8 wavefronts per workgroup (launches larger than the GPU), the
  // nibble types with one or two tokens take rounds of 2 stages (the whole
  // share for k = 4096) so the kernel fits in ~60 VGPRs and 6-8 wavefronts
  // per SIMD: more workgroups per CU overlap one another's loads and
  // compute. Q5_1, whose decode needs more registers, takes 6 wavefronts per
  // SIMD (~85 VGPRs; 4.5 % faster than 4 on 11008 x 4096, and 8 spill).
  // Q4_K fits too (62 VGPRs at one token): 11008 x 4096 10.0 -> 8.95 us,
  // 32000 x 4096 22.4 -> 19.6 us against rounds of 4 stages at 4 per SIMD.
  static constexpr bool mid = QTraits<QT>::has_qh && QTraits<QT>::has_min && NT <= 2;
  static constexpr bool lean = QTraits<QT>::nibbles && !mid && NT <= 2;
  // Q8_0 at one or two tokens (74-80 VGPRs) runs 6 wavefronts per SIMD:
  // 32000 x 4096 at 2 tokens 30.3 -> 28.5 us; one token unchanged.
  static constexpr bool q8 = !QTraits<QT>::nibbles && NT <= 2;
  static constexpr int depth_large = (lean || mid) ? 2 : depth;
  static constexpr int w_lds = 16 * G * row_stride;
  static constexpr int x_lds = 8 * 4 * NT * 16;                      // 8 blocks x 4 lane groups x NT slots x 8 halves
  static constexpr int lds_per_wave = w_lds + x_lds;
  // With several row groups per workgroup the stage copies make LDS the
  // occupancy limit (one or two workgroups of 8 wavefronts per CU), so the
  // register budget follows from it instead of the single-group tuning.
  static constexpr int lds_wg_large = kKSplitLarge * (lds_per_wave + G * 32 * 4 * 4);
  static constexpr int wgs_per_cu_large = (160 * 1024) / lds_wg_large;
  static constexpr int waves_per_simd_large =
      G > 1 ? (2 * wgs_per_cu_large < 4 ? 2 * wgs_per_cu_large : 4) : lean ? (NT == 1 ? 8 : 6) : mid || q8 ? 6 : 4;
};

// One matrix of a launch: 64 bytes, so a workgroup fetches all of it with a
// single 16-dword scalar load and one wait (field by field, the compiler
// places each scalar load next to its use, which serialises several memory
// round trips before the first weight load can be issued).
struct RMat {
  const uint8_t *W;
  const void *X;
  float *Y;
  int64_t nb1;
  int n_rows, nblk, n_tokens, k;
  int pad[4];
};
static_assert(sizeof(RMat) == 64, "one scalar load per matrix record");

// Descriptor table of a launch. Workgroup (x, y) takes row group x of matrix
// y; the grid is as wide as the largest matrix, and workgroups past a smaller
// matrix's last row group return at once.
struct RBatch {
  RMat m[kRMaxMats];
};

typedef uint32_t u32x16_t __attribute__((ext_vector_type(16)));
template <class T> using GPtr = const __attribute__((address_space(1))) T *;
// A record is read through the kernel-argument segment pointer as one vector
// (indexing the by-value parameter with a run-time index would copy the whole
// table to scratch).
typedef const __attribute__((address_space(4))) u32x16_t *KRec;
// Byte offset of the table in the kernel-argument segment: it follows
// matrix 0's eight scalar arguments (48 bytes) and two 8-byte pads.
constexpr int kRTableOffset = 64;

// Routing record of an expert-routed launch (MUL_MAT_ID), in the table's
// second slot: pair p = pair0 + blockIdx.y is (token p / n_ids, slot
// p % n_ids); its matrix is expert ids[p] of the stack (expert stride nb2),
// its activation row X[token][slot] (X[token][0] when x_slots == 1), its
// output Y[p].
// The tile form (decode-sized MUL_MAT_ID with pairs grouped by expert):
// grid row y is tile pair0 + y of `tiles` = (expert, first entry, count) of
// the pair list `ids`, and the workgroup runs the count (<= NT) pairs of the
// tile as token slots; X is read through one buffer of x_bytes bytes.
struct RRoute {
  const int32_t *ids;
  int64_t nb2;
  int n_experts, n_ids, x_slots, pair0;
  const int32_t *tiles;
  uint32_t x_bytes;
  int pad[5];
};
static_assert(sizeof(RRoute) == 64, "one table slot");
// Fourth word of a buffer resource: 32-bit data format, no swizzle.
constexpr int kRsrcWord3 = 0x00020000;

template <int QT, int NT, bool XF16, int G = 1> struct RRegs {
  u32x4_t w[RCfg<QT, NT, G>::w_loads];
  typename std::conditional<XF16, half4_t, float4_t>::type x[NT];
};

// Lane-constant placement of a stage. Weight chunk c = 64 j + lane of the 16
// rows is row c / QC, chunk c % QC of that row: byte (c / QC) nb1 + 16 (c % QC)
// of the row group, and byte (c / QC) row_stride + 16 (c % QC) of the
// wavefront's LDS copy; chunks past 16 * QC re-read chunk 0 and are not stored
// (woff < 0). The activation piece of a lane is block lane / 8 of the quad,
// elements 4 (lane % 8) .. +3, staged at LDS byte xw (token slot 0).
template <int QT, int NT, int G = 1> struct RLane {
  int woff[RCfg<QT, NT, G>::w_loads];
  uint32_t wv[RCfg<QT, NT, G>::w_loads];
  int xw;

  __device__ __forceinline__ RLane(int lane, uint32_t nb1) {
    constexpr int QC = RCfg<QT, NT, G>::quad_chunks;
#pragma unroll
    for (int j = 0; j < RCfg<QT, NT, G>::w_loads; ++j) {
      const int c = 64 * j + lane;
      const bool ok = c < 16 * G * QC;
      const uint32_t r = static_cast<uint32_t>(c) / QC;
      woff[j] = ok ? static_cast<int>(r) * RCfg<QT, NT, G>::row_stride + 16 * (c - QC * static_cast<int>(r)) : -1;
      // r nb1 + 16 (c - QC r) with one 24-bit multiply-add (nb1 < 2^24)
      wv[j] = ok ? __umul24(r, nb1 - 16 * QC) + 16 * c : 0;
    }
    const int xb = lane >> 3, xj = lane & 7;
    // element order of a lane group: Q4_0's nibble order for the 32-weight
    // nibble types, contiguous (8 g .. 8 g + 7) for Q8_0 and Q4_K
    constexpr bool nib = QTraits<QT>::nibbles && !QTraits<QT>::kquant;
    const int xg = nib ? (xj & 3) : (xj >> 1);
    const int xh = nib ? 4 * (xj >> 2) : 4 * (xj & 1);
    xw = (4 * xb + xg) * NT * 16 + 2 * xh;
  }
};

// A stage's weight chunks into the wavefront's LDS area (wl), rows
// row_stride bytes apart.
template <int QT, int NT, int G>
__device__ __forceinline__ void r_copy_w(const u32x4_t (&w)[RCfg<QT, NT, G>::w_loads], const RLane<QT, NT, G> &L,
                                         unsigned char *wl) {
  using C = RCfg<QT, NT, G>;
#pragma unroll
  for (int j = 0; j < C::w_loads; ++j)
    if (L.woff[j] >= 0) {
      if constexpr (C::row_stride % 16 == 0) {
        *reinterpret_cast<u32x4_t *>(wl + L.woff[j]) = w[j];
      } else {
        *reinterpret_cast<u32x2_t *>(wl + L.woff[j]) = u32x2_t{w[j].x, w[j].y};
        *reinterpret_cast<u32x2_t *>(wl + L.woff[j] + 8) = u32x2_t{w[j].z, w[j].w};
      }
    }
}

// Four activations (elements 4 l .. 4 l + 3 of a quad, l the lane's piece)
// of one token slot, as fp16 in MFMA operand order, into the staged set xs
// at byte xw + 16 t.
template <bool XF16>
__device__ __forceinline__ void r_stage_x(const typename std::conditional<XF16, half4_t, float4_t>::type &x,
                                          half8_t *xs, int xw, int t) {
  half4_t h;
  if constexpr (XF16) {
    h = x;
  } else {
    const half2_t a = cvt_half2(x.x, x.y), b = cvt_half2(x.z, x.w);
    h = half4_t{a.x, a.y, b.x, b.y};
  }
  *reinterpret_cast<half4_t *>(reinterpret_cast<unsigned char *>(xs) + xw + 16 * t) = h;
}

template <int QT, int NT, int G>
__device__ __forceinline__ void r_mfma(const unsigned char *wl, const half8_t *xs, int lane, float (&acc)[G][4]);

// Consume one stage: copy the weights into the wavefront's LDS area (wl) and
// the activations, as fp16 in MFMA operand order, into xs; then run the 8
// blocks (4 pairs) through the matrix cores into acc.
template <int QT, int NT, bool XF16, int G>
__device__ __forceinline__ void r_consume(const RRegs<QT, NT, XF16, G> &r, const RLane<QT, NT, G> &L, unsigned char *wl,
                                          half8_t *xs, int lane, float (&acc)[G][4]) {
  r_copy_w<QT, NT, G>(r.w, L, wl);
#pragma unroll
  for (int t = 0; t < NT; ++t) r_stage_x<XF16>(r.x[t], xs, L.xw, t);
  r_mfma<QT, NT, G>(wl, xs, lane, acc);
}

// The stage's 8 blocks (4 pairs) through the matrix cores into acc: the
// weights from the wavefront's LDS copy wl, the activations from xs.
template <int QT, int NT, int G>
__device__ __forceinline__ void r_mfma(const unsigned char *wl, const half8_t *xs, int lane, float (&acc)[G][4]) {
  using C = RCfg<QT, NT, G>;
  const int r16 = lane & 15, g = lane >> 4;
  const int slot = min(r16, NT - 1);
  if constexpr (QTraits<QT>::kquant) {
    // The quad is one Q4_K super-block: bytes 0..15 hold d | dmin and the
    // 12 scale bytes, then code chunk u (32 bytes at 16 + 32 u) carries
    // sub-block 2 u in its low nibbles and 2 u + 1 in its high ones; this
    // lane's 8 codes of a sub-block are bytes 8 g .. 8 g + 7 of the chunk.
    const half2_t m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
    auto codes = [&](uint32_t a0, uint32_t a1) {
      return make_half8(bytes01_plus_1024(a0) + m1024, bytes23_plus_1024(a0) + m1024,
                        bytes01_plus_1024(a1) + m1024, bytes23_plus_1024(a1) + m1024);
    };
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const unsigned char *rb = wl + (16 * gi + r16) * C::row_stride;
      auto ld = [&](int off) { return *reinterpret_cast<const uint32_t *>(rb + off); };
      const uint32_t h0 = ld(0), s0 = ld(4), s1 = ld(8), s2 = ld(12);
      const float d = half_bits_to_float(h0 & 0xFFFFu), dmin = half_bits_to_float(h0 >> 16);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const half8_t xe = xs[(4 * (2 * u) + g) * NT + slot];
        const half8_t xo = xs[(4 * (2 * u + 1) + g) * NT + slot];
        const uint32_t a0 = ld(16 + 32 * u + 8 * g), a1 = ld(20 + 32 * u + 8 * g);
        uint32_t sc0, mn0, sc1, mn1;
        q4k_scale_min(s0, s1, s2, 2 * u, sc0, mn0);
        q4k_scale_min(s0, s1, s2, 2 * u + 1, sc1, mn1);
        gemv_block_k<NT>(acc[gi], xe, codes(a0 & 0x0F0F0F0Fu, a1 & 0x0F0F0F0Fu), d * static_cast<float>(sc0),
                         dmin * static_cast<float>(mn0));
        gemv_block_k<NT>(acc[gi], xo, codes((a0 >> 4) & 0x0F0F0F0Fu, (a1 >> 4) & 0x0F0F0F0Fu),
                         d * static_cast<float>(sc1), dmin * static_cast<float>(mn1));
      }
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {  // pairs of blocks in the quad
    // A-operand rows past the NT token slots repeat the last slot (no
    // divergent reads; their results are never stored)
    const half8_t xe = xs[(4 * (2 * u) + g) * NT + slot];
    const half8_t xo = xs[(4 * (2 * u + 1) + g) * NT + slot];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {  // 16-row groups sharing the activations
      float *acc_g = acc[gi];
      const unsigned char *rb = wl + (16 * gi + r16) * C::row_stride + u * (2 * Block<QT>::bytes);
      auto ld = [&](int off) { return *reinterpret_cast<const uint32_t *>(rb + off); };
      if constexpr (QT == QMM_TYPE_Q4_0) {
        const uint32_t a0 = ld(4 * g), a1 = ld(4 * g + 4), b = ld(20 + 4 * g), d0 = ld(0), d1 = ld(16);
        gemv_block<NT>(acc_g, xe, gemv_codes<QT>(shift16(a0, a1), 0), d0 & 0xFFFFu);
        gemv_block<NT>(acc_g, xo, gemv_codes<QT>(b, 0), d1 >> 16);
      } else if constexpr (QT == QMM_TYPE_Q4_1) {
        // blocks at bytes 0 and 20 of the pair: d|m dword, then 4 code dwords
        const uint32_t a = ld(4 + 4 * g), b = ld(24 + 4 * g), dm0 = ld(0), dm1 = ld(20);
        gemv_block_min<NT>(acc_g, xe, gemv_codes<QT>(a, 0), dm0);
        gemv_block_min<NT>(acc_g, xo, gemv_codes<QT>(b, 0), dm1);
      } else if constexpr (QT == QMM_TYPE_Q5_0) {
        // blocks at bytes 0 and 22: d, fifth-bit word, codes (block 0's start
        // 2 bytes into a dword, block 1's are dword-aligned)
        const uint32_t w0 = ld(0), w1 = ld(4), a0 = ld(4 + 4 * g), a1 = ld(8 + 4 * g);
        const uint32_t w5 = ld(20), h1 = ld(24), b = ld(28 + 4 * g);
        gemv_block<NT>(acc_g, xe, gemv_codes5<QT>(shift16(a0, a1), shift16(w0, w1), 4 * g), w0 & 0xFFFFu);
        gemv_block<NT>(acc_g, xo, gemv_codes5<QT>(b, h1, 4 * g), w5 >> 16);
      } else if constexpr (QT == QMM_TYPE_Q5_1) {
        // blocks at bytes 0 and 24: d|m, fifth-bit word, 4 code dwords
        const uint32_t dm0 = ld(0), h0 = ld(4), a = ld(8 + 4 * g), dm1 = ld(24), h1 = ld(28), b = ld(32 + 4 * g);
        gemv_block_min<NT>(acc_g, xe, gemv_codes5<QT>(a, h0, 4 * g), dm0);
        gemv_block_min<NT>(acc_g, xo, gemv_codes5<QT>(b, h1, 4 * g), dm1);
      } else {
        const uint32_t a0 = ld(8 * g), a1 = ld(8 * g + 4), a2 = ld(8 * g + 8);
        const uint32_t b0 = ld(36 + 8 * g), b1 = ld(40 + 8 * g), d0 = ld(0), d1 = ld(32);
        gemv_block<NT>(acc_g, xe, gemv_codes<QT>(shift16(a0, a1), shift16(a1, a2)), d0 & 0xFFFFu);
        gemv_block<NT>(acc_g, xo, gemv_codes<QT>(b0, b1), d1 >> 16);
      }
    }
  }
}

// Partial sums of the wavefronts, added in wavefront order. D element e of
// lane l: token 4 (l / 16) + e, row l % 16 of row group gi. The barrier
// waits on LDS only, so weight loads in flight need not land first.
template <int NT, int WAVES, int G>
__device__ __forceinline__ void r_reduce(float *red, int wave, int lane, const float (&acc)[G][4],
                                         __attribute__((address_space(1))) float *Y, int row0, int n_rows,
                                         int n_tokens, GPtr<int32_t> tok_rows = nullptr) {
  constexpr int kRedLanes = NT > 4 ? 32 : 16;
  static_assert(16 * G * NT <= 64 * WAVES, "one thread per output of the workgroup");
  if (lane < kRedLanes) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((wave * G + gi) * 32 + lane) * 4 + e] = acc[gi][e];
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (threadIdx.x < 16 * G * NT) {
    const int gi = threadIdx.x / (16 * NT), rem = threadIdx.x - gi * (16 * NT);
    const int r = rem & 15;
    const int t = rem >> 4;
    const int src = r + 16 * (t >> 2);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[((w * G + gi) * 32 + src) * 4 + (t & 3)];
    const int row = row0 + 16 * gi + r;
    if (t < n_tokens && row < n_rows) {
      // token slot t's output row: t, or (tile form) its pair's row
      const int64_t yr = tok_rows ? static_cast<int64_t>(tok_rows[t]) : t;
      Y[yr * n_rows + row] = sum;
    }
  }
}

template <int QT, int NT, bool XF16, int WAVES, bool IDS = false, bool TILES = false, int G = 1>
__global__ __launch_bounds__(64 * WAVES, (WAVES == kKSplitLarge ? RCfg<QT, NT, G>::waves_per_simd_large : 4)) void gemv_stream_kernel(
    const uint8_t *W0, const void *X0, float *Y0, int64_t nb1_0, int n_rows0, int nblk0, int n_tokens0, int k0,
    int64_t, int64_t, const RBatch batch) {
  (void)batch;  // read through the kernel-argument pointer
  static_assert(G == 1 || (!IDS && !TILES), "row groups of 16 G rows: plain MUL_MATs only");
  using C = RCfg<QT, NT, G>;
  constexpr int QC = C::quad_chunks;
  constexpr int D = WAVES == kKSplitLarge ? C::depth_large : C::depth;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  // Matrix 0's fields are scalar arguments, which the hardware preloads into
  // scalar registers when the wavefront starts (kernel-argument preloading),
  // so its loads are issued without a memory round trip for the descriptor.
  // Other matrices read their record from the table that follows them.
  uint64_t wp0, xp0, yp0;
  int64_t nb1;
  int n_rows, nblk, n_tokens, k;
  uint32_t x_records = 0;       // bytes of X the buffer resource covers
  GPtr<int32_t> tok = nullptr;  // tile form: the tile's pairs
  int n_ids_t = 1, x_slots_t = 1;
  if constexpr (TILES) {
    static_assert(IDS && !XF16, "the tile form is expert-routed with fp32 activations");
    typedef const __attribute__((address_space(4))) char *KBytes;
    const u32x16_t rec = ((KRec)((KBytes)__builtin_amdgcn_kernarg_segment_ptr() + kRTableOffset))[1];
    const GPtr<int32_t> list = (GPtr<int32_t>)((static_cast<uint64_t>(rec[1]) << 32) | rec[0]);
    const int64_t nb2 = static_cast<int64_t>((static_cast<uint64_t>(rec[3]) << 32) | rec[2]);
    const GPtr<int32_t> tiles = (GPtr<int32_t>)((static_cast<uint64_t>(rec[9]) << 32) | rec[8]);
    const int ti = static_cast<int>(rec[7]) + static_cast<int>(blockIdx.y);
    const int e = __builtin_amdgcn_readfirstlane(tiles[4 * ti]);
    const int first = __builtin_amdgcn_readfirstlane(tiles[4 * ti + 1]);
    const int cnt = __builtin_amdgcn_readfirstlane(tiles[4 * ti + 2]);
    if (cnt == 0) return;  // whole workgroup: an unused tile
    n_ids_t = static_cast<int>(rec[5]);
    x_slots_t = static_cast<int>(rec[6]);
    x_records = rec[10];
    tok = list + first;
    nb1 = nb1_0;
    n_rows = n_rows0, nblk = nblk0, n_tokens = cnt, k = k0;
    wp0 = reinterpret_cast<uint64_t>(W0) + static_cast<uint64_t>(e) * static_cast<uint64_t>(nb2);
    xp0 = reinterpret_cast<uint64_t>(X0);
    yp0 = reinterpret_cast<uint64_t>(Y0);
  } else if constexpr (IDS) {
    // Expert-routed: matrix 0's fields describe expert 0 of the stack and
    // the shared X and Y; the routing record selects this pair's expert.
    typedef const __attribute__((address_space(4))) char *KBytes;
    const u32x16_t rec = ((KRec)((KBytes)__builtin_amdgcn_kernarg_segment_ptr() + kRTableOffset))[1];
    const GPtr<int32_t> ids = (GPtr<int32_t>)((static_cast<uint64_t>(rec[1]) << 32) | rec[0]);
    const int64_t nb2 = static_cast<int64_t>((static_cast<uint64_t>(rec[3]) << 32) | rec[2]);
    const int n_experts = static_cast<int>(rec[4]), n_ids = static_cast<int>(rec[5]);
    const int x_slots = static_cast<int>(rec[6]);
    const int p = static_cast<int>(rec[7]) + static_cast<int>(blockIdx.y);
    const int e = __builtin_amdgcn_readfirstlane(ids[p]);
    const int t = p / n_ids, slot = p - t * n_ids;
    nb1 = nb1_0;
    n_rows = n_rows0, nblk = nblk0, n_tokens = 1, k = k0;
    yp0 = reinterpret_cast<uint64_t>(Y0) + static_cast<uint64_t>(p) * static_cast<uint64_t>(n_rows) * 4;
    if (e < 0 || e >= n_experts) {
      // no such expert: this pair's rows are NaN
      const int row = static_cast<int>(blockIdx.x) * 16 + static_cast<int>(threadIdx.x);
      if (threadIdx.x < 16 && row < n_rows)
        reinterpret_cast<__attribute__((address_space(1))) float *>(yp0)[row] = __builtin_bit_cast(float, 0x7FC00000u);
      return;
    }
    wp0 = reinterpret_cast<uint64_t>(W0) + static_cast<uint64_t>(e) * static_cast<uint64_t>(nb2);
    xp0 = reinterpret_cast<uint64_t>(X0) +
          (static_cast<uint64_t>(t) * x_slots + (x_slots > 1 ? slot : 0)) * static_cast<uint64_t>(k) * 4;
  } else if (blockIdx.y == 0) {
    wp0 = reinterpret_cast<uint64_t>(W0);
    xp0 = reinterpret_cast<uint64_t>(X0);
    yp0 = reinterpret_cast<uint64_t>(Y0);
    nb1 = nb1_0;
    n_rows = n_rows0, nblk = nblk0, n_tokens = n_tokens0, k = k0;
  } else {
    typedef const __attribute__((address_space(4))) char *KBytes;
    const u32x16_t rec = ((KRec)((KBytes)__builtin_amdgcn_kernarg_segment_ptr() + kRTableOffset))[blockIdx.y];
    auto ptr = [&](int i) { return (static_cast<uint64_t>(rec[i + 1]) << 32) | rec[i]; };
    wp0 = ptr(0);
    xp0 = ptr(2);
    yp0 = ptr(4);
    nb1 = static_cast<int64_t>(ptr(6));
    n_rows = static_cast<int>(rec[8]), nblk = static_cast<int>(rec[9]), n_tokens = static_cast<int>(rec[10]),
    k = static_cast<int>(rec[11]);
  }
  const int rg = blockIdx.x;
  if (rg * 16 * G >= n_rows) return;  // whole workgroup: past this matrix's rows
  // The output pointer may be rebuilt from integers, so it is cast to the
  // global address space explicitly (a generic pointer would make the store a
  // flat access).
  __attribute__((address_space(1))) float *Y = (__attribute__((address_space(1))) float *)yp0;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = rg * 16 * G;
  // this wavefront's quads [q_lo, q_hi)
  const int qn = nblk >> 3;
  const int q_lo = (wave * qn) / WAVES, q_hi = ((wave + 1) * qn) / WAVES;

  unsigned char *wl = smem + wave * C::lds_per_wave;
  half8_t *xs = reinterpret_cast<half8_t *>(wl + C::w_lds);
  float *red = reinterpret_cast<float *>(smem + WAVES * C::lds_per_wave);
  const RLane<QT, NT, G> L(lane, static_cast<uint32_t>(nb1));

  // Weights and activations are read through buffer resources: a uniform
  // base with 32-bit per-lane offsets (one multiply per load slot, once) and
  // the quad's offset in a scalar register, so advancing a stage costs no
  // vector instructions. A raw buffer read at or past num_records returns
  // zero, so rows past n_rows need no clamp (their results are never stored).
  // Token slots past n_tokens re-read the last token.
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void *>(wp0), 0, static_cast<int>(static_cast<uint32_t>(n_rows * nb1)), kRsrcWord3);
  if constexpr (!TILES) x_records = static_cast<uint32_t>(n_tokens * k * (XF16 ? 2 : 4));
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(xp0), 0, static_cast<int>(x_records), kRsrcWord3);
  uint32_t wv[C::w_loads];
#pragma unroll
  for (int j = 0; j < C::w_loads; ++j)
    wv[j] = static_cast<uint32_t>(row0) * static_cast<uint32_t>(nb1) + L.wv[j];
  uint32_t xv[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint32_t xrow = static_cast<uint32_t>(min(t, n_tokens - 1));
    if constexpr (TILES) {
      // the pair's activation row: X[token][slot], or X[token][0] when shared
      const int p = tok[min(t, n_tokens - 1)];
      const int tt = p / n_ids_t;
      xrow = static_cast<uint32_t>(tt * x_slots_t + (x_slots_t > 1 ? p - tt * n_ids_t : 0));
    }
    xv[t] = (xrow * static_cast<uint32_t>(k) + 4 * lane) * (XF16 ? 2 : 4);
  }

  auto issue = [&](RRegs<QT, NT, XF16, G> &r, int q) {
    const int wq = q * (QC * 16), xq = q * 256 * (XF16 ? 2 : 4);
#pragma unroll
    for (int j = 0; j < C::w_loads; ++j)
      r.w[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wres, wv[j], wq, 0));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (XF16)
        r.x[t] = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(xres, xv[t], xq, 0));
      else
        r.x[t] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(xres, xv[t], xq, 0));
    }
  };

  float acc[G][4];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) acc[gi][0] = acc[gi][1] = acc[gi][2] = acc[gi][3] = 0.f;
  // Rounds of up to D stages: all loads of a round are issued at once (the
  // whole wavefront's share of k in one round for the common shapes), then
  // the stages are consumed in order. Other wavefronts on the CU overlap
  // their computation with this one's loads.
  // With 8 token slots (the heaviest stages), a wavefront raises its
  // priority while it issues a round's loads, so loads of wavefronts that
  // reach their issue point go out ahead of other wavefronts' arithmetic
  // (32000 x 4096 at 8 tokens: 26.4 -> 23.9 us; no change at 1 to 4 tokens).
  constexpr bool kIssuePrio = NT >= 8;
  RRegs<QT, NT, XF16, G> st[D];
  for (int q = q_lo; q < q_hi; q += D) {
    if constexpr (kIssuePrio) {
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (q + i < q_hi) issue(st[i], q + i);
    if constexpr (kIssuePrio) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (q + i < q_hi) r_consume<QT, NT, XF16, G>(st[i], L, wl, xs, lane, acc);
  }
  r_reduce<NT, WAVES, G>(red, wave, lane, acc, Y, row0, n_rows, n_tokens, tok);
}

// Tall matrices with 3 to 8 tokens (the output projection of a small
// decode batch). The k-split kernel above stages all n_tokens x k activations
// once per 16 or 32 rows; at 8 tokens that is 1.7 activation bytes per
// weight byte, read from L2 and converted by every workgroup. Here a
// workgroup owns 128 rows, one 16-row group per wavefront, each wavefront
// running the full k of its rows, and the workgroup stages each chunk of
// activations (up to 64 KiB of fp16) in LDS once for all eight wavefronts:
// a quarter of the activation traffic per weight byte, and no reduction
// across wavefronts (each output is one wavefront's running sum over the
// blocks in order). Weights stream as in the k-split kernel (the same
// 16-row stages, the same LDS copy and MFMAs), kTallDepth stages ahead, and
// the stream runs on across chunk boundaries.
constexpr int kTallWaves = 8;
constexpr int kTallRows = 16 * kTallWaves;
constexpr int kTallXBytes = 64 * 1024;  // staged activations per chunk
constexpr int kTallXInFlight = 4;       // activation loads a thread has in flight while staging

template <int QT, int NT> struct TallCfg {
  using C = RCfg<QT, NT>;
  // stages in flight per wavefront: 4 (2 for Q8_0, whose stage takes 20
  // registers); a power of two, so it divides the chunk
  static constexpr int depth = 4 * C::w_loads <= 16 ? 4 : 2;
  // quads per activation chunk (128 / NT)
  static constexpr int chunk_quads = kTallXBytes / C::x_lds;
  static_assert(chunk_quads % depth == 0, "chunks are whole rounds of stages");
  static constexpr size_t lds = static_cast<size_t>(kTallWaves) * C::w_lds + kTallXBytes;
};

template <int QT, int NT, bool XF16>
__global__ __launch_bounds__(64 * kTallWaves, 4) void gemv_tall_kernel(const uint8_t *W, const void *X, float *Y0,
                                                                        int64_t nb1, int n_rows, int nblk,
                                                                        int n_tokens, int k) {
  using C = RCfg<QT, NT>;
  using T = TallCfg<QT, NT>;
  constexpr int QC = C::quad_chunks;
  constexpr int D = T::depth;
  constexpr int CQ = T::chunk_quads;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  unsigned char *wl = smem + wave * C::w_lds;
  half8_t *xs = reinterpret_cast<half8_t *>(smem + kTallWaves * C::w_lds);
  __attribute__((address_space(1))) float *Y = (__attribute__((address_space(1))) float *)Y0;

  const int row0 = static_cast<int>(blockIdx.x) * kTallRows + 16 * wave;
  const RLane<QT, NT> L(lane, static_cast<uint32_t>(nb1));
  // the wavefront's rows start the resource (rows past n_rows read as zero)
  const int64_t left = static_cast<int64_t>(n_rows - row0) * nb1;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(W) + (row0 < n_rows ? static_cast<int64_t>(row0) * nb1 : 0), 0,
      static_cast<int>(static_cast<uint32_t>(left > 0 ? left : 0)), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void *>(X), 0, static_cast<int>(static_cast<uint32_t>(n_tokens * k * (XF16 ? 2 : 4))), kRsrcWord3);
  const int qn = nblk >> 3;

  u32x4_t st[D][C::w_loads];
  auto issue = [&](u32x4_t (&w)[C::w_loads], int q) {
    const int wq = q * (QC * 16);
#pragma unroll
    for (int j = 0; j < C::w_loads; ++j)
      w[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wres, L.wv[j], wq, 0));
  };
  // Stage quads [q0, q0 + nq) of every token slot: piece i is slot i / (64 nq),
  // quad i / 64 % nq, elements 4 l .. 4 l + 3 (l = i % 64) of that quad,
  // placed as the k-split kernel places a lane's piece. Token slots past
  // n_tokens repeat the last token (their outputs are not stored). A thread
  // issues the loads of kTallXInFlight pieces before converting any: the
  // staging is a chain of L2 round trips (16 per thread for 8 tokens of
  // k = 4096), and one piece per trip left the weight stream waiting
  // (32000 x 4096 at 8 tokens: 23.8-24.3 -> 22.0-22.6 us).
  auto stage = [&](int q0, int nq) {
    const int pieces = NT * nq * 64;
    using XP = typename std::conditional<XF16, half4_t, float4_t>::type;
    for (int i0 = threadIdx.x; i0 < pieces; i0 += kTallXInFlight * 64 * kTallWaves) {
      XP v[kTallXInFlight];
#pragma unroll
      for (int u = 0; u < kTallXInFlight; ++u) {
        const int i = i0 + u * 64 * kTallWaves;
        const int l = i & 63, qi = (i >> 6) % nq, t = (i >> 6) / nq;
        const uint32_t off =
            (static_cast<uint32_t>(min(t, n_tokens - 1)) * k + (q0 + qi) * 256 + 4 * l) * (XF16 ? 2 : 4);
        if (i < pieces) {
          if constexpr (XF16)
            v[u] = __builtin_bit_cast(half4_t, __builtin_amdgcn_raw_buffer_load_b64(xres, off, 0, 0));
          else
            v[u] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
        }
      }
#pragma unroll
      for (int u = 0; u < kTallXInFlight; ++u) {
        const int i = i0 + u * 64 * kTallWaves;
        const int l = i & 63, qi = (i >> 6) % nq, t = (i >> 6) / nq;
        const RLane<QT, NT> P(l, 0u);
        if (i < pieces) r_stage_x<XF16>(v[u], xs + qi * (C::x_lds / 16), P.xw, t);
      }
    }
  };

  float acc[1][4] = {{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
  for (int i = 0; i < D; ++i)
    if (i < qn) issue(st[i], i);
  for (int c0 = 0; c0 < qn; c0 += CQ) {
    const int nq = min(CQ, qn - c0);
    if (c0 > 0) {  // every wavefront is done with the previous chunk
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    stage(c0, nq);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this thread's pieces are in LDS
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // quads q = c0 + j; stage register set (q % D) is fixed at compile time
    // by stepping the chunk in whole rounds of D quads
    for (int j = 0; j < nq; j += D) {
#pragma unroll
      for (int i = 0; i < D; ++i) {
        const int q = c0 + j + i;
        if (j + i < nq) {
          // quads are issued in order, so set i holds quad q (chunks are a
          // whole number of rounds: CQ % D == 0)
          r_copy_w<QT, NT, 1>(st[i], L, wl);
          if (q + D < qn) issue(st[i], q + D);
          r_mfma<QT, NT, 1>(wl, xs + (j + i) * (C::x_lds / 16), lane, acc);
        }
      }
    }
  }
  if (lane < (NT > 4 ? 32 : 16) && row0 + (lane & 15) < n_rows) {
    const int row = row0 + (lane & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 4 * (lane >> 4) + e;
      if (t < n_tokens) Y[static_cast<int64_t>(t) * n_rows + row] = acc[0][e];
    }
  }
}

// ------------------------------------------------------------------ host side

// Row groups per workgroup. A multi-token call reads its n_tokens x k
// activations once per workgroup, so a workgroup that covers G 16-row groups
// (one staged activation set feeding G MFMA row tiles) divides that traffic
// by G, at the price of more stage registers and LDS per wavefront. Measured
// on MI355X (32000 x 4096 and 11008 x 4096 Q4_0, weights from HBM): with 8
// token slots G = 2 takes 34.4 -> 26.6 us and 14.9 -> 14.2 us, G = 4 29.5 and
// 13.7 us; with 4 slots G = 2 helps the 32000-row matrix (-7 %) and slows the
// 11008-row one (+12 %), G = 4 slows both; 2 slots and single-token calls
// gain nothing. So only 8-slot calls on launches of more row groups than CUs
// (8 wavefronts per workgroup) use G = 2, where the stage copies fit LDS.
template <int QT, int NT, int G> constexpr bool groups_fit() {
  return kKSplitLarge * RCfg<QT, NT, G>::lds_per_wave + kKSplitLarge * G * 32 * 4 * 4 <= 160 * 1024;
}
template <int QT, int NT> constexpr int row_groups_for() {
  if constexpr (NT == 8 && groups_fit<QT, NT, 2>()) return 2;
  else return 1;
}

template <int QT, int NT, bool XF16, int WAVES, int G>
static hipError_t r_go_w(const RBatch &B, int count, int max_rg, hipStream_t s) {
  const size_t lds = static_cast<size_t>(WAVES) * RCfg<QT, NT, G>::lds_per_wave + WAVES * G * 32 * 4 * sizeof(float);
  const RMat &m0 = B.m[0];
  return launch(gemv_stream_kernel<QT, NT, XF16, WAVES, false, false, G>, dim3((max_rg + G - 1) / G, count),
                dim3(64 * WAVES), lds, s, m0.W, m0.X, m0.Y, m0.nb1, m0.n_rows, m0.nblk, m0.n_tokens, m0.k, int64_t{0},
                int64_t{0}, B);
}

template <int QT, int NT, bool XF16>
static hipError_t r_go(const RBatch &B, int count, int max_rg, int waves, hipStream_t s) {
  return waves == kKSplitSmall ? r_go_w<QT, NT, XF16, kKSplitSmall, 1>(B, count, max_rg, s)
                               : r_go_w<QT, NT, XF16, kKSplitLarge, row_groups_for<QT, NT>()>(B, count, max_rg, s);
}

template <int QT, bool XF16>
static hipError_t r_nt(int nt, const RBatch &B, int count, int max_rg, int waves, hipStream_t s) {
  if (nt <= 1) return r_go<QT, 1, XF16>(B, count, max_rg, waves, s);
  if (nt <= 2) return r_go<QT, 2, XF16>(B, count, max_rg, waves, s);
  if (nt <= 4) return r_go<QT, 4, XF16>(B, count, max_rg, waves, s);
  return r_go<QT, 8, XF16>(B, count, max_rg, waves, s);
}

static int nt_slots(int64_t n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8; }

static bool streamable(const MatmulDesc &d) {
  const int64_t nblk = d.k / 32;
  // buffer offsets are 32-bit (the matrix and the activations must span less
  // than 4 GiB) and the per-lane row offsets use a 24-bit multiply
  const int64_t xbytes = d.n_tokens * d.k * (d.x_f16 ? 2 : 4);
  return reinterpret_cast<uintptr_t>(d.W) % 16 == 0 && d.nb1 % 16 == 0 && nblk % 8 == 0 &&
         d.n_rows * d.nb1 < (int64_t{1} << 32) && d.nb1 < (int64_t{1} << 24) && xbytes < (int64_t{1} << 32);
}

static RMat record(const MatmulDesc &d) {
  RMat r{};
  r.W = static_cast<const uint8_t *>(d.W);
  r.X = d.X;
  r.Y = d.Y;
  r.nb1 = d.nb1;
  r.n_rows = static_cast<int>(d.n_rows);
  r.nblk = static_cast<int>(d.k / 32);
  r.n_tokens = static_cast<int>(d.n_tokens);
  r.k = static_cast<int>(d.k);
  return r;
}

template <int QT, int WAVES>
static hipError_t id_go_w(const RBatch &B, int count, int rg, hipStream_t s) {
  const size_t lds = static_cast<size_t>(WAVES) * RCfg<QT, 1>::lds_per_wave + WAVES * 32 * 4 * sizeof(float);
  const RMat &m0 = B.m[0];
  return launch(gemv_stream_kernel<QT, 1, false, WAVES, true>, dim3(rg, count), dim3(64 * WAVES), lds, s, m0.W, m0.X,
                m0.Y, m0.nb1, m0.n_rows, m0.nblk, m0.n_tokens, m0.k, int64_t{0}, int64_t{0}, B);
}

bool id_streamable(const void *W, int64_t n_rows, int64_t k, int64_t nb1, int64_t nb2) {
  return reinterpret_cast<uintptr_t>(W) % 16 == 0 && nb1 % 16 == 0 && nb2 % 16 == 0 && (k / 32) % 8 == 0 &&
         n_rows * nb1 < (int64_t{1} << 32) && nb1 < (int64_t{1} << 24) && k * 4 < (int64_t{1} << 32);
}

hipError_t launch_gemv_id_stream(const void *W, int qtype, int64_t n_experts, int64_t n_rows, int64_t k, int64_t nb1,
                                 int64_t nb2, const float *X, int64_t x_slots, const int32_t *ids, int64_t n_ids,
                                 int64_t n_tokens, float *Y, hipStream_t stream) {
  RBatch B{};
  B.m[0] = record(MatmulDesc{W, qtype, n_rows, k, nb1, X, false, 1, Y});
  RRoute route{};
  route.ids = ids;
  route.nb2 = nb2;
  route.n_experts = static_cast<int>(n_experts);
  route.n_ids = static_cast<int>(n_ids);
  route.x_slots = static_cast<int>(x_slots);
  const int64_t pairs = n_tokens * n_ids;
  const int rg = static_cast<int>((n_rows + 15) / 16);
  const int waves = k_split_for(pairs * rg, device_cus());
  constexpr int64_t kMaxY = 65535;  // grid rows per launch
  for (int64_t p0 = 0; p0 < pairs; p0 += kMaxY) {
    route.pair0 = static_cast<int>(p0);
    static_assert(sizeof(RRoute) == sizeof(RMat), "routing record fills one table slot");
    __builtin_memcpy(&B.m[1], &route, sizeof(RRoute));
    const int count = static_cast<int>(pairs - p0 < kMaxY ? pairs - p0 : kMaxY);
    hipError_t e;
    e = by_qtype_k(qtype, [&](auto qt) {
      constexpr int QT = decltype(qt)::value;
      return waves == kKSplitSmall ? id_go_w<QT, kKSplitSmall>(B, count, rg, stream)
                                   : id_go_w<QT, kKSplitLarge>(B, count, rg, stream);
    });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int QT, int NT, int WAVES>
static hipError_t idt_go_w(const RBatch &B, int count, int rg, hipStream_t s) {
  const size_t lds = static_cast<size_t>(WAVES) * RCfg<QT, NT>::lds_per_wave + WAVES * 32 * 4 * sizeof(float);
  const RMat &m0 = B.m[0];
  return launch(gemv_stream_kernel<QT, NT, false, WAVES, true, true>, dim3(rg, count), dim3(64 * WAVES), lds, s, m0.W,
                m0.X, m0.Y, m0.nb1, m0.n_rows, m0.nblk, m0.n_tokens, m0.k, int64_t{0}, int64_t{0}, B);
}

hipError_t launch_gemv_id_tiles(const void *W, int qtype, int64_t n_experts, int64_t n_rows, int64_t k, int64_t nb1,
                                int64_t nb2, const float *X, int64_t x_slots, int64_t n_ids, int64_t n_tokens,
                                const int32_t *list, const int32_t *tiles, int64_t max_tiles, int nt, float *Y,
                                hipStream_t stream) {
  RBatch B{};
  B.m[0] = record(MatmulDesc{W, qtype, n_rows, k, nb1, X, false, 1, Y});
  RRoute route{};
  route.ids = list;
  route.nb2 = nb2;
  route.n_experts = static_cast<int>(n_experts);
  route.n_ids = static_cast<int>(n_ids);
  route.x_slots = static_cast<int>(x_slots);
  route.tiles = tiles;
  route.x_bytes = static_cast<uint32_t>(n_tokens * x_slots * k * 4);
  const int rg = static_cast<int>((n_rows + 15) / 16);
  const int waves = k_split_for(max_tiles * rg, device_cus());
  constexpr int64_t kMaxY = 65535;  // grid rows per launch
  for (int64_t t0 = 0; t0 < max_tiles; t0 += kMaxY) {
    route.pair0 = static_cast<int>(t0);
    __builtin_memcpy(&B.m[1], &route, sizeof(RRoute));
    const int count = static_cast<int>(max_tiles - t0 < kMaxY ? max_tiles - t0 : kMaxY);
    const hipError_t e = by_qtype_k(qtype, [&](auto qt) {
      constexpr int QT = decltype(qt)::value;
      auto go = [&](auto ntc) {
        constexpr int NT = decltype(ntc)::value;
        return waves == kKSplitSmall ? idt_go_w<QT, NT, kKSplitSmall>(B, count, rg, stream)
                                     : idt_go_w<QT, NT, kKSplitLarge>(B, count, rg, stream);
      };
      if (nt <= 2) return go(std::integral_constant<int, 2>{});
      if (nt <= 4) return go(std::integral_constant<int, 4>{});
      return go(std::integral_constant<int, 8>{});
    });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// A single streamable MUL_MAT of 3 to 8 tokens whose 128-row tiles nearly
// fill the GPU (at least 7/8 of a tile per compute unit) runs on the
// row-split kernel.
static bool tall_for(const MatmulDesc &d, int cus) {
  return d.n_tokens >= 3 && d.n_tokens <= 8 && cus > 0 && (d.n_rows + kTallRows - 1) / kTallRows * 8 >= 7 * cus;
}

static hipError_t launch_gemv_tall(const MatmulDesc &d, hipStream_t stream) {
  const int nt = nt_slots(d.n_tokens);
  const int tiles = static_cast<int>((d.n_rows + kTallRows - 1) / kTallRows);
  return by_qtype_k(d.qtype, [&](auto q) {
    constexpr int QT = decltype(q)::value;
    auto go = [&](auto ntc, auto xc) {
      constexpr int NT = decltype(ntc)::value;
      constexpr bool XF = decltype(xc)::value;
      return launch(gemv_tall_kernel<QT, NT, XF>, dim3(tiles), dim3(64 * kTallWaves), TallCfg<QT, NT>::lds, stream,
                    static_cast<const uint8_t *>(d.W), d.X, d.Y, d.nb1, static_cast<int>(d.n_rows),
                    static_cast<int>(d.k / 32), static_cast<int>(d.n_tokens), static_cast<int>(d.k));
    };
    auto by_x = [&](auto ntc) { return d.x_f16 ? go(ntc, std::true_type{}) : go(ntc, std::false_type{}); };
    if (nt <= 4) return by_x(std::integral_constant<int, 4>{});
    return by_x(std::integral_constant<int, 8>{});
  });
}

hipError_t launch_gemv_batch(const MatmulDesc *d, int count_all, hipStream_t stream) {
  // Consecutive streamable descriptors with the same (type, activation type,
  // token-slot count) share a launch of up to kRMaxMats matrices; the rest
  // go one by one to the general kernel.
  int i = 0;
  while (i < count_all) {
    if (!streamable(d[i])) {
      hipError_t e = launch_gemv_general(d[i].W, d[i].qtype, d[i].n_rows, d[i].k, d[i].nb1, d[i].X, d[i].x_f16,
                                         d[i].n_tokens, d[i].Y, stream);
      if (e != hipSuccess) return e;
      ++i;
      continue;
    }
    RBatch B{};
    const int qt = d[i].qtype, nt = nt_slots(d[i].n_tokens);
    const bool xf = d[i].x_f16;
    int j = i, count = 0, max_rg = 0;
    int64_t total_rg = 0;
    while (j < count_all && count < kRMaxMats && streamable(d[j]) && d[j].qtype == qt && d[j].x_f16 == xf &&
           nt_slots(d[j].n_tokens) == nt) {
      RMat &r = B.m[count++];
      r.W = static_cast<const uint8_t *>(d[j].W);
      r.X = d[j].X;
      r.Y = d[j].Y;
      r.nb1 = d[j].nb1;
      r.n_rows = static_cast<int>(d[j].n_rows);
      r.nblk = static_cast<int>(d[j].k / 32);
      r.n_tokens = static_cast<int>(d[j].n_tokens);
      r.k = static_cast<int>(d[j].k);
      max_rg = max(max_rg, static_cast<int>((d[j].n_rows + 15) / 16));
      total_rg += (d[j].n_rows + 15) / 16;
      ++j;
    }
    const int cus = device_cus();
    hipError_t e;
    if (count == 1 && tall_for(d[i], cus)) {
      e = launch_gemv_tall(d[i], stream);
    } else {
      const int waves = k_split_for(total_rg, cus);
      e = by_qtype_k(qt, [&](auto q) {
        constexpr int QT = decltype(q)::value;
        return xf ? r_nt<QT, true>(nt, B, count, max_rg, waves, stream)
                  : r_nt<QT, false>(nt, B, count, max_rg, waves, stream);
      });
    }
    if (e != hipSuccess) return e;
    i = j;
  }
  return hipSuccess;
}

}  // namespace qmm
