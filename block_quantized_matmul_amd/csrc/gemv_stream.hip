// Streaming decode MUL_MAT (1 <= n_tokens <= 8) for 16-byte-aligned layouts,
// one or several independent matrices per launch.
//
// What is computed: as in gemv.hip, y[t][r] = sum_b d_rb * sum_i (q - z) x[t][32 b + i]
// ([Bind] "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section 2.3; [Arch]
// "llama.cpp 源码完全拆解(一)：整体架构与模块全景", section "权重装载：GGUF、mmap
// 与 4 bit 块"), with the same exact-code MFMA formulation and per-block fp32
// scale (see gemv_common.h).
//
// Design (MI355X, gfx950): the kernel is an HBM stream. Launch overhead and
// the ramp of a kernel cost about as much as reading ten megabytes, so a
// launch covers several MUL_MATs when the caller has them, and one resident
// workgroup per CU walks a contiguous range of 16-row groups across all of
// them (persistent grid = number of CUs).
//
// Weight path: the 8 wavefronts of a workgroup split a row group's k into
// contiguous ranges of quads (8 blocks = 144 bytes Q4_0 / 272 bytes Q8_0,
// always a whole number of 16-byte chunks). A wavefront moves one stage (two
// Q4_0 quads or one Q8_0 quad, for all 16 rows) with fully coalesced
// 16-byte loads: consecutive lanes take consecutive chunks of a row. The next
// stage is in flight in registers while the current one is copied into the
// wavefront's own LDS buffer and consumed; the prefetch runs straight across
// row-group boundaries, and workgroup barriers wait on LDS only, so the
// weight stream never drains. Lanes then read their MFMA operands from LDS.
//
// Activations are staged once per matrix per workgroup into LDS as fp16 in
// operand order (2 * k * n_tokens bytes; at most 64 KiB).
#include "common.h"
#include "gemv_common.h"
#include "launch.h"

#include <stddef.h>

#include <mutex>

namespace qmm {

constexpr int kSWaves = 8;
constexpr int kSThreads = 64 * kSWaves;
constexpr int kSMaxMats = 16;
constexpr int kSXBudget = 64 * 1024;

template <int QT> struct SGeo;
template <> struct SGeo<QMM_TYPE_Q4_0> {
  static constexpr int quad_chunks = 9;     // 8 blocks = 144 bytes
  static constexpr int stage_quads = 2;
  static constexpr int row_stride = 19 * 16;  // 18 chunks + one of padding (LDS banks)
};
template <> struct SGeo<QMM_TYPE_Q8_0> {
  static constexpr int quad_chunks = 17;    // 8 blocks = 272 bytes
  static constexpr int stage_quads = 1;
  static constexpr int row_stride = 18 * 16;
};
template <int QT> constexpr int s_stage_chunks() { return 16 * SGeo<QT>::quad_chunks * SGeo<QT>::stage_quads; }
template <int QT> constexpr int s_loads() { return (s_stage_chunks<QT>() + 63) / 64; }

struct SMat {
  const uint8_t *W;
  const void *X;
  float *Y;
  int64_t nb1;
  int n_rows, nblk, n_tokens, k;
  int rg_end;  // row groups of this matrix and all before it
};
struct SBatch {
  SMat m[kSMaxMats];
  int count;
  int total_rg;
};

// The batch is the kernel's first argument, so its descriptors sit at the
// start of the kernel-argument segment. Reading them through that (constant
// address space) pointer gives uniform scalar loads; indexing the by-value
// parameter directly would copy the whole table to scratch.
typedef const __attribute__((address_space(4))) SBatch *KBatch;
static_assert(offsetof(SBatch, m) == 0, "descriptor table must lead the batch");

__device__ __forceinline__ KBatch s_args() { return (KBatch)__builtin_amdgcn_kernarg_segment_ptr(); }
__device__ __forceinline__ int s_mat_of(KBatch B, int rg) {
  int m = 0;
  while (m + 1 < B->count && rg >= B->m[m].rg_end) ++m;
  return m;
}
__device__ __forceinline__ SMat s_get(KBatch B, int m) {
  SMat r;
  r.W = B->m[m].W;
  r.X = B->m[m].X;
  r.Y = B->m[m].Y;
  r.nb1 = B->m[m].nb1;
  r.n_rows = B->m[m].n_rows;
  r.nblk = B->m[m].nblk;
  r.n_tokens = B->m[m].n_tokens;
  r.k = B->m[m].k;
  r.rg_end = B->m[m].rg_end;
  return r;
}
__device__ __forceinline__ int s_rg_begin(KBatch B, int m) { return m == 0 ? 0 : B->m[m - 1].rg_end; }

// Wait for this wave's LDS traffic, then meet the workgroup. Unlike
// __syncthreads(), this leaves outstanding global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int QT> struct SRegs { u32x4_t v[s_loads<QT>()]; };

// This wave's quads [q_lo, q_hi) of a matrix with nblk blocks.
__device__ __forceinline__ void s_quads(int nblk, int wave, int &q_lo, int &q_hi) {
  const int qn = nblk >> 3;
  q_lo = (wave * qn) / kSWaves;
  q_hi = ((wave + 1) * qn) / kSWaves;
}

// Lane-constant placement of a stage's 16-byte chunks: chunk c = 64 j + lane
// is (row, chunk within the row's segment). Computed once per kernel for a
// full stage (nq = stage_quads) and for a one-quad stage.
template <int QT> struct SPlace {
  int off[s_loads<QT>()];   // LDS byte offset within the wave's stage buffer, or -1 if no such chunk
  int row[s_loads<QT>()];   // row within the 16-row group
  int col[s_loads<QT>()];   // byte offset within the row's stage segment
};

template <int QT>
__device__ __forceinline__ SPlace<QT> s_place(int nq, int lane) {
  constexpr int QC = SGeo<QT>::quad_chunks;
  const int cpr = QC * nq, total = 16 * cpr;
  SPlace<QT> p;
#pragma unroll
  for (int j = 0; j < s_loads<QT>(); ++j) {
    const int c = 64 * j + lane;
    const int row = c / cpr, cc = c - (c / cpr) * cpr;
    p.row[j] = row;
    p.col[j] = 16 * cc;
    p.off[j] = c < total ? row * SGeo<QT>::row_stride + 16 * cc : -1;
  }
  return p;
}

template <int QT>
__device__ __forceinline__ void s_load(SRegs<QT> &r, const SMat &M, int row0, int quad0, const SPlace<QT> &P) {
  const uint8_t *base = M.W + static_cast<int64_t>(quad0) * (SGeo<QT>::quad_chunks * 16);
#pragma unroll
  for (int j = 0; j < s_loads<QT>(); ++j) {
    if (P.off[j] >= 0) {
      const int grow = min(row0 + P.row[j], M.n_rows - 1);
      r.v[j] = *reinterpret_cast<const u32x4_t *>(base + static_cast<int64_t>(grow) * M.nb1 + P.col[j]);
    }
  }
}

template <int QT>
__device__ __forceinline__ void s_store(unsigned char *wl, const SRegs<QT> &r, const SPlace<QT> &P) {
#pragma unroll
  for (int j = 0; j < s_loads<QT>(); ++j)
    if (P.off[j] >= 0) *reinterpret_cast<u32x4_t *>(wl + P.off[j]) = r.v[j];
}

__device__ __forceinline__ uint32_t lds_u32(const unsigned char *p) { return *reinterpret_cast<const uint32_t *>(p); }

// Consume one stage from LDS: pairs uu = 0 .. 4 nq - 1 starting at quad quad0.
template <int QT, int NT>
__device__ __forceinline__ void s_compute(float acc[4], const unsigned char *wl, const half8_t *xs, int quad0,
                                          int nq, int g, int r16, int xslot) {
  constexpr int PB = 2 * Block<QT>::bytes;  // bytes per pair
  const unsigned char *rb0 = wl + r16 * SGeo<QT>::row_stride;
#pragma unroll
  for (int uu = 0; uu < 4 * SGeo<QT>::stage_quads; ++uu) {
    if (uu < 4 * nq) {
      const unsigned char *rb = rb0 + uu * PB;
      const int blk = 2 * (4 * quad0 + uu);  // global index of the pair's even block
      const half8_t xe = xs[(4 * blk + g) * NT + xslot];
      const half8_t xo = xs[(4 * (blk + 1) + g) * NT + xslot];
      if constexpr (QT == QMM_TYPE_Q4_0) {
        const uint32_t a0 = lds_u32(rb + 4 * g), a1 = lds_u32(rb + 4 * g + 4);
        const uint32_t b = lds_u32(rb + 20 + 4 * g);
        const uint32_t d0 = lds_u32(rb), d1 = lds_u32(rb + 16);
        gemv_block<NT>(acc, xe, gemv_codes<QT>(shift16(a0, a1), 0), d0 & 0xFFFFu);
        gemv_block<NT>(acc, xo, gemv_codes<QT>(b, 0), d1 >> 16);
      } else {
        const uint32_t a0 = lds_u32(rb + 8 * g), a1 = lds_u32(rb + 8 * g + 4), a2 = lds_u32(rb + 8 * g + 8);
        const uint32_t b0 = lds_u32(rb + 36 + 8 * g), b1 = lds_u32(rb + 40 + 8 * g);
        const uint32_t d0 = lds_u32(rb), d1 = lds_u32(rb + 32);
        gemv_block<NT>(acc, xe, gemv_codes<QT>(shift16(a0, a1), shift16(a1, a2)), d0 & 0xFFFFu);
        gemv_block<NT>(acc, xo, gemv_codes<QT>(b0, b1), d1 >> 16);
      }
    }
  }
}

// Dynamic LDS layout: [x: x_bytes][weights: kSWaves * 16 * row_stride][red: 2 * kSWaves * 32 * 4 floats].
template <int QT, int NT, bool XF16>
__global__ __launch_bounds__(kSThreads) void gemv_stream_kernel(const SBatch batch, int x_bytes) {
  (void)batch;  // read through s_args()
  const KBatch B = s_args();
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int S = SGeo<QT>::stage_quads;
  half8_t *xs = reinterpret_cast<half8_t *>(smem);
  unsigned char *wl_all = smem + x_bytes;
  float *red = reinterpret_cast<float *>(wl_all + kSWaves * 16 * SGeo<QT>::row_stride);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar control flow
  const int r16 = lane & 15;
  const int g = lane >> 4;
  unsigned char *wl = wl_all + wave * 16 * SGeo<QT>::row_stride;
  const SPlace<QT> P_full = s_place<QT>(S, lane);
  const SPlace<QT> P_one = s_place<QT>(1, lane);

  const int rg_lo = static_cast<int>((static_cast<int64_t>(blockIdx.x) * B->total_rg) / gridDim.x);
  const int rg_hi = static_cast<int>((static_cast<int64_t>(blockIdx.x + 1) * B->total_rg) / gridDim.x);
  if (rg_lo >= rg_hi) return;  // whole workgroup

  // Prefetch cursor: the next (row group, stage) this wave will consume.
  int p_rg = rg_lo, p_s = 0;
  int p_m = s_mat_of(B, p_rg);
  SMat PM = s_get(B, p_m);
  int p_q_lo, p_q_hi;
  s_quads(PM.nblk, wave, p_q_lo, p_q_hi);
  // Advance the cursor past row groups in which this wave has no quads.
  auto settle = [&]() {
    while (p_rg < rg_hi && p_q_lo + S * p_s >= p_q_hi) {
      ++p_rg;
      p_s = 0;
      if (p_rg < rg_hi) {
        const int m = s_mat_of(B, p_rg);
        if (m != p_m) {
          p_m = m;
          PM = s_get(B, m);
          s_quads(PM.nblk, wave, p_q_lo, p_q_hi);
        }
      }
    }
  };
  settle();
  SRegs<QT> pre;
  if (p_rg < rg_hi) {
    const int q0 = p_q_lo + S * p_s;
    s_load<QT>(pre, PM, (p_rg - s_rg_begin(B, p_m)) * 16, q0, p_q_hi - q0 >= S ? P_full : P_one);
  }

  int cur_m = -1;
  SMat M = PM;
  int q_lo = 0, q_hi = 0;
  for (int rg = rg_lo; rg < rg_hi; ++rg) {
    const int m = s_mat_of(B, rg);
    if (m != cur_m) {
      // New matrix: stage its activations. All waves finished reading the
      // previous ones before the last row group's reduction barrier.
      cur_m = m;
      M = s_get(B, m);
      s_quads(M.nblk, wave, q_lo, q_hi);
      gemv_stage_x<QT, NT, XF16, kSThreads>(xs, M.X, M.n_tokens, M.k, 0, M.nblk);
      lds_barrier();
    }
    const int row0 = (rg - s_rg_begin(B, m)) * 16;
    const int xslot = min(r16, M.n_tokens - 1);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; q_lo + S * s < q_hi; ++s) {
      const int quad0 = q_lo + S * s;
      const int nq = min(S, q_hi - quad0);
      const SRegs<QT> cur = pre;
      // issue the next stage (possibly of a later row group) before consuming this one
      ++p_s;
      settle();
      if (p_rg < rg_hi) {
        const int q0 = p_q_lo + S * p_s;
        s_load<QT>(pre, PM, (p_rg - s_rg_begin(B, p_m)) * 16, q0, p_q_hi - q0 >= S ? P_full : P_one);
      }
      s_store<QT>(wl, cur, nq == S ? P_full : P_one);
      s_compute<QT, NT>(acc, wl, xs, quad0, nq, g, r16, xslot);
    }

    // Row-group reduction across the 8 wavefronts (double-buffered by parity).
    constexpr int kRedLanes = NT > 4 ? 32 : 16;
    float *rp = red + ((rg - rg_lo) & 1) * (kSWaves * 32 * 4);
    if (lane < kRedLanes) {
#pragma unroll
      for (int e = 0; e < 4; ++e) rp[(wave * 32 + lane) * 4 + e] = acc[e];
    }
    lds_barrier();
    if (threadIdx.x < 16 * NT) {
      const int r = threadIdx.x & 15;
      const int t = threadIdx.x >> 4;
      const int src = r + 16 * (t >> 2);
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) sum += rp[(w * 32 + src) * 4 + (t & 3)];
      const int orow = row0 + r;
      if (t < M.n_tokens && orow < M.n_rows) M.Y[static_cast<int64_t>(t) * M.n_rows + orow] = sum;
    }
  }
}

// ------------------------------------------------------------------ host side

static int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  static std::mutex mu;
  static int cached[64] = {0};
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static size_t s_lds_bytes(int qtype, int x_bytes) {
  const int rs = qtype == QMM_TYPE_Q4_0 ? SGeo<QMM_TYPE_Q4_0>::row_stride : SGeo<QMM_TYPE_Q8_0>::row_stride;
  return static_cast<size_t>(x_bytes) + kSWaves * 16 * rs + 2 * kSWaves * 32 * 4 * sizeof(float);
}

template <typename K> static hipError_t s_allow_lds(K kernel) {
  static const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  static_cast<int>(s_lds_bytes(QMM_TYPE_Q4_0, kSXBudget)));
  return e;
}

template <int QT, int NT, bool XF16>
static hipError_t s_go(const SBatch &B, int x_bytes, hipStream_t s) {
  hipError_t e = s_allow_lds(gemv_stream_kernel<QT, NT, XF16>);
  if (e != hipSuccess) return e;
  const int grid = min(B.total_rg, cu_count());
  return launch(gemv_stream_kernel<QT, NT, XF16>, dim3(grid), dim3(kSThreads), s_lds_bytes(QT, x_bytes), s, B, x_bytes);
}

template <int QT, bool XF16>
static hipError_t s_nt(int nt, const SBatch &B, int x_bytes, hipStream_t s) {
  if (nt <= 1) return s_go<QT, 1, XF16>(B, x_bytes, s);
  if (nt <= 2) return s_go<QT, 2, XF16>(B, x_bytes, s);
  if (nt <= 4) return s_go<QT, 4, XF16>(B, x_bytes, s);
  return s_go<QT, 8, XF16>(B, x_bytes, s);
}

static int nt_slots(int64_t n) { return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : 8; }

static bool streamable(const MatmulDesc &d) {
  const int64_t nblk = d.k / 32;
  return reinterpret_cast<uintptr_t>(d.W) % 16 == 0 && d.nb1 % 16 == 0 && nblk % 8 == 0 &&
         2 * d.k * nt_slots(d.n_tokens) <= kSXBudget && d.n_rows * d.nb1 < (int64_t{1} << 40);
}

hipError_t launch_gemv_batch(const MatmulDesc *d, int count, hipStream_t stream) {
  // Group consecutive streamable descriptors with the same (type, x type,
  // token-slot count) into launches of at most kSMaxMats matrices.
  int i = 0;
  while (i < count) {
    if (!streamable(d[i])) {
      hipError_t e = launch_gemv_general(d[i].W, d[i].qtype, d[i].n_rows, d[i].k, d[i].nb1, d[i].X, d[i].x_f16,
                                         d[i].n_tokens, d[i].Y, stream);
      if (e != hipSuccess) return e;
      ++i;
      continue;
    }
    SBatch B{};
    int x_bytes = 0;
    const int qt = d[i].qtype, nt = nt_slots(d[i].n_tokens);
    const bool xf = d[i].x_f16;
    int j = i, rg = 0;
    while (j < count && B.count < kSMaxMats && streamable(d[j]) && d[j].qtype == qt && d[j].x_f16 == xf &&
           nt_slots(d[j].n_tokens) == nt) {
      SMat &m = B.m[B.count++];
      m.W = static_cast<const uint8_t *>(d[j].W);
      m.X = d[j].X;
      m.Y = d[j].Y;
      m.nb1 = d[j].nb1;
      m.n_rows = static_cast<int>(d[j].n_rows);
      m.nblk = static_cast<int>(d[j].k / 32);
      m.n_tokens = static_cast<int>(d[j].n_tokens);
      m.k = static_cast<int>(d[j].k);
      rg += static_cast<int>((d[j].n_rows + 15) / 16);
      m.rg_end = rg;
      x_bytes = max(x_bytes, static_cast<int>(2 * d[j].k * nt));
      ++j;
    }
    B.total_rg = rg;
    for (int r = B.count; r < kSMaxMats; ++r) B.m[r].rg_end = rg;
    hipError_t e;
    if (qt == QMM_TYPE_Q4_0)
      e = xf ? s_nt<QMM_TYPE_Q4_0, true>(nt, B, x_bytes, stream) : s_nt<QMM_TYPE_Q4_0, false>(nt, B, x_bytes, stream);
    else
      e = xf ? s_nt<QMM_TYPE_Q8_0, true>(nt, B, x_bytes, stream) : s_nt<QMM_TYPE_Q8_0, false>(nt, B, x_bytes, stream);
    if (e != hipSuccess) return e;
    i = j;
  }
  return hipSuccess;
}

}  // namespace qmm
