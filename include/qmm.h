/*
 * qmm.h - C ABI of the block-quantized MUL_MAT library for AMD MI355X (gfx950).
 *
 * The library computes ggml's MUL_MAT of a GGUF block-quantized weight matrix
 * with fp32 (or fp16) activations, dequantising the blocks inside the
 * kernels. Sources, cited by page title and section:
 *
 *   [Bind]  "llama.cpp 源码分析：GGUF 权重与计算图的绑定", section 2.3
 *           "量化类型与数据布局": struct block_q4_0 { ggml_half d;
 *           uint8_t qs[16]; } holds 32 weights; ggml_nbytes depends on the
 *           type; blocks are read and dequantised inside MUL_MAT, then
 *           multiplied. Section 3.2: weights are created as {ne0 = k,
 *           ne1 = rows} (e.g. ffn_up {n_embd, n_ff}).
 *   [Arch]  "llama.cpp 源码完全拆解(一)：整体架构与模块全景", section
 *           "权重装载：GGUF、mmap 与 4 bit 块": block reconstruction
 *           w_hat = s (q - z); legacy types (Q4_0 ... Q8_0) use 32 weights per
 *           block with one shared scale, Q4_1 with an extra minimum offset
 *           (the paragraph on the three quantisation families); the
 *           quantised matmul kernels decode
 *           scale and integer weights per block and multiply-add them with the
 *           activations in registers, with no separate fp16 restore step.
 *   [Graph] "llama.cpp 源码完全拆解(二)：ggml 计算图与内存分配器", section
 *           "ggml_tensor：一个图节点的全部字段": nb[0] is the block size in
 *           bytes, nb[1] = nb[0] * (ne[0] / block_size) + padding, ne[0] is
 *           the contiguous dimension.
 *   [Load]  "llama.cpp 源码完全拆解(三)：GGUF 装载、mmap 与张量放置", section
 *           "第六步：能力校验": MUL_MAT takes F32 activations of shape
 *           [ne0, n_tokens] and backends use different kernels for one token
 *           and for many; section "校验": rows with NaN/Inf scales are
 *           rejected when a model is loaded.
 *
 * Data layout (all entry points):
 *   W  weights, n_rows rows; row r starts at W + r * row_stride_bytes and holds
 *      k / 32 consecutive blocks. Q4_0 block = 18 bytes: little-endian binary16
 *      d, then 16 bytes qs; element j (0..15) is the low nibble of qs[j],
 *      element j + 16 the high nibble; weight = d * (q - 8). Q4_1 block = 20
 *      bytes: binary16 d, binary16 m, then 16 bytes qs in Q4_0's nibble
 *      order; weight = d * q + m (unsigned codes; the layout of d, m and qs
 *      is this library's reading of the minimum-offset type). Q5_0 block = 22
 *      bytes: binary16 d, a little-endian 32-bit word whose bit j is the
 *      fifth bit of element j, then 16 bytes qs with the low four bits in
 *      Q4_0's nibble order; weight = d * (q - 16), codes 0..31. Q5_1 block =
 *      24 bytes: d, m, the fifth-bit word, qs; weight = d * q + m (the
 *      packing of both is this library's reading: the pages give none). Q8_0 block = 34
 *      bytes: binary16 d, then 32 int8 codes; weight = d * q. Q4_K (a k-quant:
 *      256-weight super-blocks with scales and minimums in two levels, [Arch]
 *      paragraph on the three quantisation families; a Q4_K row is k / 256
 *      blocks, [Graph]; the bit layout is this library's reading, the GGUF
 *      one) super-block = 144 bytes: binary16 d, binary16 dmin, 12 bytes of
 *      eight 6-bit sub-block scales sc_j and minimums m_j (j < 4: sc_j =
 *      s[j] & 63, m_j = s[j+4] & 63; j >= 4: sc_j = (s[j+4] & 15) |
 *      (s[j-4] >> 6) << 4, m_j = (s[j+4] >> 4) | (s[j] >> 6) << 4), then 128
 *      code bytes (byte 32c + l: element 64c + l in the low nibble, element
 *      64c + 32 + l in the high one); weight = d * sc_j * q - dmin * m_j.
 *      Q4_K needs k a multiple of 256, W 16-byte aligned, a row stride that
 *      is a multiple of 16 and a matrix under 4 GiB. Bytes between
 *      the last block of a row and the next row (padding) are never read.
 *   X  activations [n_tokens][k], k contiguous (fp32, or fp16 for *_x16).
 *   Y  output [n_tokens][n_rows] fp32, n_rows contiguous; fully overwritten.
 *
 * Ownership and asynchrony: every pointer is device memory owned by the
 * caller; the library keeps no reference after a call returns, allocates
 * nothing and holds no mutable global state, so calls on different streams
 * may run concurrently. Work is enqueued on `stream` (a hipStream_t; NULL is
 * the default stream) and the call returns without waiting. A fault inside a
 * kernel surfaces at the caller's next synchronisation. Y must not overlap W
 * or X.
 *
 * Errors: arguments are validated before anything is launched; a failing
 * check returns its negative status code and enqueues nothing. A launch that
 * HIP rejects returns QMM_ERR_HIP. qmm_status_string() names every code.
 *
 * Numerics: dequantised weights are exact (fp32 d * (q - z) is exact for every
 * finite binary16 d; the d * q + m of Q4_1 / Q5_1 is that exact product plus
 * m, rounded once to fp32; Q4_K's d sc q - dmin m is two exact products,
 * rounded once). The matmul accumulates in fp32. Decode-sized calls
 * (n_tokens <= QMM_GEMV_MAX_TOKENS) round activations to fp16 and multiply
 * them by the exact integer codes, applying d in fp32 once per block (Q4_1,
 * Q5_1: plus m times the block's sum of the fp16 activations); larger
 * calls round both the dequantised weights and the activations to fp16 for
 * the matrix cores. Every element satisfies
 *   |y - y_exact| <= 1e-3 * sum_i |w_i x_i| + 1e-5
 * when every activation is 0 or of magnitude in [2^-14, 65504] (the fp16
 * normal range) and, on the matrix-core path, every dequantised weight is 0
 * or in that range too (always so for Q4_0, Q5_0 and Q8_0 whose fp16 scale
 * is finite: their weights are exact in fp16 or rounded relatively). Below
 * 2^-14 fp16 rounding is absolute: activations add at most 2^-25 sum_i |w_i|
 * to the bound, and on the matrix-core path weights of Q4_1, Q5_1 and Q4_K
 * whose minimum nearly cancels d q add at most 2^-25 sum_i |x_i|. The
 * decode kernels' d sum(q x) + m sum(x) split of Q4_1, Q5_1 and Q4_K can
 * lose the bound's relative part in fp32 when both terms nearly cancel over
 * a whole block. Activations beyond 65504 overflow fp16: every output they
 * touch is non-finite. Scales d must be finite (the loader rejects NaN/Inf
 * scales); a non-finite d or x yields a non-finite result in every output it
 * touches.
 */
#ifndef QMM_H
#define QMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight types; the values follow ggml's type enumeration. */
#define QMM_TYPE_Q4_0 2
#define QMM_TYPE_Q4_1 3
#define QMM_TYPE_Q5_0 6
#define QMM_TYPE_Q5_1 7
#define QMM_TYPE_Q8_0 8
#define QMM_TYPE_Q4_K 12

/* Activation element types for qmm_matmul_path. */
#define QMM_X_F32 0
#define QMM_X_F16 1

/* Kernel choice for qmm_matmul_path. */
#define QMM_PATH_AUTO 0 /* decode kernel if n_tokens <= QMM_GEMV_MAX_TOKENS, else matrix-core kernel */
#define QMM_PATH_GEMV 1 /* decode kernel; n_tokens must be <= QMM_GEMV_MAX_TOKENS */
#define QMM_PATH_GEMM 2 /* matrix-core (MFMA) kernel; any n_tokens */

#define QMM_GEMV_MAX_TOKENS 8

/* Status codes. */
#define QMM_OK 0
#define QMM_ERR_NULL (-1)   /* a required pointer is NULL */
#define QMM_ERR_TYPE (-2)   /* unknown ggml_type or activation type */
#define QMM_ERR_SHAPE (-3)  /* k not a positive multiple of 32, negative or too large sizes */
#define QMM_ERR_STRIDE (-4) /* row_stride_bytes odd or smaller than the row's blocks */
#define QMM_ERR_ALIGN (-5)  /* pointer alignment requirement not met */
#define QMM_ERR_HIP (-6)    /* HIP reported an error for the launch */
#define QMM_ERR_PATH (-7)   /* unknown path, or GEMV forced with too many tokens */
#define QMM_ERR_WORKSPACE (-8) /* workspace NULL or smaller than the call needs */
#define QMM_ERR_SCRATCH (-9)   /* the call needs more scratch than qmm_matmul_id_noalloc holds */

/* Bytes of device scratch qmm_matmul_id_noalloc holds per GPU (1 MiB). */
#define QMM_NOALLOC_SCRATCH_BYTES 1048576

/*
 * qmm_matmul - Y = MUL_MAT(W, X) with fp32 activations ([Bind] section 2.3,
 * [Load] section 第六步, [Arch] section 权重装载).
 *   W                device pointer, 2-byte aligned, n_rows rows of
 *                    row_stride_bytes bytes (see layout above)
 *   ggml_type        QMM_TYPE_Q4_0, _Q4_1, _Q5_0, _Q5_1, _Q8_0 or _Q4_K
 *   n_rows           ne1 of W (>= 0)
 *   k                ne0 of W and of X; positive multiple of 32
 *   row_stride_bytes nb1 of W; even and >= qmm_row_bytes(ggml_type, k)
 *   X                device pointer, fp32 [n_tokens][k], 4-byte aligned
 *   n_tokens         ne1 of X (>= 0)
 *   Y                device pointer, fp32 [n_tokens][n_rows], 4-byte aligned
 *   stream           hipStream_t or NULL
 * n_rows == 0 or n_tokens == 0 returns QMM_OK and launches nothing. Sizes must
 * satisfy n_rows, n_tokens, k < 2^31, n_rows * row_stride_bytes <= 2^62 and
 * n_tokens * k, n_tokens * n_rows <= 2^60 (QMM_ERR_SHAPE otherwise, so every
 * byte count stays inside int64). Returns QMM_OK or a negative code.
 */
int qmm_matmul(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
               const float *X, int64_t n_tokens, float *Y, void *stream);

/*
 * qmm_matmul_x16 - as qmm_matmul, but X holds fp16 (IEEE binary16 bit
 * patterns) activations [n_tokens][k], 4-byte aligned.
 */
int qmm_matmul_x16(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
                   const uint16_t *X, int64_t n_tokens, float *Y, void *stream);

/*
 * qmm_matmul_path - as qmm_matmul with the activation type (x_type =
 * QMM_X_F32 or QMM_X_F16) and the kernel (path = QMM_PATH_*) chosen by the
 * caller. QMM_PATH_GEMV with n_tokens > QMM_GEMV_MAX_TOKENS returns
 * QMM_ERR_PATH. Meant for tests that compare the two kernels.
 */
int qmm_matmul_path(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
                    const void *X, int x_type, int64_t n_tokens, float *Y, int path, void *stream);

/*
 * qmm_matmul_workspace_bytes - device workspace qmm_matmul_ws needs for this
 * shape on the current device: 0 when the call runs as qmm_matmul_path with
 * QMM_PATH_AUTO, otherwise the bytes of its k split (counters and one
 * 128 KiB partial tile per part). The split is taken by fp16 activations of
 * at least 256 tokens, a 32-weight block type and an even block count, in
 * two cases: (1) the 128-row x 256-token tiles number at most half the
 * compute units and k is long enough for 2 to 4 parts per tile of at least
 * 32 stages of 64 (k >= 4096 for 2 parts); (2) the tiles number more than
 * the compute units and the last of their rounds would occupy at most half
 * of them (k >= 4096): that round's tiles run in 2 parts, the others whole.
 * Every other shape returns 0. Negative status for invalid sizes or types.
 */
int64_t qmm_matmul_workspace_bytes(int ggml_type, int64_t n_rows, int64_t k, int64_t n_tokens, int x_type);

/*
 * qmm_matmul_ws - the MUL_MAT of qmm_matmul_path (QMM_PATH_AUTO; the same
 * computation, [Bind] section 2.3) with a caller workspace that lets the
 * matrix-core kernel split k across workgroups where its tiles would leave
 * most compute units idle: few output tiles with a long k (e.g. a 4096-row
 * projection over k = 14336 at the 512-token batch of [Load] section
 * 第六步), or a last round of tiles that would leave half of them idle. A
 * split tile is summed as 2 to 4 partial sums over equal k ranges, added in
 * k order by the workgroup that finishes last; no workgroup waits for
 * another.
 *   W ... stream   as in qmm_matmul_path (x_type QMM_X_F32 or QMM_X_F16)
 *   workspace      device pointer, 16-byte aligned, at least
 *                  qmm_matmul_workspace_bytes(...) bytes, caller-owned; may
 *                  be NULL when that is 0. It must hold zeros when first
 *                  used (e.g. filled by hipMemset once); every call leaves
 *                  its counters at zero again, so one workspace serves any
 *                  later call enqueued after it. Calls that may run at the
 *                  same time need workspaces of their own.
 *   workspace_bytes its size
 * Returns QMM_ERR_WORKSPACE if the workspace is NULL or too small where one
 * is needed, QMM_ERR_ALIGN if it is misaligned, else as qmm_matmul_path.
 * Results are reproducible bit for bit for a given shape on a given device
 * (the split depends on the shape and the compute unit count) and may differ
 * in their last bits from qmm_matmul_x16's, within the same error bound.
 */
int qmm_matmul_ws(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
                  const void *X, int x_type, int64_t n_tokens, float *Y, void *workspace, int64_t workspace_bytes,
                  void *stream);

/* One MUL_MAT of a qmm_matmul_batch call; fields as in qmm_matmul_path. */
typedef struct qmm_matmul_desc {
  const void *W;
  int ggml_type;
  int64_t n_rows;
  int64_t k;
  int64_t row_stride_bytes;
  const void *X;
  int x_type; /* QMM_X_F32 or QMM_X_F16 */
  int64_t n_tokens;
  float *Y;
} qmm_matmul_desc;

/*
 * qmm_matmul_batch - `count` independent MUL_MATs enqueued on one stream, as
 * if each were passed to qmm_matmul_path with QMM_PATH_AUTO. A model issues
 * several MUL_MATs that share an input and do not depend on each other
 * ([Bind] section 3.2: a layer's attn_q/k/v, or ffn_gate and ffn_up); the
 * decode-sized ones (n_tokens <= QMM_GEMV_MAX_TOKENS) with 16-byte-aligned
 * layouts are grouped into shared launches, which removes the per-launch
 * fixed cost that dominates small decode matmuls. Many-token ones with fp16
 * activations and the same type, rows, k, row stride and token count (up to
 * 4 together) share one matrix-core launch where its tiles suit the
 * two-group kernel, so the MUL_MATs fill its rounds together. `descs` is a host array
 * read only during the call. Every descriptor is validated before anything is
 * launched; on failure the status of the first invalid descriptor is
 * returned and nothing is enqueued. Outputs must not overlap any input or
 * each other. Results are reproducible for a given batch; a MUL_MAT in a batch
 * may differ in its last bits from the same MUL_MAT called alone, because the
 * decode kernel splits k according to the size of its launch, and a shared
 * matrix-core launch may take the two-group kernel where a lone call takes
 * the one-group kernel with its k split inside the workgroup (both are
 * within the stated error bound). count == 0 is a no-op; count < 0 or
 * descs == NULL with count > 0 returns QMM_ERR_SHAPE / QMM_ERR_NULL.
 */
int qmm_matmul_batch(const qmm_matmul_desc *descs, int count, void *stream);

/*
 * qmm_matmul_batch_workspace_bytes - device workspace qmm_matmul_batch_ws
 * needs for these descriptors on the current device: the largest k split
 * of its matrix-core launches (as qmm_matmul_workspace_bytes, over the
 * tiles of a shared launch), 0 if none splits. Negative status for an
 * invalid descriptor (as qmm_matmul_batch).
 */
int64_t qmm_matmul_batch_workspace_bytes(const qmm_matmul_desc *descs, int count);

/*
 * qmm_matmul_batch_ws - qmm_matmul_batch with a caller workspace that lets
 * its matrix-core launches split k as qmm_matmul_ws does ([Bind] section
 * 3.2 for the independent MUL_MATs of a layer; [Bind] section 2.3 for each
 * one). For ffn_gate and ffn_up of 11008 x 4096 at 2048 tokens, the shared
 * launch has 1376 tiles: five full rounds on 256 compute units and a sixth
 * of 96 tiles, which run in two halves of k on 192 of them.
 *   descs, count, stream  as in qmm_matmul_batch
 *   workspace      device pointer, 16-byte aligned, at least
 *                  qmm_matmul_batch_workspace_bytes(descs, count) bytes,
 *                  caller-owned, zero when first used, left at zero by every
 *                  call (as for qmm_matmul_ws); may be NULL when that is 0.
 *                  The launches of one call run in order on the stream and
 *                  share it. Calls that may run at the same time need
 *                  workspaces of their own.
 *   workspace_bytes its size
 * Returns QMM_ERR_WORKSPACE if the workspace is NULL or too small where one
 * is needed, QMM_ERR_ALIGN if it is misaligned, else as qmm_matmul_batch.
 * Results repeat bit for bit for given descriptors on a given device; split
 * tiles may differ in their last bits from qmm_matmul_batch's, within the
 * same error bound.
 */
int qmm_matmul_batch_ws(const qmm_matmul_desc *descs, int count, void *workspace, int64_t workspace_bytes,
                        void *stream);

/*
 * qmm_dequantize - the block decoder alone ([Bind] section 2.3 layout,
 * [Arch] reconstruction equation): out[r][i] = fp32(d) * fp32(q - z) for
 * element i of row r. out is fp32 [n_rows][k], 4-byte aligned, caller-owned.
 * The result is bit-exact (NaN scales give NaN). n_rows == 0 is a no-op.
 * Sizes as in qmm_matmul, with n_rows * k <= 2^60.
 */
int qmm_dequantize(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
                   float *out, void *stream);

/*
 * qmm_get_rows - GET_ROWS on a quantised weight: out[i][j] = the dequantised
 * element j of row ids[i] of W, bit-exact as in qmm_dequantize (the op the
 * capability probe builds for token-embedding tensors with an I32 index
 * vector, [Load] section 第六步).
 *   W, ggml_type, n_rows, k, row_stride_bytes  as in qmm_matmul
 *   ids      device pointer, int32 [n_ids], 4-byte aligned, caller-owned
 *   n_ids    number of rows to gather (>= 0, n_ids * k <= 2^60; 0 is a no-op)
 *   out      device pointer, fp32 [n_ids][k], 4-byte aligned, caller-owned
 *   stream   hipStream_t or NULL
 * An index outside [0, n_rows) cannot be checked on the host (ids are device
 * data): its output row is filled with quiet NaNs and nothing is read for it.
 * Returns QMM_OK, or the status of the first failed check (QMM_ERR_NULL,
 * _TYPE, _SHAPE, _STRIDE, _ALIGN) without launching, or QMM_ERR_HIP.
 */
int qmm_get_rows(const void *W, int ggml_type, int64_t n_rows, int64_t k, int64_t row_stride_bytes,
                 const int32_t *ids, int64_t n_ids, float *out, void *stream);

/*
 * qmm_matmul_id - MUL_MAT_ID, the expert-routed MUL_MAT that serves MoE
 * expert routing (and adapter routing): for every token t and slot i,
 *   Y[t][i][r] = sum_j dequant(W_e)[r][j] * X[t][s][j],  e = ids[t][i],
 * with s = i when x_slots == n_ids and s = 0 when x_slots == 1 (one
 * activation row shared by all slots). This is the op the capability probe
 * builds with activations F32 [k, n_ids, tokens] and ids I32 [n_ids, tokens]
 * ([Load] section 第六步, the GGML_OP_MUL_MAT_ID case).
 *   W                    device pointer to n_experts matrices, each n_rows rows
 *                        of row_stride_bytes, expert e at e * expert_stride_bytes
 *                        (2-byte aligned, caller-owned, read only)
 *   ggml_type, k, row_stride_bytes  as in qmm_matmul
 *   n_experts            matrices in the stack (>= 0)
 *   expert_stride_bytes  even, >= n_rows * row_stride_bytes
 *   X                    device pointer, fp32 [n_tokens][x_slots][k], 4-byte aligned
 *   x_slots              1 or n_ids
 *   ids                  device pointer, int32 [n_tokens][n_ids], 4-byte aligned
 *   n_ids, n_tokens      >= 0, n_ids * n_tokens < 2^31; 0 is a no-op
 *                        (also n_experts * expert_stride_bytes <= 2^62 and
 *                        n_tokens * x_slots * k, n_tokens * n_ids * n_rows
 *                        <= 2^60, else QMM_ERR_SHAPE)
 *   Y                    device pointer, fp32 [n_tokens][n_ids][n_rows], 4-byte aligned
 *   workspace            device scratch of at least
 *                        qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens)
 *                        bytes, 4-byte aligned, caller-owned; may be NULL when
 *                        that size is 0. Its contents are overwritten; two
 *                        calls in flight must not share one.
 *   stream               hipStream_t or NULL
 * The route follows from the sizes alone (at most 4096 experts for the
 * grouped ones, which first bucket the pairs by expert in the workspace):
 * one token, or about one pair per selected expert: every pair is a
 * single-token product on the decode kernels; more than QMM_GEMV_MAX_TOKENS
 * tokens and at least 4 pairs per expert on average: a matrix-core kernel
 * runs tiles of pairs of one expert (128 per tile, or 160 on the two-group
 * kernel when the workspace also holds the fp16 copy of X, see
 * qmm_matmul_id_workspace_bytes_x16); otherwise the streaming decode
 * kernel runs tiles of 2, 4 or 8 pairs of one expert (the per-pair route
 * when the weights do not have the streaming layout: 16-byte aligned W,
 * row and expert strides, k a multiple of 256). Results do not depend on the route's tile order. An id outside
 * [0, n_experts) cannot be checked on the host: that pair's output row is
 * filled with quiet NaNs and nothing is read for it.
 * Returns QMM_OK, or the status of the first failed check (QMM_ERR_NULL,
 * _TYPE, _SHAPE, _STRIDE, _ALIGN, _WORKSPACE) without launching, or
 * QMM_ERR_HIP.
 */
int qmm_matmul_id(const void *W, int ggml_type, int64_t n_experts, int64_t n_rows, int64_t k,
                  int64_t row_stride_bytes, int64_t expert_stride_bytes, const float *X, int64_t x_slots,
                  const int32_t *ids, int64_t n_ids, int64_t n_tokens, float *Y, void *workspace,
                  int64_t workspace_bytes, void *stream);

/*
 * qmm_matmul_id_noalloc - qmm_matmul_id for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same routes, kernels and results,
 * but the routing table of the grouped routes lives in a device array of
 * QMM_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, so the call takes no workspace and calls no
 * allocator. Its address is looked up (hipGetSymbolAddress) on the first
 * call on each device, with that device current.
 *   Arguments: as qmm_matmul_id, without workspace and workspace_bytes.
 *   Scratch: the array is shared by every call on the same GPU and keeps the
 *   last call's contents (each call rewrites every entry it reads, so
 *   nothing has to start at zero); calls that overlap on one GPU (on
 *   different streams, or from different threads) race on it and must not
 *   be issued.
 * Returns QMM_OK, or the status of the first failed check (as qmm_matmul_id;
 * QMM_ERR_SCRATCH when qmm_matmul_id_workspace_bytes(n_experts, n_ids,
 * n_tokens) exceeds QMM_NOALLOC_SCRATCH_BYTES) without launching, or
 * QMM_ERR_HIP (also when the scratch address cannot be obtained).
 */
int qmm_matmul_id_noalloc(const void *W, int ggml_type, int64_t n_experts, int64_t n_rows, int64_t k,
                          int64_t row_stride_bytes, int64_t expert_stride_bytes, const float *X, int64_t x_slots,
                          const int32_t *ids, int64_t n_ids, int64_t n_tokens, float *Y, void *stream);

/*
 * qmm_matmul_id_workspace_bytes - the workspace qmm_matmul_id needs for these
 * sizes (0 when the call takes the per-pair route), or QMM_ERR_SHAPE for
 * negative or too large sizes.
 */
int64_t qmm_matmul_id_workspace_bytes(int64_t n_experts, int64_t n_ids, int64_t n_tokens);

/*
 * qmm_matmul_id_workspace_bytes_x16 - the workspace with which qmm_matmul_id
 * takes its fastest route for these sizes: for the matrix-core route, the
 * routing table plus an fp16 copy of X (n_tokens * x_slots * k * 2 bytes),
 * from which a kernel that runs two tiles of 128 pairs per workgroup copies
 * activations straight into LDS when the call has enough tiles to fill the
 * GPU; otherwise the same as qmm_matmul_id_workspace_bytes. A call given at
 * least qmm_matmul_id_workspace_bytes but fewer than these bytes takes the
 * one-tile kernel, which reads X in fp32; both round X to fp16 the same way
 * and add the same products in the same order, so the result is the same
 * bits. QMM_ERR_SHAPE for negative or too large sizes, k <= 0, or x_slots
 * other than 1 or n_ids.
 */
int64_t qmm_matmul_id_workspace_bytes_x16(int64_t n_experts, int64_t n_ids, int64_t n_tokens, int64_t k,
                                          int64_t x_slots);

/*
 * qmm_row_bytes - the dense row stride (k / 32) * block bytes, i.e. nb[1]
 * without padding ([Graph] ggml_tensor stride comment). Negative status code
 * for an unknown type or a k that is not a positive multiple of 32.
 */
int64_t qmm_row_bytes(int ggml_type, int64_t k);

/*
 * qmm_supports - 1 if (ggml_type, k, row_stride_bytes) is a weight layout the
 * library accepts, else 0 (the role a backend's supports_op query plays for
 * MUL_MAT in [Load] section 第六步). Pointer alignment is checked per call.
 */
int qmm_supports(int ggml_type, int64_t k, int64_t row_stride_bytes);

/* qmm_status_string - a static, human-readable name for a status code. */
const char *qmm_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
