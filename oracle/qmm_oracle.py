"""Plain CPU oracle for block-quantized MUL_MAT on GGUF Q4_0 / Q4_1 / Q5_0 / Q5_1 /
Q8_0 weights.

TEST INFRASTRUCTURE. Only the tests, the package entry point's smoke check and
the benchmark's CPU-baseline leg may import this module. The library never
calls it, links it or shares code with it: it is the independent definition
the HIP kernels are checked against. It is deliberately plain and slow.

Sources (the pages are cited by title and section):
  [Bind]  "llama.cpp 源码分析：GGUF 权重与计算图的绑定" (yeyulingfeng.com),
          section 2.3 "量化类型与数据布局" (the block_q4_0 struct and the
          remark that blocks are dequantised inside MUL_MAT), section 3.2
          "load_tensors()" (weight shapes {ne0 = k, ne1 = rows}).
  [Arch]  "llama.cpp 源码完全拆解(一)：整体架构与模块全景" (pinghaoyang.com.cn),
          section "权重装载：GGUF、mmap 与 4 bit 块": the uniform block
          quantisation equation q(w) = clip(round(w/s) + z, qmin, qmax) with
          reconstruction w_hat = s (q - z), the error-variance equation, the
          legacy-family paragraph (32 weights per block, one shared scale,
          Q4_1 with an extra minimum offset) and the quality table (Q8_0
          row: 46.87 % smaller than F16).
  [Graph] "llama.cpp 源码完全拆解(二)：ggml 计算图与内存分配器", section
          "ggml_tensor：一个图节点的全部字段" (nb[0] = block bytes,
          nb[1] = nb[0] * ne[0] / block_size + padding, ne[0] contiguous).
  [Load]  "llama.cpp 源码完全拆解(三)：GGUF 装载、mmap 与张量放置", section
          "第六步：能力校验" (the MUL_MAT probe takes F32 activations of shape
          [ne0, 512]) and section "校验：--check-tensors 与并行验证" (rows with
          NaN/Inf scales are rejected when a model is loaded).

Readings taken where the pages are silent (also listed in the design notes):
  * Q4_0 nibble order: low nibble of code byte j is element j, high nibble is
    element j + 16.
  * Q4_0 zero point z = 8 with 4-bit codes 0..15, so w = d * (q - 8); Q8_0 has
    z = 0 and signed int8 codes, so w = d * q.
  * Q8_0 block = fp16 d followed by 32 int8 codes (34 bytes); 34/32 bytes per
    weight is exactly the table's 46.87 % reduction versus 16-bit weights.
  * Q4_1 block = fp16 d, fp16 m (the minimum offset), then the 16 code
    bytes in Q4_0's nibble order (20 bytes); 4-bit codes 0..15 with
    w = d * q + m, the reconstruction with the stored minimum in place of
    the zero point.
  * Q5_0 / Q5_1 (legacy types with 5-bit codes; the pages give neither the
    packing nor the field order): d (and, for Q5_1, m as in Q4_1), then a
    32-bit little-endian word whose bit j is the fifth bit of element j,
    then the 16 nibble bytes in Q4_0's order holding the low four bits.
    Codes 0..31; Q5_0 has z = 16 (w = d * (q - 16)), Q5_1 w = d * q + m.
  * Q4_K (a k-quant; [Arch] says k-quants use 256-weight blocks with scales
    and minimums stored in two levels, 6-bit upper and 4-bit lower, and
    [Graph]/[Load] size a Q4_K tensor as ne[0] / 256 blocks; the bit layout
    is not printed, so this is the GGUF layout taken as a reading): a
    144-byte super-block of 256 weights = binary16 d, binary16 dmin, 12
    bytes holding eight 6-bit sub-block scales sc_j and minimums m_j, then
    128 code bytes. Scale bytes s[0..11]: for j < 4, sc_j = s[j] & 63 and
    m_j = s[j + 4] & 63; for j >= 4, sc_j = (s[j + 4] & 15) | (s[j - 4] >> 6) << 4
    and m_j = (s[j + 4] >> 4) | (s[j] >> 6) << 4. Code byte 32 c + l holds
    element 64 c + l (sub-block 2 c) in its low nibble and element
    64 c + 32 + l (sub-block 2 c + 1) in its high nibble. Weight of element i
    of sub-block j: w = d * sc_j * q_i - dmin * m_j, rounded once to fp32
    (both products are exact).
  * The scale d (and m) is stored little-endian as IEEE-754 binary16.
  * Activations X are [n_tokens][k] with k contiguous; Y is [n_tokens][n_rows]
    with rows contiguous, fully overwritten.
  * Dequantisation is to fp32 (the product d * (q - z) is exact in fp32 for
    every finite binary16 d and every code); the dot products are
    accumulated in fp64 here.

Parity pins live in tests/test_oracle_pins.py and tests/test_q4_k_pins.py. No function here
is unpinned.
"""
from __future__ import annotations

import numpy as np

# Type ids follow ggml's enumeration (the pages name the types, not the ids).
TYPE_Q4_0 = 2
TYPE_Q4_1 = 3
TYPE_Q5_0 = 6
TYPE_Q5_1 = 7
TYPE_Q8_0 = 8
TYPE_Q4_K = 12

QK = 32  # weights per block of the legacy types ([Arch] legacy-family paragraph)
QK_K = 256  # weights per k-quant super-block ([Arch] k-quants: block size raised to 256)

BLOCK_BYTES = {
    TYPE_Q4_0: 2 + QK // 2,      # ggml_half d + uint8_t qs[16]  ([Bind] section 2.3)
    TYPE_Q4_1: 2 + 2 + QK // 2,  # d, the minimum m, qs[16]      (reading, see header)
    TYPE_Q5_0: 2 + 4 + QK // 2,  # d, qh (fifth bits), qs[16]    (reading, see header)
    TYPE_Q5_1: 2 + 2 + 4 + QK // 2,  # d, m, qh, qs[16]          (reading, see header)
    TYPE_Q8_0: 2 + QK,           # ggml_half d + int8 qs[32]     (reading, see header)
    TYPE_Q4_K: 2 + 2 + 12 + QK_K // 2,  # d, dmin, 6-bit scales/mins, 4-bit codes (per 256; reading)
}
# weights per block (the block that BLOCK_BYTES describes)
BLOCK_WEIGHTS = {TYPE_Q4_0: QK, TYPE_Q4_1: QK, TYPE_Q5_0: QK, TYPE_Q5_1: QK, TYPE_Q8_0: QK, TYPE_Q4_K: QK_K}

ZERO_POINT = {TYPE_Q4_0: 8, TYPE_Q4_1: 0, TYPE_Q5_0: 16, TYPE_Q5_1: 0, TYPE_Q8_0: 0}
CODE_RANGE = {TYPE_Q4_0: (0, 15), TYPE_Q4_1: (0, 15), TYPE_Q5_0: (0, 31), TYPE_Q5_1: (0, 31),
              TYPE_Q8_0: (-128, 127)}
HAS_MIN = {TYPE_Q4_0: False, TYPE_Q4_1: True, TYPE_Q5_0: False, TYPE_Q5_1: True, TYPE_Q8_0: False}
# byte offset of the 32-bit fifth-bit word (types with 5-bit codes)
QH_OFFSET = {TYPE_Q5_0: 2, TYPE_Q5_1: 4}
# bytes before the code bytes: d, m where the type has one, qh where it has one
CODE_OFFSET = {TYPE_Q4_0: 2, TYPE_Q4_1: 4, TYPE_Q5_0: 6, TYPE_Q5_1: 8, TYPE_Q8_0: 2}
NIBBLE_TYPES = (TYPE_Q4_0, TYPE_Q4_1, TYPE_Q5_0, TYPE_Q5_1)


# --------------------------------------------------------------------------
# IEEE-754 binary16 -> real number, written out from the format's definition.
# --------------------------------------------------------------------------
def half_bits_to_double(bits) -> np.ndarray:
    """Value of each binary16 bit pattern, as float64 (always exact).

    sign s = bit 15, exponent e = bits 14..10, fraction m = bits 9..0:
      e == 0        -> (-1)^s * m * 2^-24            (zero and subnormals)
      1 <= e <= 30  -> (-1)^s * (1024 + m) * 2^(e-25) (normal numbers)
      e == 31       -> (-1)^s * inf if m == 0, else NaN
    """
    b = np.asarray(bits, dtype=np.uint32) & 0xFFFF
    s = (b >> 15) & 1
    e = ((b >> 10) & 0x1F).astype(np.int64)
    m = (b & 0x3FF).astype(np.float64)
    sign = np.where(s == 1, -1.0, 1.0)
    sub = m * np.ldexp(1.0, -24)
    nrm = np.ldexp(1024.0 + m, np.clip(e - 25, -24, 5))
    special = np.where(m == 0.0, np.inf, np.nan)
    mag = np.where(e == 0, sub, np.where(e == 31, special, nrm))
    return sign * mag


def row_bytes(qtype: int, k: int) -> int:
    """Dense row stride nb[1] without padding: (k / block weights) blocks of
    nb[0] bytes ([Graph] ggml_tensor stride comment; [Bind] section 2.3 on
    ggml_nbytes; for Q4_K, ne[0] / 256 blocks as [Graph] and [Load] state)."""
    if qtype not in BLOCK_BYTES:
        raise ValueError(f"unsupported type {qtype}")
    bw = BLOCK_WEIGHTS[qtype]
    if k <= 0 or k % bw:
        raise ValueError(f"k must be a positive multiple of {bw}")
    return (k // bw) * BLOCK_BYTES[qtype]


def _check_layout(W: np.ndarray, qtype: int, n_rows: int, k: int, nb1: int) -> np.ndarray:
    W = np.asarray(W, dtype=np.uint8)
    dense = row_bytes(qtype, k)
    if nb1 < dense:
        raise ValueError("row stride smaller than the row's blocks")
    if W.ndim != 2 or W.shape[0] != n_rows or W.shape[1] != nb1:
        raise ValueError(f"W must be uint8 [{n_rows}][{nb1}], got {W.shape}")
    return W


# --------------------------------------------------------------------------
# Block decoder ([Bind] section 2.3 struct; [Arch] reconstruction equation).
# --------------------------------------------------------------------------
def block_scales_and_codes(W, qtype: int, n_rows: int, k: int, nb1: int):
    """Split every block of every row into (d as float64, integer codes q).

    Returns d with shape [n_rows, k/32] and q with shape [n_rows, k] (int64),
    where q[r, 32*b + i] is the code of element i of block b. Padding bytes
    beyond the row's blocks are never looked at.
    """
    W = _check_layout(W, qtype, n_rows, k, nb1)
    nblk = k // QK
    bpb = BLOCK_BYTES[qtype]
    blocks = W[:, : nblk * bpb].reshape(n_rows, nblk, bpb)
    d_bits = blocks[:, :, 0].astype(np.uint32) | (blocks[:, :, 1].astype(np.uint32) << 8)
    d = half_bits_to_double(d_bits)
    payload = blocks[:, :, CODE_OFFSET[qtype]:]
    if qtype in NIBBLE_TYPES:
        low = (payload & 0x0F).astype(np.int64)   # element j      <- low nibble of byte j
        high = (payload >> 4).astype(np.int64)    # element j + 16 <- high nibble of byte j
        q = np.concatenate([low, high], axis=2)   # [n_rows, nblk, 32]
        if qtype in QH_OFFSET:
            o = QH_OFFSET[qtype]
            qh = np.zeros((n_rows, nblk), dtype=np.int64)
            for b in range(4):                    # little-endian 32-bit word
                qh |= blocks[:, :, o + b].astype(np.int64) << (8 * b)
            bits = (qh[:, :, None] >> np.arange(32)) & 1   # bit j: fifth bit of element j
            q = q | (bits << 4)
    else:
        q = payload.view(np.int8).astype(np.int64)
    return d, q.reshape(n_rows, k)


def block_mins(W, qtype: int, n_rows: int, k: int, nb1: int) -> np.ndarray:
    """The minimum offset m of every block (float64 [n_rows, k/32]): the
    binary16 after d in a Q4_1 or Q5_1 block; zero for types without one."""
    W = _check_layout(W, qtype, n_rows, k, nb1)
    nblk = k // QK
    if not HAS_MIN[qtype]:
        return np.zeros((n_rows, nblk))
    bpb = BLOCK_BYTES[qtype]
    blocks = W[:, : nblk * bpb].reshape(n_rows, nblk, bpb)
    m_bits = blocks[:, :, 2].astype(np.uint32) | (blocks[:, :, 3].astype(np.uint32) << 8)
    return half_bits_to_double(m_bits)


def dequantize(W, qtype: int, n_rows: int, k: int, nb1: int) -> np.ndarray:
    """Weights as fp32 [n_rows][k]: w = fp32(d) * fp32(q - z), plus fp32(m)
    for the types with a minimum (Q4_1, Q5_1).

    z = 8 for Q4_0, 16 for Q5_0 and 0 otherwise. The multiply is a single
    IEEE fp32 multiply; for finite d it is exact (an 11-bit significand
    times a code of at most 8 bits). Q4_1 / Q5_1 then add m with one fp32
    rounding, so w = fp32(d q + m) exactly rounded. This is the bit-exact
    target.
    """
    if qtype == TYPE_Q4_K:
        return dequantize_q4_k(W, n_rows, k, nb1)
    d, q = block_scales_and_codes(W, qtype, n_rows, k, nb1)
    c = (q - ZERO_POINT[qtype]).astype(np.float32)
    d32 = np.repeat(d.astype(np.float32), QK, axis=1)
    with np.errstate(invalid="ignore", over="ignore"):
        w = d32 * c
        if HAS_MIN[qtype]:
            w = w + np.repeat(block_mins(W, qtype, n_rows, k, nb1).astype(np.float32), QK, axis=1)
        return w


# --------------------------------------------------------------------------
# Q4_K super-blocks (reading of [Arch]'s k-quant description; see header).
# --------------------------------------------------------------------------
def q4_k_unpack_scales(s) -> tuple:
    """Eight 6-bit sub-block scales and minimums from the 12 scale bytes
    (uint8 [..., 12]) -> (sc, m), each int64 [..., 8]."""
    s = np.asarray(s, dtype=np.int64)
    sc = np.empty(s.shape[:-1] + (8,), dtype=np.int64)
    m = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = s[..., j] & 63
        m[..., j] = s[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
        m[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return sc, m


def q4_k_fields(W, n_rows: int, k: int, nb1: int) -> tuple:
    """Split every Q4_K super-block into (d, dmin) as float64 [n_rows, k/256],
    (sc, m) as int64 [n_rows, k/256, 8] and the codes q as int64
    [n_rows, k/256, 256] in element order."""
    W = _check_layout(W, TYPE_Q4_K, n_rows, k, nb1)
    nsb = k // QK_K
    blocks = W[:, : nsb * 144].reshape(n_rows, nsb, 144)
    d = half_bits_to_double(blocks[:, :, 0].astype(np.uint32) | (blocks[:, :, 1].astype(np.uint32) << 8))
    dmin = half_bits_to_double(blocks[:, :, 2].astype(np.uint32) | (blocks[:, :, 3].astype(np.uint32) << 8))
    sc, m = q4_k_unpack_scales(blocks[:, :, 4:16])
    qs = blocks[:, :, 16:].reshape(n_rows, nsb, 4, 32).astype(np.int64)
    # chunk c: elements 64 c .. 64 c + 31 in the low nibbles, 64 c + 32 .. in the high ones
    q = np.concatenate([qs & 15, qs >> 4], axis=3).reshape(n_rows, nsb, 256)
    return d, dmin, sc, m, q


def dequantize_q4_k(W, n_rows: int, k: int, nb1: int) -> np.ndarray:
    """Q4_K weights as fp32 [n_rows][k]: w = fp32(d * sc_j * q - dmin * m_j),
    the exact value (products of binary16 numbers with small integers, exact
    in fp64) rounded once."""
    d, dmin, sc, m, q = q4_k_fields(W, n_rows, k, nb1)
    j = np.arange(256) // 32                           # sub-block of each element
    with np.errstate(invalid="ignore", over="ignore"):
        w = d[:, :, None] * sc[:, :, j] * q - dmin[:, :, None] * m[:, :, j]
        return w.reshape(n_rows, k).astype(np.float32)


def q4_k_pack(d_bits, dmin_bits, sc, m, q) -> np.ndarray:
    """Lay out Q4_K super-blocks from binary16 d and dmin (uint16 [rows, nsb]),
    6-bit sc and m (int [rows, nsb, 8]) and 4-bit codes (int [rows, nsb, 256]
    in element order): uint8 [rows, nsb * 144]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    dmin_bits = np.asarray(dmin_bits, dtype=np.uint16)
    sc = np.asarray(sc, dtype=np.int64)
    m = np.asarray(m, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    rows, nsb = d_bits.shape
    out = np.zeros((rows, nsb, 144), dtype=np.uint8)
    out[:, :, 0], out[:, :, 1] = d_bits & 0xFF, d_bits >> 8
    out[:, :, 2], out[:, :, 3] = dmin_bits & 0xFF, dmin_bits >> 8
    s = np.zeros((rows, nsb, 12), dtype=np.int64)
    for j in range(4):
        s[:, :, j] |= sc[:, :, j] & 63
        s[:, :, j + 4] |= m[:, :, j] & 63
    for j in range(4, 8):
        s[:, :, j + 4] |= (sc[:, :, j] & 15) | ((m[:, :, j] & 15) << 4)
        s[:, :, j - 4] |= (sc[:, :, j] >> 4) << 6
        s[:, :, j] |= (m[:, :, j] >> 4) << 6
    out[:, :, 4:16] = s.astype(np.uint8)
    qc = q.reshape(rows, nsb, 4, 2, 32)
    out[:, :, 16:] = ((qc[:, :, :, 0, :] & 15) | ((qc[:, :, :, 1, :] & 15) << 4)).reshape(rows, nsb, 128)
    return out.reshape(rows, nsb * 144)


def q4_k_quantize_codes(w, d, dmin, sc, m) -> np.ndarray:
    """Test quantiser for given super-block fields: q = clip(round((w + dmin m_j)
    / (d sc_j)), 0, 15) (round half away from zero; q = 0 where d sc_j = 0).
    w is float [rows, nsb, 256]; returns int64 codes of the same shape."""
    w = np.asarray(w, dtype=np.float64)
    j = np.arange(256) // 32
    step = np.asarray(d, np.float64)[:, :, None] * np.asarray(sc, np.float64)[:, :, j]
    off = np.asarray(dmin, np.float64)[:, :, None] * np.asarray(m, np.float64)[:, :, j]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(step != 0.0, _round_half_away((w + off) / np.where(step != 0.0, step, 1.0)), 0.0)
    return np.clip(r, 0, 15).astype(np.int64)


def get_rows(W, qtype: int, n_rows: int, k: int, nb1: int, ids) -> np.ndarray:
    """GET_ROWS on a quantised weight: fp32 [len(ids)][k], row i = the
    dequantised row ids[i] of W ([Load] section "第六步：能力校验": the op
    built for a weight with an I32 index vector). An index outside
    [0, n_rows) has no row to take; its output row is NaN (the library's
    documented reading, since device-side indices cannot be validated).
    """
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    out = np.full((ids.size, k), np.nan, dtype=np.float32)
    ok = (ids >= 0) & (ids < n_rows)
    if n_rows > 0 and ok.any():
        out[ok] = dequantize(W, qtype, n_rows, k, nb1)[ids[ok]]
    return out


def _activations_f64(X, k: int) -> np.ndarray:
    X = np.asarray(X)
    if X.dtype not in (np.float32, np.float16):
        raise ValueError("activations must be float32 or float16")
    if X.ndim != 2 or X.shape[1] != k:
        raise ValueError(f"X must be [n_tokens][{k}]")
    return X.astype(np.float64)  # widening is exact


def matmul(W, qtype: int, n_rows: int, k: int, nb1: int, X):
    """MUL_MAT of quantised W [n_rows][k] with activations X [n_tokens][k].

    Returns (y, s), both float64 [n_tokens][n_rows]:
      y[t][r] = sum_i w[r][i] * x[t][i]
      s[t][r] = sum_i |w[r][i] * x[t][i]|   (scale of the rounding tolerance)
    with w the fp32 dequantised weights, everything widened to fp64, and the
    sums taken by a library fp64 matrix product.
    """
    Wd = dequantize(W, qtype, n_rows, k, nb1).astype(np.float64)
    X64 = _activations_f64(X, k)
    with np.errstate(invalid="ignore", over="ignore"):
        y = X64 @ Wd.T
        s = np.abs(X64) @ np.abs(Wd).T
    return y, s


def matmul_id(W, qtype: int, n_experts: int, n_rows: int, k: int, nb1: int, nb2: int, X, ids):
    """MUL_MAT_ID: expert-routed MUL_MAT ([Load] section "第六步：能力校验":
    ggml_mul_mat_id(ctx, w, b, ids) with w the stacked experts, b F32
    [ne0 = k, n_ids_used, n_tokens] and ids I32 [n_ids_used, n_tokens]).

    W  : uint8 [n_experts][nb2]; expert e's row r starts at byte r * nb1 of
         W[e] (nb2 >= n_rows * nb1).
    X  : [n_tokens][x_slots][k], x_slots = n_ids (one activation row per
         selected expert, the pages' shape) or 1 (one row shared by all).
    ids: int [n_tokens][n_ids].
    Returns (y, s), float64 [n_tokens][n_ids][n_rows]: for token t and slot i
    the MUL_MAT of expert ids[t][i] with X[t][i] (or X[t][0]). An id outside
    [0, n_experts) selects no expert; its row is NaN (the library's reading).
    """
    ids = np.asarray(ids, dtype=np.int64)
    X = np.asarray(X)
    n_tokens, n_ids = ids.shape
    if X.ndim != 3 or X.shape[0] != n_tokens or X.shape[1] not in (1, n_ids) or X.shape[2] != k:
        raise ValueError("X must be [n_tokens][1 or n_ids][k]")
    W = np.asarray(W, dtype=np.uint8)
    if W.shape != (n_experts, nb2) or nb2 < n_rows * nb1:
        raise ValueError("W must be [n_experts][nb2] with nb2 >= n_rows * nb1")
    y = np.full((n_tokens, n_ids, n_rows), np.nan)
    s = np.full((n_tokens, n_ids, n_rows), np.nan)
    for t in range(n_tokens):
        for i in range(n_ids):
            e = ids[t, i]
            if not 0 <= e < n_experts:
                continue
            We = W[e, :n_rows * nb1].reshape(n_rows, nb1)
            xr = X[t, i if X.shape[1] > 1 else 0].reshape(1, k)
            yt, st = matmul(We, qtype, n_rows, k, nb1, xr)
            y[t, i], s[t, i] = yt[0], st[0]
    return y, s


def matmul_sampled(W, qtype: int, n_rows: int, k: int, nb1: int, X, tokens, rows):
    """y and s for the listed (token, row) pairs only, each as a plain fp64
    dot product of one dequantised row with one activation row."""
    X64 = _activations_f64(X, k)
    tokens = np.asarray(tokens, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    W = _check_layout(W, qtype, n_rows, k, nb1)
    uniq, inv = np.unique(rows, return_inverse=True)
    Wd = dequantize(W[uniq], qtype, len(uniq), k, nb1).astype(np.float64)
    y = np.empty(len(rows))
    s = np.empty(len(rows))
    with np.errstate(invalid="ignore", over="ignore"):
        for n, (t, j) in enumerate(zip(tokens, inv)):
            p = Wd[j] * X64[t]
            y[n] = np.sum(p)
            s[n] = np.sum(np.abs(p))
    return y, s


def within_tolerance(y, y_ref, s, rel: float = 1e-3, abs_: float = 1e-5) -> np.ndarray:
    """Element-wise acceptance of a result y against the oracle's (y_ref, s).

      y_ref NaN        -> y must be NaN;
      y_ref +/-inf     -> y must be the infinity of the same sign;
      y_ref finite     -> y must be finite and |y - y_ref| <= rel * s + abs_
                          (the bound is inclusive).

    The bound is the per-element tolerance the method is held to, with
    s = sum_i |w_i x_i|; NaN positions (and infinities) must match exactly.
    """
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        close = np.isfinite(y) & (np.abs(y - y_ref) <= rel * s + abs_)
        same_inf = y == y_ref  # true only for an infinity of the same sign here
    return np.where(np.isnan(y_ref), np.isnan(y), np.where(np.isinf(y_ref), same_inf, close))


# --------------------------------------------------------------------------
# Test quantiser ([Arch] uniform block quantisation equation). Used only to
# build round-trip inputs; the configured workloads draw codes directly.
# --------------------------------------------------------------------------
def _round_half_away(v: np.ndarray) -> np.ndarray:
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def quantize_codes(w, d, qtype: int) -> np.ndarray:
    """q = clip(round(w / d) + z, qmin, qmax) per element, for a given block
    scale d (broadcast over the block). d == 0 gives q = z."""
    w = np.asarray(w, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    lo, hi = CODE_RANGE[qtype]
    z = ZERO_POINT[qtype]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d != 0.0, _round_half_away(w / np.where(d != 0.0, d, 1.0)), 0.0)
    return np.clip(r + z, lo, hi).astype(np.int64)


def quantize(w, qtype: int) -> np.ndarray:
    """Quantise fp32 weights [n_rows][k] into dense rows of blocks (uint8
    [n_rows][row_bytes]). Scale choice: d = fp16(amax / 7) for Q4_0,
    fp16(amax / 15) for Q5_0 and fp16(amax / 127) for Q8_0, so |w / d| stays
    inside the code range; for Q4_1 / Q5_1, m = fp16(block minimum) and
    d = fp16((max - min) / qmax), codes q = clip(round((w - m) / d), 0, qmax)
    with qmax = 15 / 31."""
    w = np.asarray(w, dtype=np.float32)
    n_rows, k = w.shape
    nblk = k // QK
    wb = w.reshape(n_rows, nblk, QK).astype(np.float64)
    if HAS_MIN[qtype]:
        lo, hi = np.min(wb, axis=2), np.max(wb, axis=2)
        d16 = ((hi - lo) / float(CODE_RANGE[qtype][1])).astype(np.float16)
        m16 = lo.astype(np.float16)
        d = d16.astype(np.float64)[:, :, None]
        q = quantize_codes(wb - m16.astype(np.float64)[:, :, None], d, qtype)
        return pack_blocks(d16.view(np.uint16), q, qtype, m16.view(np.uint16))
    amax = np.max(np.abs(wb), axis=2)
    div = {TYPE_Q4_0: 7.0, TYPE_Q5_0: 15.0, TYPE_Q8_0: 127.0}[qtype]
    d16 = (amax / div).astype(np.float16)
    d = d16.astype(np.float64)
    q = quantize_codes(wb, d[:, :, None], qtype)
    return pack_blocks(d16.view(np.uint16), q, qtype)


def pack_blocks(d_bits, q, qtype: int, m_bits=None) -> np.ndarray:
    """Lay out blocks: d as little-endian binary16, m likewise (Q4_1, Q5_1),
    the fifth bits as a little-endian 32-bit word (Q5_0, Q5_1), then the
    codes (nibble types: low four bits of element j in the low nibble and of
    element j + 16 in the high nibble of byte j; Q8_0: 32 int8 codes). q has
    shape [n_rows, nblk, 32]."""
    d_bits = np.asarray(d_bits, dtype=np.uint16)
    q = np.asarray(q, dtype=np.int64)
    n_rows, nblk = d_bits.shape
    bpb = BLOCK_BYTES[qtype]
    c0 = CODE_OFFSET[qtype]
    out = np.zeros((n_rows, nblk, bpb), dtype=np.uint8)
    out[:, :, 0] = d_bits & 0xFF
    out[:, :, 1] = d_bits >> 8
    if HAS_MIN[qtype]:
        m_bits = np.asarray(m_bits, dtype=np.uint16)
        out[:, :, 2] = m_bits & 0xFF
        out[:, :, 3] = m_bits >> 8
    if qtype in NIBBLE_TYPES:
        out[:, :, c0:] = ((q[:, :, :16] & 0xF) | ((q[:, :, 16:] & 0xF) << 4)).astype(np.uint8)
        if qtype in QH_OFFSET:
            qh = np.zeros((n_rows, nblk), dtype=np.int64)
            for j in range(32):
                qh |= ((q[:, :, j] >> 4) & 1) << j
            for b in range(4):
                out[:, :, QH_OFFSET[qtype] + b] = (qh >> (8 * b)) & 0xFF
    else:
        out[:, :, c0:] = q.astype(np.int8).view(np.uint8)
    return out.reshape(n_rows, nblk * bpb)
