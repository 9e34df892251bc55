"""Host-side checks of the C ABI (no GPU needed).

The shared library must load, export every function include/qmm.h declares,
and reject each class of invalid argument with its status code before any
HIP call. Pointers passed here are fake (never dereferenced): validation
happens on the host first, and zero-sized calls return before any launch.
"""
import ctypes
import os
import re

import pytest

import block_quantized_matmul_amd as qmm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmm.h")
Q4, Q8 = qmm.QMM_TYPE_Q4_0, qmm.QMM_TYPE_Q8_0

P = ctypes.c_void_p(0x10000)   # fake, 16-byte-aligned device addresses
P2 = ctypes.c_void_p(0x20000)
P3 = ctypes.c_void_p(0x30000)
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def L():
    return qmm.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s+\*?\s*(qmm_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["qmm_matmul", "qmm_matmul_x16", "qmm_matmul_path", "qmm_matmul_batch",
                            "qmm_matmul_batch_ws", "qmm_matmul_batch_workspace_bytes",
                            "qmm_matmul_ws", "qmm_matmul_workspace_bytes",
                            "qmm_dequantize", "qmm_get_rows", "qmm_matmul_id", "qmm_matmul_id_noalloc",
                            "qmm_matmul_id_workspace_bytes", "qmm_matmul_id_workspace_bytes_x16", "qmm_row_bytes",
                            "qmm_supports", "qmm_status_string"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert hasattr(qmm, name), f"python binding lacks {name}"


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name, val in re.findall(r"#define (QMM_[A-Z_0-9]+) \(?(-?\d+)\)?", text):
        assert getattr(qmm, name) == int(val), name


def test_row_bytes_and_supports(L):
    assert L.qmm_row_bytes(Q4, 4096) == 2304
    assert L.qmm_row_bytes(Q8, 4096) == 4352
    assert L.qmm_row_bytes(Q4, 11008) == 6192
    assert L.qmm_row_bytes(Q8, 32) == 34
    assert L.qmm_row_bytes(qmm.QMM_TYPE_Q4_1, 4096) == 2560
    assert L.qmm_supports(qmm.QMM_TYPE_Q4_1, 64, 40) == 1 and L.qmm_supports(qmm.QMM_TYPE_Q4_1, 64, 38) == 0
    assert L.qmm_row_bytes(qmm.QMM_TYPE_Q5_0, 4096) == 2816 and L.qmm_row_bytes(qmm.QMM_TYPE_Q5_1, 4096) == 3072
    for bad_type in (0, 1, 4, 5, 9, 11, 13):
        assert L.qmm_row_bytes(bad_type, 4096) == qmm.QMM_ERR_TYPE
    for bad_k in (0, -32, 48, 1 << 31):
        assert L.qmm_row_bytes(Q4, bad_k) == qmm.QMM_ERR_SHAPE
    assert L.qmm_supports(Q4, 4096, 2304) == 1
    assert L.qmm_supports(Q4, 4096, 2560) == 1
    assert L.qmm_supports(Q4, 96, 54) == 1
    assert L.qmm_supports(Q4, 4096, 2303) == 0
    assert L.qmm_supports(Q4, 4096, 2302) == 0
    assert L.qmm_supports(Q8, 48, 100) == 0
    assert L.qmm_supports(5, 4096, 4096) == 0


def test_q4_k_layout_rules(L):
    QK = qmm.QMM_TYPE_Q4_K
    assert L.qmm_row_bytes(QK, 4096) == 2304 and L.qmm_row_bytes(QK, 256) == 144
    assert L.qmm_row_bytes(QK, 11008) == 43 * 144
    for bad_k in (32, 128, 4000, 0):
        assert L.qmm_row_bytes(QK, bad_k) == qmm.QMM_ERR_SHAPE
    assert L.qmm_supports(QK, 256, 144) == 1 and L.qmm_supports(QK, 256, 160) == 1
    assert L.qmm_supports(QK, 256, 146) == 0   # rows must stay 16-byte aligned
    assert L.qmm_supports(QK, 256, 128) == 0   # smaller than the row's block
    assert L.qmm_supports(QK, 32, 144) == 0
    # host checks, nothing launched
    assert _mm(L, t=QK, k=96, nb1=144) == qmm.QMM_ERR_SHAPE
    assert _mm(L, t=QK, k=256, nb1=152) == qmm.QMM_ERR_STRIDE
    assert _mm(L, t=QK, k=256, nb1=144, W=ctypes.c_void_p(0x10008)) == qmm.QMM_ERR_ALIGN
    assert _mm(L, t=QK, k=256, nb1=144, n=0) == qmm.QMM_OK   # empty: no launch
    assert _mm(L, t=QK, k=256, nb1=1 << 24, rows=2) == qmm.QMM_ERR_SHAPE  # beyond 32-bit offsets
    assert _mid(L, t=QK, k=256, nb1=144, rows=4, nb2=584) == qmm.QMM_ERR_STRIDE  # expert stride not 16-aligned
    assert _mid(L, t=QK, k=256, nb1=144, rows=4, nb2=576, n=0) == qmm.QMM_OK


def test_status_strings(L):
    for code in range(-9, 1):
        s = qmm.qmm_status_string(code)
        assert s.startswith("QMM_OK" if code == 0 else "QMM_ERR_")
    assert qmm.qmm_status_string(-99) == "unknown qmm status"


def _mm(L, W=P, t=Q4, rows=16, k=64, nb1=36, X=P2, xt=qmm.QMM_X_F32, n=1, Y=P3, path=0):
    return L.qmm_matmul_path(W, t, rows, k, nb1, X, xt, n, Y, path, NULL)


def test_validation_codes(L):
    E = qmm
    assert _mm(L, W=NULL) == E.QMM_ERR_NULL
    assert _mm(L, X=NULL) == E.QMM_ERR_NULL
    assert _mm(L, Y=NULL) == E.QMM_ERR_NULL
    assert _mm(L, t=0) == E.QMM_ERR_TYPE
    assert _mm(L, t=1) == E.QMM_ERR_TYPE
    assert _mm(L, xt=2) == E.QMM_ERR_TYPE
    assert _mm(L, k=0) == E.QMM_ERR_SHAPE
    assert _mm(L, k=40) == E.QMM_ERR_SHAPE
    assert _mm(L, k=-64) == E.QMM_ERR_SHAPE
    assert _mm(L, rows=-1) == E.QMM_ERR_SHAPE
    assert _mm(L, rows=1 << 31) == E.QMM_ERR_SHAPE
    assert _mm(L, n=-1) == E.QMM_ERR_SHAPE
    assert _mm(L, nb1=35) == E.QMM_ERR_STRIDE
    assert _mm(L, nb1=34) == E.QMM_ERR_STRIDE
    assert _mm(L, t=Q8, nb1=36) == E.QMM_ERR_STRIDE
    assert _mm(L, W=ctypes.c_void_p(0x10001)) == E.QMM_ERR_ALIGN
    assert _mm(L, X=ctypes.c_void_p(0x20002)) == E.QMM_ERR_ALIGN
    assert _mm(L, Y=ctypes.c_void_p(0x30002)) == E.QMM_ERR_ALIGN
    assert _mm(L, path=3) == E.QMM_ERR_PATH
    assert _mm(L, path=qmm.QMM_PATH_GEMV, n=9) == E.QMM_ERR_PATH


def _ws(L, W=P, t=Q4, rows=16, k=64, nb1=36, X=P2, xt=qmm.QMM_X_F16, n=1, Y=P3, ws=NULL, ws_bytes=0):
    return L.qmm_matmul_ws(W, t, rows, k, nb1, X, xt, n, Y, ws, ws_bytes, NULL)


def test_matmul_ws_validation(L):
    """qmm_matmul_ws runs qmm_matmul_path's checks first, then the
    workspace's; the size query rejects what the call rejects. (Without a
    GPU the size query sees no compute units and asks for no workspace.)"""
    E = qmm
    assert _ws(L, W=NULL) == E.QMM_ERR_NULL
    assert _ws(L, X=NULL) == E.QMM_ERR_NULL
    assert _ws(L, Y=NULL) == E.QMM_ERR_NULL
    assert _ws(L, t=1) == E.QMM_ERR_TYPE
    assert _ws(L, xt=2) == E.QMM_ERR_TYPE
    assert _ws(L, k=40) == E.QMM_ERR_SHAPE
    assert _ws(L, n=-1) == E.QMM_ERR_SHAPE
    assert _ws(L, rows=1 << 31) == E.QMM_ERR_SHAPE
    assert _ws(L, nb1=35) == E.QMM_ERR_STRIDE
    assert _ws(L, X=ctypes.c_void_p(0x20002)) == E.QMM_ERR_ALIGN
    assert _ws(L, n=0) == E.QMM_OK and _ws(L, rows=0, n=600) == E.QMM_OK   # empty: no launch
    assert _ws(L, n=0, ws=ctypes.c_void_p(0x50001), ws_bytes=-5) == E.QMM_OK  # unused workspace not checked
    wb = L.qmm_matmul_workspace_bytes
    assert wb(1, 16, 64, 600, qmm.QMM_X_F16) == E.QMM_ERR_TYPE
    assert wb(Q4, 16, 64, 600, 2) == E.QMM_ERR_TYPE
    assert wb(Q4, 16, 40, 600, qmm.QMM_X_F16) == E.QMM_ERR_SHAPE
    assert wb(Q4, -1, 64, 600, qmm.QMM_X_F16) == E.QMM_ERR_SHAPE
    assert wb(Q4, 16, 64, -1, qmm.QMM_X_F16) == E.QMM_ERR_SHAPE
    assert wb(Q4, 16, 64, 1 << 31, qmm.QMM_X_F16) == E.QMM_ERR_SHAPE
    assert wb(Q4, (1 << 31) - 1, (1 << 31) - 32, 1 << 30, qmm.QMM_X_F16) == E.QMM_ERR_SHAPE  # n * k > 2^60
    for n in (0, 1, 8):
        assert wb(Q4, 4096, 4096, n, qmm.QMM_X_F16) == 0   # decode sizes never split
    assert wb(Q4, 0, 4096, 600, qmm.QMM_X_F16) == 0
    assert wb(Q4, 4096, 4096, 512, qmm.QMM_X_F32) == 0     # fp32 activations never split


def test_zero_sized_calls_launch_nothing(L):
    # 2-byte-aligned W and a padded odd stride are valid; nothing is launched.
    assert _mm(L, rows=0) == qmm.QMM_OK
    assert _mm(L, n=0) == qmm.QMM_OK
    assert _mm(L, W=ctypes.c_void_p(0x10002), nb1=38, n=0) == qmm.QMM_OK
    assert _mm(L, path=qmm.QMM_PATH_GEMM, n=0) == qmm.QMM_OK
    assert L.qmm_matmul(P, Q8, 0, 64, 68, P2, 4, P3, NULL) == qmm.QMM_OK
    assert L.qmm_matmul_x16(P, Q8, 5, 64, 68, P2, 0, P3, NULL) == qmm.QMM_OK
    assert L.qmm_dequantize(P, Q4, 0, 64, 36, P2, NULL) == qmm.QMM_OK


def test_dequantize_validation(L):
    assert L.qmm_dequantize(NULL, Q4, 4, 64, 36, P2, NULL) == qmm.QMM_ERR_NULL
    assert L.qmm_dequantize(P, Q4, 4, 64, 36, NULL, NULL) == qmm.QMM_ERR_NULL
    assert L.qmm_dequantize(P, 9, 4, 64, 36, P2, NULL) == qmm.QMM_ERR_TYPE
    assert L.qmm_dequantize(P, Q4, 4, 63, 36, P2, NULL) == qmm.QMM_ERR_SHAPE
    assert L.qmm_dequantize(P, Q4, 4, 64, 30, P2, NULL) == qmm.QMM_ERR_STRIDE
    assert L.qmm_dequantize(P, Q4, 4, 64, 36, ctypes.c_void_p(0x20002), NULL) == qmm.QMM_ERR_ALIGN


def test_get_rows_validation(L):
    A = ctypes.c_void_p(0x40000)  # fake 16-byte-aligned index pointer
    assert L.qmm_get_rows(NULL, Q4, 4, 64, 36, A, 3, P2, NULL) == qmm.QMM_ERR_NULL
    assert L.qmm_get_rows(P, Q4, 4, 64, 36, NULL, 3, P2, NULL) == qmm.QMM_ERR_NULL
    assert L.qmm_get_rows(P, Q4, 4, 64, 36, A, 3, NULL, NULL) == qmm.QMM_ERR_NULL
    assert L.qmm_get_rows(P, 9, 4, 64, 36, A, 3, P2, NULL) == qmm.QMM_ERR_TYPE
    assert L.qmm_get_rows(P, Q4, 4, 63, 36, A, 3, P2, NULL) == qmm.QMM_ERR_SHAPE
    assert L.qmm_get_rows(P, Q4, 4, 64, 36, A, -1, P2, NULL) == qmm.QMM_ERR_SHAPE
    assert L.qmm_get_rows(P, Q4, 4, 64, 30, A, 3, P2, NULL) == qmm.QMM_ERR_STRIDE
    assert L.qmm_get_rows(P, Q4, 4, 64, 36, ctypes.c_void_p(0x40002), 3, P2, NULL) == qmm.QMM_ERR_ALIGN
    assert L.qmm_get_rows(P, Q4, 4, 64, 36, A, 3, ctypes.c_void_p(0x20002), NULL) == qmm.QMM_ERR_ALIGN
    # zero indices: nothing is launched
    assert L.qmm_get_rows(P, Q4, 4, 64, 36, A, 0, P2, NULL) == qmm.QMM_OK


def _mid(L, W=P, t=Q4, ne=8, rows=16, k=64, nb1=36, nb2=576, X=P2, xs=2, ids=ctypes.c_void_p(0x40000), n_ids=2,
         n=3, Y=P3, ws=NULL, ws_bytes=0):
    return L.qmm_matmul_id(W, t, ne, rows, k, nb1, nb2, X, xs, ids, n_ids, n, Y, ws, ws_bytes, NULL)


def test_matmul_id_validation(L):
    # nothing below is launched: every call fails a host check or is empty
    assert _mid(L, W=NULL) == qmm.QMM_ERR_NULL
    assert _mid(L, X=NULL) == qmm.QMM_ERR_NULL
    assert _mid(L, ids=NULL) == qmm.QMM_ERR_NULL
    assert _mid(L, Y=NULL) == qmm.QMM_ERR_NULL
    assert _mid(L, t=5) == qmm.QMM_ERR_TYPE
    assert _mid(L, k=48) == qmm.QMM_ERR_SHAPE
    assert _mid(L, ne=-1) == qmm.QMM_ERR_SHAPE
    assert _mid(L, n_ids=-1, xs=1) == qmm.QMM_ERR_SHAPE
    assert _mid(L, n=-1) == qmm.QMM_ERR_SHAPE
    assert _mid(L, xs=3) == qmm.QMM_ERR_SHAPE            # x_slots must be 1 or n_ids
    assert _mid(L, n_ids=1 << 16, xs=1, n=1 << 16) == qmm.QMM_ERR_SHAPE  # 2^32 pairs
    assert _mid(L, nb1=35) == qmm.QMM_ERR_STRIDE
    assert _mid(L, nb2=575) == qmm.QMM_ERR_STRIDE         # below n_rows * nb1
    assert _mid(L, nb2=577) == qmm.QMM_ERR_STRIDE         # odd
    assert _mid(L, W=ctypes.c_void_p(0x10001)) == qmm.QMM_ERR_ALIGN
    assert _mid(L, X=ctypes.c_void_p(0x20002)) == qmm.QMM_ERR_ALIGN
    assert _mid(L, ids=ctypes.c_void_p(0x40002)) == qmm.QMM_ERR_ALIGN
    assert _mid(L, Y=ctypes.c_void_p(0x30002)) == qmm.QMM_ERR_ALIGN
    # more tokens than the decode kernels take: the grouped GEMM route needs a workspace
    need = L.qmm_matmul_id_workspace_bytes(8, 2, 64)
    assert need >= 64 * 2 * 4 + 16 * 8
    assert _mid(L, n=64, ws=NULL, ws_bytes=need) == qmm.QMM_ERR_WORKSPACE
    assert _mid(L, n=64, ws=ctypes.c_void_p(0x50000), ws_bytes=need - 1) == qmm.QMM_ERR_WORKSPACE
    assert _mid(L, n=64, ws=ctypes.c_void_p(0x50002), ws_bytes=need) == qmm.QMM_ERR_ALIGN
    assert _mid(L, n=64, ws=ctypes.c_void_p(0x50000), ws_bytes=need, k=48) == qmm.QMM_ERR_SHAPE
    # empty calls succeed without a launch
    assert _mid(L, n=0) == qmm.QMM_OK
    assert _mid(L, n_ids=0, xs=1) == qmm.QMM_OK
    assert _mid(L, rows=0, nb2=0) == qmm.QMM_OK


def test_matmul_id_workspace_sizes(L):
    W = L.qmm_matmul_id_workspace_bytes
    assert W(8, 2, 1) == 0                               # one token: per-pair decode
    assert W(8, 2, 4) == 0                               # about one pair per expert: per-pair
    assert W(8, 2, 8) == 64 + 16 * (8 + 8)               # 2 pairs per expert: decode tiles of 2
    assert W(8, 0, 512) == 0
    assert W(5000, 2, 512) == 0                          # too many experts to bucket in LDS
    assert W(8, 2, 15) == 128 + 16 * (8 + 8)             # 30 pairs: decode tiles of 4
    assert W(8, 2, 16) == 128 + 16 * (1 + 8)             # 4 pairs per expert: 128-pair GEMM tiles
    assert W(64, 8, 9) == 288 + 16 * (36 + 64)           # 72 pairs over 64 experts: tiles of 2
    assert W(64, 8, 32) > 0
    # 1024 pairs in up to 8 + 8 tiles of 128, plus the pair list
    assert W(8, 2, 512) == 1024 * 4 + 16 * (8 + 8)
    assert W(2, 1, 9) == 48 + 16 * (1 + 2)
    assert W(-1, 2, 512) == qmm.QMM_ERR_SHAPE
    assert W(8, 1 << 16, 1 << 16) == qmm.QMM_ERR_SHAPE


def test_matmul_id_workspace_sizes_x16(L):
    W, X16 = L.qmm_matmul_id_workspace_bytes, L.qmm_matmul_id_workspace_bytes_x16
    # the matrix-core route adds an fp16 copy of X: n_tokens * x_slots * k * 2 bytes
    assert X16(8, 2, 512, 4096, 1) == W(8, 2, 512) + 512 * 4096 * 2
    assert X16(8, 2, 512, 4096, 2) == W(8, 2, 512) + 512 * 2 * 4096 * 2
    assert X16(8, 2, 16, 256, 2) == W(8, 2, 16) + 16 * 2 * 256 * 2
    # other routes need no copy
    for args in ((8, 2, 1), (8, 2, 8), (8, 2, 15), (5000, 2, 512), (8, 0, 512)):
        assert X16(*args, 4096, 1) == W(*args), args
    # bad sizes
    assert X16(8, 2, 512, 0, 1) == qmm.QMM_ERR_SHAPE
    assert X16(8, 2, 512, 4096, 3) == qmm.QMM_ERR_SHAPE
    assert X16(-1, 2, 512, 4096, 1) == qmm.QMM_ERR_SHAPE
    assert X16(8, 2, 1 << 20, 1 << 16, 2) == qmm.QMM_ERR_SHAPE


def _mid_na(L, W=P, t=Q4, ne=8, rows=16, k=64, nb1=36, nb2=576, X=P2, xs=2, ids=ctypes.c_void_p(0x40000), n_ids=2,
            n=3, Y=P3):
    return L.qmm_matmul_id_noalloc(W, t, ne, rows, k, nb1, nb2, X, xs, ids, n_ids, n, Y, NULL)


def test_matmul_id_noalloc_validation(L):
    # the same host checks as qmm_matmul_id, none of which touches the GPU
    assert _mid_na(L, W=NULL) == qmm.QMM_ERR_NULL
    assert _mid_na(L, ids=NULL) == qmm.QMM_ERR_NULL
    assert _mid_na(L, t=5) == qmm.QMM_ERR_TYPE
    assert _mid_na(L, k=48) == qmm.QMM_ERR_SHAPE
    assert _mid_na(L, xs=3) == qmm.QMM_ERR_SHAPE
    assert _mid_na(L, nb2=575) == qmm.QMM_ERR_STRIDE
    assert _mid_na(L, Y=ctypes.c_void_p(0x30002)) == qmm.QMM_ERR_ALIGN
    # a call whose routing table would exceed the held scratch is refused before any HIP call
    n = 200000
    assert L.qmm_matmul_id_workspace_bytes(8, 2, n) > qmm.QMM_NOALLOC_SCRATCH_BYTES
    assert _mid_na(L, n=n, xs=1) == qmm.QMM_ERR_SCRATCH
    assert "QMM_NOALLOC_SCRATCH_BYTES" in qmm.qmm_status_string(qmm.QMM_ERR_SCRATCH)
    # empty calls succeed without touching the device
    assert _mid_na(L, n=0) == qmm.QMM_OK
    assert _mid_na(L, rows=0, nb2=0) == qmm.QMM_OK


def test_binding_refuses_cpu_tensors():
    import torch
    W = torch.zeros((4, 36), dtype=torch.uint8)
    X = torch.zeros((1, 64), dtype=torch.float32)
    with pytest.raises(TypeError):
        qmm.qmm_matmul(W, Q4, 64, X, Y=torch.empty((1, 4)))
    with pytest.raises(TypeError):
        qmm.qmm_dequantize(W, Q4, 64, out=torch.empty((4, 64)))


def test_batch_validation(L):
    D = qmm.qmm_matmul_desc
    ok = D(0x10000, Q4, 16, 64, 36, 0x20000, qmm.QMM_X_F32, 0, 0x30000)   # zero tokens: valid, no launch
    bad_stride = D(0x10000, Q4, 16, 64, 35, 0x20000, qmm.QMM_X_F32, 1, 0x30000)
    bad_type = D(0x10000, 5, 16, 64, 36, 0x20000, qmm.QMM_X_F32, 1, 0x30000)
    bad_x = D(0x10000, Q4, 16, 64, 36, 0x20000, 3, 1, 0x30000)
    arr = (D * 3)(ok, ok, ok)
    assert L.qmm_matmul_batch(arr, 3, NULL) == qmm.QMM_OK
    assert L.qmm_matmul_batch(arr, 0, NULL) == qmm.QMM_OK
    assert L.qmm_matmul_batch(None, 0, NULL) == qmm.QMM_OK
    assert L.qmm_matmul_batch(None, 2, NULL) == qmm.QMM_ERR_NULL
    assert L.qmm_matmul_batch(arr, -1, NULL) == qmm.QMM_ERR_SHAPE
    # the first invalid descriptor's status is returned, nothing launched
    assert L.qmm_matmul_batch((D * 3)(ok, bad_stride, bad_type), 3, NULL) == qmm.QMM_ERR_STRIDE
    assert L.qmm_matmul_batch((D * 2)(bad_type, bad_stride), 2, NULL) == qmm.QMM_ERR_TYPE
    assert L.qmm_matmul_batch((D * 1)(bad_x), 1, NULL) == qmm.QMM_ERR_TYPE
    nullw = D(0, Q4, 16, 64, 36, 0x20000, qmm.QMM_X_F32, 1, 0x30000)
    assert L.qmm_matmul_batch((D * 2)(ok, nullw), 2, NULL) == qmm.QMM_ERR_NULL


def test_batch_ws_validation(L):
    """The workspace form validates as the plain batch does, sizes no
    workspace for decode-sized, empty or fp32 descriptors, and checks the
    workspace only where one is needed."""
    D = qmm.qmm_matmul_desc
    empty = D(0x10000, Q4, 16, 64, 36, 0x20000, qmm.QMM_X_F16, 0, 0x30000)
    decode = D(0x10000, Q4, 4096, 4096, 2304, 0x20000, qmm.QMM_X_F32, 1, 0x30000)
    f32 = D(0x10000, Q4, 4096, 4096, 2304, 0x20000, qmm.QMM_X_F32, 2048, 0x30000)
    bad_stride = D(0x10000, Q4, 16, 64, 35, 0x20000, qmm.QMM_X_F16, 600, 0x30000)
    wb, bw = L.qmm_matmul_batch_workspace_bytes, L.qmm_matmul_batch_ws
    assert wb((D * 3)(empty, decode, f32), 3) == 0
    assert wb(None, 0) == 0 and wb(None, 1) == qmm.QMM_ERR_NULL and wb((D * 1)(empty), -1) == qmm.QMM_ERR_SHAPE
    assert wb((D * 2)(empty, bad_stride), 2) == qmm.QMM_ERR_STRIDE
    assert bw((D * 2)(empty, bad_stride), 2, NULL, 0, NULL) == qmm.QMM_ERR_STRIDE
    assert bw((D * 2)(empty, empty), 2, NULL, 0, NULL) == qmm.QMM_OK        # nothing to launch
    assert bw((D * 1)(empty), 1, ctypes.c_void_p(0x50001), -5, NULL) == qmm.QMM_OK  # unused workspace not checked
    assert bw(None, 0, NULL, 0, NULL) == qmm.QMM_OK
    assert bw(None, 2, NULL, 0, NULL) == qmm.QMM_ERR_NULL
