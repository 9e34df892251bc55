"""Block-quantized MUL_MAT (GGUF Q4_0 / Q8_0) for the AMD MI355X (gfx950).

A thin ctypes binding over libqmm.so, whose C ABI is declared in
include/qmm.h. The functions here carry the C names and only marshal
arguments: torch tensors supply device pointers and the current HIP stream;
every step of the computation runs in the library's HIP kernels. There is no
CPU fallback: a missing library or a tensor that is not on a GPU raises.
"""
from __future__ import annotations

import ctypes
import os

QMM_TYPE_Q4_0 = 2
QMM_TYPE_Q4_1 = 3
QMM_TYPE_Q5_0 = 6
QMM_TYPE_Q5_1 = 7
QMM_TYPE_Q8_0 = 8
QMM_TYPE_Q4_K = 12
QMM_X_F32 = 0
QMM_X_F16 = 1
QMM_PATH_AUTO = 0
QMM_PATH_GEMV = 1
QMM_PATH_GEMM = 2
QMM_GEMV_MAX_TOKENS = 8

QMM_OK = 0
QMM_ERR_NULL = -1
QMM_ERR_TYPE = -2
QMM_ERR_SHAPE = -3
QMM_ERR_STRIDE = -4
QMM_ERR_ALIGN = -5
QMM_ERR_HIP = -6
QMM_ERR_PATH = -7
QMM_ERR_WORKSPACE = -8
QMM_ERR_SCRATCH = -9
QMM_NOALLOC_SCRATCH_BYTES = 1048576

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqmm.so")

_lib = None


class qmm_matmul_desc(ctypes.Structure):
    """Mirror of the C struct qmm_matmul_desc (include/qmm.h)."""
    _fields_ = [("W", ctypes.c_void_p), ("ggml_type", ctypes.c_int), ("n_rows", ctypes.c_int64),
                ("k", ctypes.c_int64), ("row_stride_bytes", ctypes.c_int64), ("X", ctypes.c_void_p),
                ("x_type", ctypes.c_int), ("n_tokens", ctypes.c_int64), ("Y", ctypes.c_void_p)]


class QmmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {qmm_status_string(status)} ({status})")


def lib() -> ctypes.CDLL:
    """The loaded libqmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run python -m block_quantized_matmul_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.qmm_matmul.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp]
        L.qmm_matmul_x16.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp]
        L.qmm_matmul_path.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, vp, i32, vp]
        L.qmm_dequantize.argtypes = [vp, i32, i64, i64, i64, vp, vp]
        L.qmm_matmul_batch.argtypes = [ctypes.POINTER(qmm_matmul_desc), i32, vp]
        L.qmm_matmul_batch_ws.argtypes = [ctypes.POINTER(qmm_matmul_desc), i32, vp, i64, vp]
        L.qmm_matmul_batch_workspace_bytes.argtypes = [ctypes.POINTER(qmm_matmul_desc), i32]
        L.qmm_matmul_batch_workspace_bytes.restype = i64
        L.qmm_get_rows.argtypes = [vp, i32, i64, i64, i64, vp, i64, vp, vp]
        L.qmm_matmul_id.argtypes = [vp, i32, i64, i64, i64, i64, i64, vp, i64, vp, i64, i64, vp, vp, i64, vp]
        L.qmm_matmul_id_noalloc.argtypes = [vp, i32, i64, i64, i64, i64, i64, vp, i64, vp, i64, i64, vp, vp]
        L.qmm_matmul_id_workspace_bytes.argtypes = [i64, i64, i64]
        L.qmm_matmul_id_workspace_bytes.restype = i64
        L.qmm_matmul_id_workspace_bytes_x16.argtypes = [i64, i64, i64, i64, i64]
        L.qmm_matmul_id_workspace_bytes_x16.restype = i64
        L.qmm_matmul_ws.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, vp, vp, i64, vp]
        L.qmm_matmul_workspace_bytes.argtypes = [i32, i64, i64, i64, i32]
        L.qmm_matmul_workspace_bytes.restype = i64
        for f in ("qmm_matmul", "qmm_matmul_x16", "qmm_matmul_path", "qmm_matmul_ws", "qmm_dequantize",
                  "qmm_matmul_batch", "qmm_matmul_batch_ws", "qmm_get_rows", "qmm_matmul_id",
                  "qmm_matmul_id_noalloc"):
            getattr(L, f).restype = i32
        L.qmm_row_bytes.argtypes = [i32, i64]
        L.qmm_row_bytes.restype = i64
        L.qmm_supports.argtypes = [i32, i64, i64]
        L.qmm_supports.restype = i32
        L.qmm_status_string.argtypes = [i32]
        L.qmm_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def qmm_status_string(status: int) -> str:
    return lib().qmm_status_string(int(status)).decode()


def qmm_row_bytes(ggml_type: int, k: int) -> int:
    return int(lib().qmm_row_bytes(int(ggml_type), int(k)))


def qmm_supports(ggml_type: int, k: int, row_stride_bytes: int) -> bool:
    return bool(lib().qmm_supports(int(ggml_type), int(k), int(row_stride_bytes)))


def _gpu_ptr(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (the library has no CPU path)")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check_span(t, dtype, n_elems, name):
    """t must be a contiguous GPU tensor of `dtype` holding at least n_elems
    elements: the C entry points trust the sizes they are given, so the
    binding checks that the buffers behind them are large enough."""
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < n_elems:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n_elems}")


def _weights_span(ggml_type, k, n_rows, nb1, n_experts=1, nb2=0):
    """Bytes of W the kernels may read: up to the end of the last row's blocks."""
    if n_rows <= 0 or n_experts <= 0:
        return 0
    dense = qmm_row_bytes(ggml_type, k)
    if dense < 0:
        return 0  # the C call reports the type or shape error
    return (n_experts - 1) * nb2 + (n_rows - 1) * nb1 + dense


def _weights_geometry(W, n_rows, row_stride_bytes):
    import torch
    if W.dtype != torch.uint8:
        raise TypeError("W must be a uint8 tensor of raw blocks")
    if n_rows is None or row_stride_bytes is None:
        if W.dim() != 2 or not W.is_contiguous():
            raise ValueError("pass n_rows and row_stride_bytes for a W that is not a contiguous [rows][nb1] tensor")
        n_rows, row_stride_bytes = W.shape
    return int(n_rows), int(row_stride_bytes)


def _matmul_args(W, ggml_type, k, X, n_rows, row_stride_bytes, n_tokens, Y):
    """Geometry, activation type and checked buffers of a MUL_MAT call."""
    import torch
    n_rows, nb1 = _weights_geometry(W, n_rows, row_stride_bytes)
    if X.dtype == torch.float32:
        x_type = QMM_X_F32
    elif X.dtype == torch.float16:
        x_type = QMM_X_F16
    else:
        raise TypeError("X must be float32 or float16")
    if n_tokens is None:
        if X.dim() != 2 or not X.is_contiguous():
            raise ValueError("X must be a contiguous [n_tokens][k] tensor")
        n_tokens = X.shape[0]
    if Y is None:
        Y = torch.empty((int(n_tokens), n_rows), dtype=torch.float32, device=X.device)
    _check_span(W, torch.uint8, _weights_span(ggml_type, k, n_rows, nb1), "W")
    _check_span(X, X.dtype, int(n_tokens) * int(k), "X")
    _check_span(Y, torch.float32, int(n_tokens) * n_rows, "Y")
    return n_rows, nb1, x_type, int(n_tokens), Y


def qmm_matmul_path(W, ggml_type, k, X, n_rows=None, row_stride_bytes=None, n_tokens=None, Y=None,
                    path=QMM_PATH_AUTO, stream=None):
    """Y[n_tokens][n_rows] = MUL_MAT(W, X) with the kernel chosen by `path`.
    X is a GPU fp32 or fp16 tensor [n_tokens][k]; Y is allocated if None."""
    n_rows, nb1, x_type, n_tokens, Y = _matmul_args(W, ggml_type, k, X, n_rows, row_stride_bytes, n_tokens, Y)
    st = lib().qmm_matmul_path(_gpu_ptr(W, "W"), int(ggml_type), n_rows, int(k), nb1, _gpu_ptr(X, "X"), x_type,
                               int(n_tokens), _gpu_ptr(Y, "Y"), int(path), _stream(stream))
    if st != QMM_OK:
        raise QmmError(st, "qmm_matmul_path")
    return Y


def qmm_matmul(W, ggml_type, k, X, n_rows=None, row_stride_bytes=None, n_tokens=None, Y=None, stream=None):
    """MUL_MAT with fp32 activations (C: qmm_matmul)."""
    import torch
    if X.dtype != torch.float32:
        raise TypeError("qmm_matmul takes float32 activations; use qmm_matmul_x16 for float16")
    return qmm_matmul_path(W, ggml_type, k, X, n_rows, row_stride_bytes, n_tokens, Y, QMM_PATH_AUTO, stream)


def qmm_matmul_x16(W, ggml_type, k, X, n_rows=None, row_stride_bytes=None, n_tokens=None, Y=None, stream=None):
    """MUL_MAT with fp16 activations (C: qmm_matmul_x16)."""
    import torch
    if X.dtype != torch.float16:
        raise TypeError("qmm_matmul_x16 takes float16 activations")
    return qmm_matmul_path(W, ggml_type, k, X, n_rows, row_stride_bytes, n_tokens, Y, QMM_PATH_AUTO, stream)


def qmm_matmul_workspace_bytes(ggml_type: int, n_rows: int, k: int, n_tokens: int, x_type: int = QMM_X_F16) -> int:
    return int(lib().qmm_matmul_workspace_bytes(int(ggml_type), int(n_rows), int(k), int(n_tokens), int(x_type)))


def qmm_matmul_ws(W, ggml_type, k, X, workspace, n_rows=None, row_stride_bytes=None, n_tokens=None, Y=None,
                  stream=None):
    """MUL_MAT with a caller workspace that lets the matrix-core kernel split
    k across workgroups (C: qmm_matmul_ws). `workspace` is a GPU uint8 tensor
    of at least qmm_matmul_workspace_bytes bytes that held zeros when first
    used (torch.zeros), or None when that size is 0."""
    import torch
    n_rows, nb1, x_type, n_tokens, Y = _matmul_args(W, ggml_type, k, X, n_rows, row_stride_bytes, n_tokens, Y)
    if workspace is not None:
        _check_span(workspace, torch.uint8, 0, "workspace")
    ws = _gpu_ptr(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() if workspace is not None else 0
    st = lib().qmm_matmul_ws(_gpu_ptr(W, "W"), int(ggml_type), n_rows, int(k), nb1, _gpu_ptr(X, "X"), x_type,
                             n_tokens, _gpu_ptr(Y, "Y"), ws, ws_bytes, _stream(stream))
    if st != QMM_OK:
        raise QmmError(st, "qmm_matmul_ws")
    return Y


def qmm_dequantize(W, ggml_type, k, n_rows=None, row_stride_bytes=None, out=None, stream=None):
    """The block decoder alone: fp32 [n_rows][k] (C: qmm_dequantize)."""
    import torch
    n_rows, nb1 = _weights_geometry(W, n_rows, row_stride_bytes)
    if out is None:
        out = torch.empty((n_rows, int(k)), dtype=torch.float32, device=W.device)
    _check_span(W, torch.uint8, _weights_span(ggml_type, k, n_rows, nb1), "W")
    _check_span(out, torch.float32, n_rows * int(k), "out")
    st = lib().qmm_dequantize(_gpu_ptr(W, "W"), int(ggml_type), n_rows, int(k), nb1, _gpu_ptr(out, "out"),
                              _stream(stream))
    if st != QMM_OK:
        raise QmmError(st, "qmm_dequantize")
    return out


def qmm_get_rows(W, ggml_type, k, ids, n_rows=None, row_stride_bytes=None, out=None, stream=None):
    """GET_ROWS: fp32 [len(ids)][k], row i = dequantised row ids[i] of W
    (C: qmm_get_rows; an index outside [0, n_rows) gives a row of NaNs).
    ids is a contiguous int32 GPU tensor."""
    import torch
    n_rows, nb1 = _weights_geometry(W, n_rows, row_stride_bytes)
    if ids.dtype != torch.int32 or ids.dim() != 1 or not ids.is_contiguous():
        raise TypeError("ids must be a contiguous 1-D int32 tensor")
    n_ids = int(ids.shape[0])
    if out is None:
        out = torch.empty((n_ids, int(k)), dtype=torch.float32, device=W.device)
    _check_span(W, torch.uint8, _weights_span(ggml_type, k, n_rows, nb1), "W")
    _check_span(out, torch.float32, n_ids * int(k), "out")
    st = lib().qmm_get_rows(_gpu_ptr(W, "W"), int(ggml_type), n_rows, int(k), nb1, _gpu_ptr(ids, "ids"), n_ids,
                            _gpu_ptr(out, "out"), _stream(stream))
    if st != QMM_OK:
        raise QmmError(st, "qmm_get_rows")
    return out


def qmm_matmul_id_workspace_bytes(n_experts: int, n_ids: int, n_tokens: int) -> int:
    return int(lib().qmm_matmul_id_workspace_bytes(int(n_experts), int(n_ids), int(n_tokens)))


def qmm_matmul_id_workspace_bytes_x16(n_experts: int, n_ids: int, n_tokens: int, k: int, x_slots: int) -> int:
    return int(lib().qmm_matmul_id_workspace_bytes_x16(int(n_experts), int(n_ids), int(n_tokens), int(k),
                                                       int(x_slots)))


def _matmul_id_args(W, ggml_type, k, X, ids, n_experts, n_rows, row_stride_bytes, expert_stride_bytes, Y):
    """Geometry and checked buffers of a MUL_MAT_ID call (shared by both entry points)."""
    import torch
    if W.dtype != torch.uint8:
        raise TypeError("W must be a uint8 tensor of raw blocks")
    if any(v is None for v in (n_experts, n_rows, row_stride_bytes, expert_stride_bytes)):
        if W.dim() != 3 or not W.is_contiguous():
            raise ValueError("pass the geometry for a W that is not a contiguous [experts][rows][nb1] tensor")
        n_experts, n_rows, row_stride_bytes = W.shape
        expert_stride_bytes = n_rows * row_stride_bytes
    if X.dtype != torch.float32 or X.dim() != 3 or not X.is_contiguous():
        raise TypeError("X must be a contiguous float32 [n_tokens][x_slots][k] tensor")
    if ids.dtype != torch.int32 or ids.dim() != 2 or not ids.is_contiguous():
        raise TypeError("ids must be a contiguous int32 [n_tokens][n_ids] tensor")
    n_tokens, n_ids = int(ids.shape[0]), int(ids.shape[1])
    if int(X.shape[0]) != n_tokens or int(X.shape[2]) != int(k):
        raise ValueError("X must be [n_tokens][x_slots][k] with the n_tokens of ids")
    if Y is None:
        Y = torch.empty((n_tokens, n_ids, int(n_rows)), dtype=torch.float32, device=X.device)
    _check_span(W, torch.uint8, _weights_span(ggml_type, k, int(n_rows), int(row_stride_bytes), int(n_experts),
                                              int(expert_stride_bytes)), "W")
    _check_span(Y, torch.float32, n_tokens * n_ids * int(n_rows), "Y")
    geo = (int(n_experts), int(n_rows), int(k), int(row_stride_bytes), int(expert_stride_bytes))
    return geo, n_ids, n_tokens, Y


def qmm_matmul_id(W, ggml_type, k, X, ids, n_experts=None, n_rows=None, row_stride_bytes=None,
                  expert_stride_bytes=None, Y=None, workspace=None, stream=None):
    """MUL_MAT_ID (C: qmm_matmul_id): Y[t][i] = MUL_MAT(expert ids[t][i], X[t][i or 0]).

    W is a contiguous uint8 [n_experts][n_rows][nb1] GPU tensor, or any uint8
    GPU tensor with the four geometry arguments given. X is a contiguous fp32
    [n_tokens][x_slots][k] tensor (x_slots 1 or n_ids), ids a contiguous int32
    [n_tokens][n_ids] tensor; Y (fp32 [n_tokens][n_ids][n_rows]) is allocated
    if None. An id outside [0, n_experts) gives a row of NaNs. Without a
    workspace, one of qmm_matmul_id_workspace_bytes_x16 bytes is allocated
    (the fastest route); a given workspace needs at least
    qmm_matmul_id_workspace_bytes."""
    import torch
    geo, n_ids, n_tokens, Y = _matmul_id_args(W, ggml_type, k, X, ids, n_experts, n_rows, row_stride_bytes,
                                              expert_stride_bytes, Y)
    if workspace is None:
        need = qmm_matmul_id_workspace_bytes_x16(geo[0], n_ids, n_tokens, int(k), int(X.shape[1]))
    else:
        need = qmm_matmul_id_workspace_bytes(geo[0], n_ids, n_tokens)
    if need < 0:
        raise QmmError(need, "qmm_matmul_id_workspace_bytes")
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws = _gpu_ptr(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    e, r, kk, nb1, nb2 = geo
    st = lib().qmm_matmul_id(_gpu_ptr(W, "W"), int(ggml_type), e, r, kk, nb1, nb2, _gpu_ptr(X, "X"), int(X.shape[1]),
                             _gpu_ptr(ids, "ids"), n_ids, n_tokens, _gpu_ptr(Y, "Y"), ws, ws_bytes, _stream(stream))
    if st != QMM_OK:
        raise QmmError(st, "qmm_matmul_id")
    return Y


def qmm_matmul_id_noalloc(W, ggml_type, k, X, ids, n_experts=None, n_rows=None, row_stride_bytes=None,
                          expert_stride_bytes=None, Y=None, stream=None):
    """MUL_MAT_ID on the library's own per-GPU scratch (C: qmm_matmul_id_noalloc):
    the same arguments and result as qmm_matmul_id, no workspace. Pass a
    preallocated Y to keep the call free of allocations."""
    geo, n_ids, n_tokens, Y = _matmul_id_args(W, ggml_type, k, X, ids, n_experts, n_rows, row_stride_bytes,
                                              expert_stride_bytes, Y)
    e, r, kk, nb1, nb2 = geo
    st = lib().qmm_matmul_id_noalloc(_gpu_ptr(W, "W"), int(ggml_type), e, r, kk, nb1, nb2, _gpu_ptr(X, "X"),
                                     int(X.shape[1]), _gpu_ptr(ids, "ids"), n_ids, n_tokens, _gpu_ptr(Y, "Y"),
                                     _stream(stream))
    if st != QMM_OK:
        raise QmmError(st, "qmm_matmul_id_noalloc")
    return Y


def _batch_descs(items):
    import torch
    arr = (qmm_matmul_desc * max(1, len(items)))()
    for i, (W, t, k, X, Y) in enumerate(items):
        rows, nb1 = _weights_geometry(W, None, None)
        if X.dtype not in (torch.float32, torch.float16):
            raise TypeError("X must be float32 or float16")
        _check_span(X, X.dtype, int(X.shape[0]) * int(k), "X")
        _check_span(Y, torch.float32, int(X.shape[0]) * rows, "Y")
        arr[i] = qmm_matmul_desc(_gpu_ptr(W, "W").value, int(t), rows, int(k), nb1, _gpu_ptr(X, "X").value,
                                 QMM_X_F16 if X.dtype == torch.float16 else QMM_X_F32, int(X.shape[0]),
                                 _gpu_ptr(Y, "Y").value)
    return arr


def qmm_matmul_batch(items, stream=None):
    """Independent MUL_MATs in one call (C: qmm_matmul_batch).

    items: sequence of (W, ggml_type, k, X, Y) with W a contiguous uint8
    [rows][nb1] GPU tensor, X a contiguous fp32/fp16 [n_tokens][k] GPU tensor
    and Y a preallocated fp32 [n_tokens][rows] GPU tensor. Returns the Ys.
    """
    st = lib().qmm_matmul_batch(_batch_descs(items), len(items), _stream(stream))
    if st != QMM_OK:
        raise QmmError(st, "qmm_matmul_batch")
    return [it[4] for it in items]


def qmm_matmul_batch_workspace_bytes(items) -> int:
    """Workspace qmm_matmul_batch_ws needs for these items (C:
    qmm_matmul_batch_workspace_bytes); items as in qmm_matmul_batch."""
    n = int(lib().qmm_matmul_batch_workspace_bytes(_batch_descs(items), len(items)))
    if n < 0:
        raise QmmError(n, "qmm_matmul_batch_workspace_bytes")
    return n


def qmm_matmul_batch_ws(items, workspace, stream=None):
    """qmm_matmul_batch with a caller workspace that lets its matrix-core
    launches split k (C: qmm_matmul_batch_ws). `workspace` is a GPU uint8
    tensor of at least qmm_matmul_batch_workspace_bytes(items) bytes that held
    zeros when first used, or None when that size is 0. Returns the Ys."""
    import torch
    if workspace is not None:
        _check_span(workspace, torch.uint8, 0, "workspace")
    ws = _gpu_ptr(workspace, "workspace") if workspace is not None else ctypes.c_void_p(0)
    ws_bytes = workspace.numel() if workspace is not None else 0
    st = lib().qmm_matmul_batch_ws(_batch_descs(items), len(items), ws, ws_bytes, _stream(stream))
    if st != QMM_OK:
        raise QmmError(st, "qmm_matmul_batch_ws")
    return [it[4] for it in items]
