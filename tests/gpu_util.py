"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
call the library through its C ABI, and compare with the oracle."""
import sys

import numpy as np
import torch

import block_quantized_matmul_amd as qmm
import oracle.qmm_oracle as O


def say(msg):
    """Name the case before each GPU step (and flush), so a failure names it."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def place_weights(Wnp: np.ndarray, offset: int = 0) -> tuple:
    """Copy W rows to the GPU starting `offset` bytes into a fresh buffer
    (offset 2 gives a 2-byte-aligned W). Returns (keepalive buffer, view)."""
    flat = np.ascontiguousarray(Wnp).reshape(-1)
    buf = torch.zeros(flat.size + offset + 16, dtype=torch.uint8, device="cuda")
    buf[offset:offset + flat.size] = dev(flat)
    return buf, buf[offset:offset + flat.size]


def run_matmul(Wnp, qtype, k, Xnp, path=qmm.QMM_PATH_AUTO, w_offset=0):
    rows, nb1 = Wnp.shape
    _buf, W = place_weights(Wnp, w_offset)
    X = dev(Xnp)
    Y = qmm.qmm_matmul_path(W, qtype, k, X, n_rows=rows, row_stride_bytes=nb1, n_tokens=Xnp.shape[0], path=path)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def run_dequant(Wnp, qtype, k, w_offset=0):
    rows, nb1 = Wnp.shape
    _buf, W = place_weights(Wnp, w_offset)
    out = qmm.qmm_dequantize(W, qtype, k, n_rows=rows, row_stride_bytes=nb1)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_close_to_oracle(Y, Wnp, qtype, k, Xnp, what=""):
    rows, nb1 = Wnp.shape
    y_ref, s = O.matmul(Wnp, qtype, rows, k, nb1, Xnp)
    ok = O.within_tolerance(Y, y_ref, s)
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        det = [(int(t), int(r), float(Y[t, r]), float(y_ref[t, r]), float(s[t, r])) for t, r in bad]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; first (t, r, y, ref, s): {det}")
    return worst_ratio(Y, y_ref, s)


def worst_ratio(Y, y_ref, s):
    fin = np.isfinite(y_ref)
    if not fin.any():
        return 0.0
    return float(np.max(np.abs(Y[fin] - y_ref[fin]) / (1e-3 * s[fin] + 1e-5)))


def assert_bitwise(got, want, what=""):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, what
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), f"{what}: NaN positions differ"
    g, w = got[~nan].view(np.uint32), want[~nan].view(np.uint32)
    if not np.array_equal(g, w):
        i = int(np.argmax(g != w))
        raise AssertionError(f"{what}: {int((g != w).sum())} elements differ, e.g. {got[~nan][i]!r} vs {want[~nan][i]!r}")
