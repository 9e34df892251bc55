"""Q4_K on the GPU: the block decoder bit for bit, GET_ROWS, MUL_MAT on the
decode and matrix-core kernels element by element within
|y - y_ref| <= 1e-3 * sum|w x| + 1e-5, and MUL_MAT_ID on each of its routes,
all against the oracle's reading of the Q4_K super-block."""
import numpy as np
import pytest
import torch

import block_quantized_matmul_amd as qmm
import oracle.qmm_oracle as O
from block_quantized_matmul_amd import synth
from gpu_util import assert_bitwise, assert_close_to_oracle, dev, run_dequant, run_matmul, say

pytestmark = pytest.mark.gpu
QK4 = O.TYPE_Q4_K
GEMV, GEMM, AUTO = qmm.QMM_PATH_GEMV, qmm.QMM_PATH_GEMM, qmm.QMM_PATH_AUTO


def _weights(rows, k, extra=0, seed=0):
    rng = np.random.Generator(np.random.PCG64([seed, rows, k, extra, 12]))
    return synth.make_weights(QK4, rows, k, synth.dense_row_bytes(QK4, k) + extra, rng), rng


@pytest.mark.parametrize("rows,k,extra", [(1, 256, 0), (37, 512, 16), (300, 4096, 0), (17, 11008, 48)])
def test_dequant_bit_exact(rows, k, extra):
    W, _ = _weights(rows, k, extra)
    say(f"q4_k dequant rows={rows} k={k} nb1={W.shape[1]}")
    assert_bitwise(run_dequant(W, QK4, k), O.dequantize(W, QK4, rows, k, W.shape[1]), "q4_k dequant")


@pytest.mark.parametrize("field", [0, 2])
def test_dequant_every_d_and_dmin_pattern(field):
    """65536 super-blocks: block i has d (field 0) or dmin (field 2) bits i,
    so every binary16 value, subnormals, infinities and NaNs included, goes
    through the decoder; NaN positions must match the oracle's."""
    rows, k = 2048, 256 * 32
    W, _ = _weights(rows, k, seed=7 + field)
    blk = W.reshape(rows, 32, 144)
    pat = np.arange(65536, dtype=np.uint16).reshape(rows, 32)
    blk[:, :, field:field + 2] = pat.view(np.uint8).reshape(rows, 32, 2)
    say(f"q4_k dequant every {'d' if field == 0 else 'dmin'} pattern")
    assert_bitwise(run_dequant(W, QK4, k), O.dequantize(W, QK4, rows, k, W.shape[1]), "q4_k patterns")


def test_get_rows():
    rows, k = 300, 512
    W, rng = _weights(rows, k, 16)
    ids = rng.integers(0, rows, 64).astype(np.int32)
    ids[:4] = [0, rows - 1, -1, rows]
    say("q4_k get_rows")
    out = qmm.qmm_get_rows(dev(W), QK4, k, dev(ids))
    torch.cuda.synchronize()
    assert_bitwise(out.cpu().numpy(), O.get_rows(W, QK4, rows, k, W.shape[1], ids), "q4_k get_rows")


@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8])
def test_decode_kernel(xdt, n):
    for rows, k, extra in ((1, 256, 0), (37, 512, 16), (300, 4096, 32), (17, 11008, 0), (4112, 512, 0)):
        W, rng = _weights(rows, k, extra, seed=n)
        X = synth.make_activations(n, k, rng, xdt)
        say(f"q4_k gemv rows={rows} k={k} nb1={W.shape[1]} n={n} x={np.dtype(xdt).name}")
        assert_close_to_oracle(run_matmul(W, QK4, k, X, GEMV), W, QK4, k, X, "q4_k gemv")


@pytest.mark.parametrize("xdt", [np.float16, np.float32])
@pytest.mark.parametrize("rows,k,n", [(37, 256, 9), (300, 512, 37), (129, 4096, 200), (4230, 512, 1030),
                                      (1000, 1024, 300)])
def test_gemm_kernel(xdt, rows, k, n):
    """64-row tiles with the in-workgroup k split (k = 512, 1024, 4096), the
    k = 256 case without it, and 128-row tiles (more tiles than CUs)."""
    W, rng = _weights(rows, k, 16)
    X = synth.make_activations(n, k, rng, xdt)
    say(f"q4_k gemm rows={rows} k={k} n={n} x={np.dtype(xdt).name}")
    assert_close_to_oracle(run_matmul(W, QK4, k, X, GEMM), W, QK4, k, X, "q4_k gemm")


@pytest.mark.parametrize("rows,k,n,extra", [(2000, 512, 4000, 16), (11003, 256, 505, 0), (1500, 1024, 3900, 0)])
def test_gemm_two_group_tiles(rows, k, n, extra):
    """fp16 activations with 128 x 256 tiles for at least 2/3 of the CUs:
    the two-group kernel decodes whole super-blocks per pair of 64-wide
    stages; every element against the oracle, and bitwise the same as the
    fp32 copy of the activations on the one-group kernel."""
    assert ((rows + 127) // 128) * ((n + 255) // 256) in (172, 192, 256)
    W, rng = _weights(rows, k, extra, seed=3)
    X = synth.make_activations(n, k, rng, np.float16)
    say(f"q4_k gemm two-group rows={rows} k={k} n={n} nb1={W.shape[1]}")
    Y = run_matmul(W, QK4, k, X, GEMM)
    assert_close_to_oracle(Y, W, QK4, k, X, "q4_k gemm two-group")
    say("fp32 copy of the activations")
    assert_bitwise(run_matmul(W, QK4, k, X.astype(np.float32), GEMM), Y, "q4_k one-group vs two-group")


def test_zero_scales_and_mins_give_zero():
    rows, k = 64, 512
    W, rng = _weights(rows, k)
    W.reshape(rows, 2, 144)[:, :, 4:16] = 0   # every sc_j = m_j = 0
    X = synth.make_activations(20, k, rng)
    for path, n in ((GEMV, 3), (GEMM, 20)):
        say(f"q4_k zero scales path={path}")
        assert np.all(run_matmul(W, QK4, k, X[:n], path) == 0.0)


def test_gemv_and_gemm_agree_with_each_other():
    rows, k = 300, 1024
    W, rng = _weights(rows, k)
    X = synth.make_activations(8, k, rng)
    say("q4_k gemv vs gemm")
    y1 = run_matmul(W, QK4, k, X, GEMV)
    y2 = run_matmul(W, QK4, k, X, GEMM)
    y_ref, s = O.matmul(W, QK4, rows, k, W.shape[1], X)
    assert O.within_tolerance(y1, y_ref, s).all() and O.within_tolerance(y2, y_ref, s).all()
    assert np.all(np.abs(y1 - y2) <= 2e-3 * s + 2e-5)


@pytest.mark.parametrize("n_tokens,n_ids,n_experts", [(1, 2, 4), (8, 2, 4), (300, 2, 8)])
@pytest.mark.parametrize("shared_x", [False, True])
def test_matmul_id_routes(n_tokens, n_ids, n_experts, shared_x):
    """One token (per-pair decode), 8 tokens over 4 experts (decode tiles) and
    300 tokens (the routed matrix-core kernel); one id names no expert."""
    rows, k = 96, 512
    nb1 = synth.dense_row_bytes(QK4, k)
    rng = np.random.Generator(np.random.PCG64([n_tokens, n_ids, n_experts, int(shared_x)]))
    Wn = synth.make_weights(QK4, n_experts * rows, k, nb1, rng)
    slots = 1 if shared_x else n_ids
    Xn = synth.make_activations(n_tokens * slots, k, rng).reshape(n_tokens, slots, k)
    ids = np.stack([rng.permutation(n_experts)[:n_ids] for _ in range(n_tokens)]).astype(np.int32)
    ids[0, 0] = n_experts
    say(f"q4_k matmul_id tokens={n_tokens} ids={n_ids} experts={n_experts} shared_x={shared_x}")
    Y = qmm.qmm_matmul_id(dev(Wn).view(n_experts, rows, nb1), QK4, k, dev(Xn), dev(ids))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    y_ref, s = O.matmul_id(Wn.reshape(n_experts, rows * nb1), QK4, n_experts, rows, k, nb1, rows * nb1, Xn, ids)
    ok = O.within_tolerance(Y, y_ref, s)
    assert ok.all(), f"{int((~ok).sum())} of {ok.size} outside tolerance"
