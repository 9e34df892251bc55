"""MUL_MAT at the numeric edges of its fp16 matrix-core operands, against the
oracle: worst-case rounding on the matrix-core path with fp32 activations,
scales in the fp16 subnormal range, weights that cancel to subnormals,
activations below and beyond fp16's normal range (the documented behaviour
in each case)."""
import numpy as np
import pytest

import block_quantized_matmul_amd as qmm
import oracle.qmm_oracle as O
from block_quantized_matmul_amd import synth
from gpu_util import run_matmul, say

pytestmark = pytest.mark.gpu
Q4 = O.TYPE_Q4_0
GEMV, GEMM = qmm.QMM_PATH_GEMV, qmm.QMM_PATH_GEMM


def _q4_rows(d_bits, codes_byte, rows, k):
    nblk = k // 32
    d = np.full((rows, nblk), d_bits, np.uint16)
    codes = np.full((rows, nblk, 16), codes_byte, np.uint8)
    return synth.assemble_rows(d, codes, synth.dense_row_bytes(Q4, k))


def test_gemm_fp32_activations_worst_case_rounding():
    """Every weight d (q - 8) = 293 * 2^-11 * 7 = 1 + 3 * 2^-11 and every
    activation x = 1 + 3 * 2^-11 (exact in fp32) lie half-way between two
    fp16 neighbours and round up to 1 + 2^-9 (round to nearest even), so
    every product of the matrix-core path is 2 * 2^-11 / (1 + 3 * 2^-11)
    ~ 9.74e-4 too large, all with the same sign, over k = 11008."""
    rows, k, n = 256, 11008, 16
    d = np.float16(293 * 2.0 ** -11)
    assert float(d) * 7 == 1 + 3 * 2.0 ** -11
    W = _q4_rows(d.view(np.uint16), 0xFF, rows, k)          # every code 15: q - 8 = 7
    X = np.full((n, k), 1 + 3 * 2.0 ** -11, np.float32)
    say("gemm worst-case fp16 rounding k=11008 fp32 x")
    y = run_matmul(W, Q4, k, X, GEMM)
    y_ref, s = O.matmul(W, Q4, rows, k, W.shape[1], X)
    rel = np.abs(y - y_ref) / s
    assert O.within_tolerance(y, y_ref, s).all(), f"worst relative error {rel.max():.3e}"
    # the rounding really is the worst case (not absorbed by the accumulation)
    assert rel.min() > 9.5e-4


def test_gemm_subnormal_scales_zero_point_type():
    """Scales in the fp16 subnormal range: d is a multiple of 2^-24, so every
    d (q - 8) is too and is stored exactly by the matrix-core path; the plain
    bound holds (here mainly through its absolute term, the values being
    tiny), on both kernels."""
    rows, k, n = 300, 4096, 24
    rng = np.random.Generator(np.random.PCG64(31))
    W = synth.make_weights(Q4, rows, k, None, rng, d_lo=2.0 ** -22, d_hi=2.0 ** -15)
    X = synth.make_activations(n, k, rng) * np.float32(1000.0)
    for path, m in ((GEMM, n), (GEMV, 4)):
        say(f"subnormal scales path={path}")
        y = run_matmul(W, Q4, k, X[:m], path)
        y_ref, s = O.matmul(W, Q4, rows, k, W.shape[1], X[:m])
        assert O.within_tolerance(y, y_ref, s).all()


def test_gemm_min_offset_cancellation():
    """Q4_1 blocks whose minimum nearly cancels d q (m = -d * 8 + a tiny
    remainder): weights d q + m near zero fall into the fp16 subnormal range
    on the matrix-core path, whose rounding is then absolute (at most 2^-25
    per weight) instead of relative, so the bound there is
    1e-3 s + 1e-5 + 2^-25 sum |x| (documented)."""
    Q41 = O.TYPE_Q4_1
    rows, k, n = 128, 2048, 16
    rng = np.random.Generator(np.random.PCG64(33))
    nblk = k // 32
    d = np.full((rows, nblk), np.float16(2.0 ** -12))
    m = (-8 * d.astype(np.float64) + rng.uniform(-2.0 ** -18, 2.0 ** -18, (rows, nblk))).astype(np.float16)
    payload = np.empty((rows, nblk, 18), np.uint8)
    payload[:, :, 0:2] = m.view(np.uint8).reshape(rows, nblk, 2)
    payload[:, :, 2:] = rng.integers(0, 256, (rows, nblk, 16), dtype=np.uint8)
    W = synth.assemble_rows(d.view(np.uint16), payload, synth.dense_row_bytes(Q41, k))
    X = synth.make_activations(n, k, rng) * np.float32(100.0)
    say("gemm q4_1 cancelling minimum")
    y = run_matmul(W, Q41, k, X, GEMM)
    y_ref, s = O.matmul(W, Q41, rows, k, W.shape[1], X)
    sx = np.abs(X.astype(np.float64)).sum(axis=1, keepdims=True)
    assert np.all(np.abs(y - y_ref) <= 1e-3 * s + 1e-5 + 2.0 ** -25 * sx)


@pytest.mark.parametrize("path", [GEMV, GEMM])
def test_tiny_activations(path):
    """Activations below 2^-14 are fp16 subnormals: both kernels round them
    to the nearest multiple of 2^-24 (absolute error at most 2^-25), so the
    bound is 1e-3 s + 1e-5 + 2^-25 sum |w| (documented). With x = 3e-8 and
    weights of magnitude 7 the plain bound alone would fail."""
    rows, k = 64, 4096
    nblk = k // 32
    W = synth.assemble_rows(np.full((rows, nblk), 0x3C00, np.uint16), np.full((rows, nblk, 16), 0xFF, np.uint8),
                            synth.dense_row_bytes(Q4, k))        # d = 1, every weight 7
    n = 2 if path == GEMV else 16
    X = np.full((n, k), 3e-8, np.float32)
    say(f"tiny activations path={path}")
    y = run_matmul(W, Q4, k, X, path)
    y_ref, s = O.matmul(W, Q4, rows, k, W.shape[1], X)
    sw = 7.0 * k
    assert np.all(np.abs(y - y_ref) <= 1e-3 * s + 1e-5 + 2.0 ** -25 * sw)
    assert not O.within_tolerance(y, y_ref, s).all()


def test_decode_activations_beyond_fp16_range():
    """The decode kernel rounds activations to fp16, so an activation beyond
    65504 becomes infinite and every output of that token becomes non-finite
    (documented); the other tokens are unaffected."""
    rows, k = 64, 512
    rng = np.random.Generator(np.random.PCG64(32))
    W = synth.make_weights(Q4, rows, k, None, rng)
    X = synth.make_activations(3, k, rng)
    X[1, 100] = 70000.0
    say("gemv activation beyond fp16 range")
    y = run_matmul(W, Q4, k, X, GEMV)
    assert not np.isfinite(y[1]).any()
    y_ref, s = O.matmul(W, Q4, rows, k, W.shape[1], X[[0, 2]])
    assert O.within_tolerance(y[[0, 2]], y_ref, s).all()
