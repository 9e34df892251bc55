"""The row-split decode kernel for tall matrices at 3 to 8 tokens (128-row
workgroups, activations staged once per workgroup in chunks of up to 64 KiB):
element by element against the oracle at ragged row counts for every type
and both activation types, across activation chunk boundaries, on the full
32000 x 4096 output projection at 8 tokens, and repeatable bit for bit."""
import numpy as np
import pytest
import torch

import block_quantized_matmul_amd as qmm
import oracle.qmm_oracle as O
from block_quantized_matmul_amd import synth
from gpu_util import assert_bitwise, assert_close_to_oracle, run_matmul, say

pytestmark = pytest.mark.gpu
Q4, Q41, Q50, Q51, Q8, QK = (O.TYPE_Q4_0, O.TYPE_Q4_1, O.TYPE_Q5_0, O.TYPE_Q5_1, O.TYPE_Q8_0,
                             qmm.QMM_TYPE_Q4_K)


def _tall_rows(extra=5):
    """Fewest rows (plus `extra`) for which the library takes the row-split
    kernel: 128-row tiles numbering at least 7/8 of the compute units."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = (7 * cus + 7) // 8
    return 128 * (tiles - 1) + extra


def _inputs(qtype, rows, k, n, seed, xdt=np.float32, extra=0):
    rng = np.random.Generator(np.random.PCG64([seed, qtype, rows, k, n, 91]))
    nb1 = synth.dense_row_bytes(qtype, k) + extra
    return synth.make_weights(qtype, rows, k, nb1, rng), synth.make_activations(n, k, rng, xdt)


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8, QK])
@pytest.mark.parametrize("n", [3, 8])
def test_tall_every_type(qtype, n):
    rows = _tall_rows()
    W, X = _inputs(qtype, rows, 512, n, 1, extra=16)
    say(f"tall type={qtype} rows={rows} k=512 n={n}")
    assert_close_to_oracle(run_matmul(W, qtype, 512, X), W, qtype, 512, X, f"tall type {qtype} n {n}")


@pytest.mark.parametrize("n", [3, 4, 5, 6, 7])
@pytest.mark.parametrize("xdt", [np.float32, np.float16])
def test_tall_token_counts(n, xdt):
    rows = _tall_rows(extra=77)
    W, X = _inputs(Q4, rows, 768, n, 2, xdt)
    say(f"tall q4_0 rows={rows} k=768 n={n} x={np.dtype(xdt).name}")
    assert_close_to_oracle(run_matmul(W, Q4, 768, X), W, Q4, 768, X, f"tall n {n}")


@pytest.mark.parametrize("qtype,n,k", [(Q4, 8, 4864), (Q4, 4, 8448), (Q8, 8, 4352), (Q51, 5, 8704)])
def test_tall_activation_chunks(qtype, n, k):
    """k longer than one staged chunk (4096 activations at 8 token slots, 8192
    at 4): the stream of weights runs on across the chunk boundary."""
    rows = _tall_rows(extra=3)
    W, X = _inputs(qtype, rows, k, n, 3)
    say(f"tall chunks type={qtype} rows={rows} k={k} n={n}")
    Y = run_matmul(W, qtype, k, X)
    rng = np.random.default_rng(k)
    rr = np.concatenate([np.arange(16), np.arange(rows - 16, rows), rng.integers(0, rows, 4000)])
    tt = rng.integers(0, n, rr.size)
    y_ref, s = O.matmul_sampled(W, qtype, rows, k, W.shape[1], X, tt, rr)
    assert O.within_tolerance(Y[tt, rr], y_ref, s).all()


def test_output_projection_full_at_8_tokens():
    """The 32000 x 4096 (nb1 = 2560, random padding) output projection at 8
    fp32 tokens, every element against the oracle, and a second run equal bit
    for bit."""
    case = synth.config_cases()[3][-1]
    assert case.n_tokens == 8
    W, X = case.weights(), case.activations()
    say(case.name)
    Y = run_matmul(W, case.qtype, case.k, X)
    assert_close_to_oracle(Y, W, case.qtype, case.k, X, case.name)
    assert_bitwise(run_matmul(W, case.qtype, case.k, X), Y, "repeat")
