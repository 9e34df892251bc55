"""MUL_MAT_ID parity: the expert-routed decode against the oracle's
matmul_id, within the MUL_MAT tolerance, with NaN rows exactly where an id
names no expert. Covers both decode kernels (the streaming layout and a
padded, 2-byte-aligned one), activations shared by all slots or one per
slot, repeated ids, ragged row counts and more pairs than one launch's grid
holds."""
import numpy as np
import pytest

import oracle.qmm_oracle as O
from block_quantized_matmul_amd import synth
from gpu_util import dev, say

pytestmark = pytest.mark.gpu
Q4, Q8 = O.TYPE_Q4_0, O.TYPE_Q8_0


def _stack(qtype, n_experts, rows, k, nb1, nb2, rng):
    """n_experts matrices of seeded blocks, expert e at byte e * nb2; the
    bytes between experts are random too (they must never be read)."""
    W = rng.integers(0, 256, size=(n_experts, nb2), dtype=np.uint8)
    for e in range(n_experts):
        W[e, :rows * nb1] = synth.make_weights(qtype, rows, k, nb1, rng).reshape(-1)
    return W


def _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset=0):
    import torch
    import block_quantized_matmul_amd as qmm
    from gpu_util import place_weights
    _keep, Wd = place_weights(W, offset)
    Y = qmm.qmm_matmul_id(Wd, qtype, k, dev(X), dev(ids), n_experts=n_experts, n_rows=rows, row_stride_bytes=nb1,
                          expert_stride_bytes=nb2)
    torch.cuda.synchronize()
    return Y.cpu().numpy()


def _check(Y, y_ref, s, what):
    nan = np.isnan(y_ref)
    assert np.array_equal(np.isnan(Y), nan), f"{what}: NaN rows differ"
    ok = O.within_tolerance(Y[~nan], y_ref[~nan], s[~nan])
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance"


@pytest.mark.parametrize("qtype", [Q4, Q8])
@pytest.mark.parametrize("layout", ["stream", "general"])
@pytest.mark.parametrize("shared_x", [False, True])
@pytest.mark.parametrize("n_tokens", [1, 3])
def test_matmul_id_small(qtype, layout, shared_x, n_tokens):
    rng = np.random.Generator(np.random.PCG64([500, qtype, n_tokens, int(shared_x), len(layout)]))
    n_experts, n_ids, rows, k = 8, 2, 200, 512
    dense = synth.dense_row_bytes(qtype, k)
    if layout == "stream":   # 16-byte rows and expert stride, 16-aligned base
        nb1, nb2, offset = dense, rows * dense + 64, 0
    else:                    # padded rows, odd-half-word base: the general kernel
        nb1, nb2, offset = dense + 2, rows * (dense + 2) + 6, 2
    W = _stack(qtype, n_experts, rows, k, nb1, nb2, rng)
    X = synth.make_activations(n_tokens * (1 if shared_x else n_ids), k, rng, np.float32)
    X = X.reshape(n_tokens, 1 if shared_x else n_ids, k)
    ids = rng.integers(0, n_experts, size=(n_tokens, n_ids)).astype(np.int32)
    ids[0] = [n_experts - 1, n_experts - 1]        # the last expert, twice
    if n_tokens > 1:
        ids[1] = [-1, 0]                           # no expert, the first expert
        ids[2, 1] = n_experts                      # one past the last
    say(f"matmul_id {layout} type={qtype} tokens={n_tokens} x_slots={X.shape[1]} ids={ids.tolist()}")
    Y = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset)
    y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
    _check(Y, y_ref, s, f"matmul_id {layout}")


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_matmul_id_more_pairs_than_one_grid(qtype):
    """70000 pairs (over the 65535 grid rows of one launch): tokens are
    independent, so a sample of them, from both launches, is checked."""
    rng = np.random.Generator(np.random.PCG64([501, qtype]))
    n_experts, n_ids, rows, k, n_tokens = 4, 2, 24, 256, 35000
    nb1 = synth.dense_row_bytes(qtype, k)
    nb2 = rows * nb1
    W = _stack(qtype, n_experts, rows, k, nb1, nb2, rng)
    X = synth.make_activations(n_tokens * n_ids, k, rng).reshape(n_tokens, n_ids, k)
    ids = rng.integers(-1, n_experts, size=(n_tokens, n_ids)).astype(np.int32)
    say(f"matmul_id pairs={n_tokens * n_ids} type={qtype}")
    Y = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
    sample = np.unique(np.concatenate([[0, 32767, 32768, n_tokens - 1], rng.integers(0, n_tokens, 60)]))
    y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X[sample], ids[sample])
    _check(Y[sample], y_ref, s, "matmul_id many pairs")


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_matmul_id_mixtral_sized_sampled(qtype):
    """Decode of one token through 8 experts of 14336 x 4096 with 2 selected,
    the routed-FFN shape the bench times; sampled rows of each selected
    expert against the oracle."""
    import torch
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([502, qtype]))
    n_experts, rows, k, n_ids = 8, 14336, 4096, 2
    nb1 = synth.dense_row_bytes(qtype, k)
    Wn = synth.make_weights(qtype, n_experts * rows, k, nb1, rng)
    X = synth.make_activations(1, k, rng, np.float32).reshape(1, 1, k)
    ids = np.array([[5, 2]], np.int32)
    say(f"matmul_id experts={n_experts} rows={rows} k={k} type={qtype}")
    W = dev(Wn.reshape(n_experts, rows, nb1))
    Y = qmm.qmm_matmul_id(W, qtype, k, dev(X), dev(ids))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    rsamp = np.unique(np.concatenate([[0, 15, 16, rows - 1], rng.integers(0, rows, 200)]))
    for i, e in enumerate(ids[0]):
        We = Wn[e * rows:(e + 1) * rows]
        y_ref, s = O.matmul_sampled(We, qtype, rows, k, nb1, X[0], np.zeros_like(rsamp), rsamp)
        ok = O.within_tolerance(Y[0, i, rsamp], y_ref, s)
        assert ok.all(), f"expert {e}: {int((~ok).sum())} sampled rows outside tolerance"
