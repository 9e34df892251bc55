"""qmm_matmul_id_noalloc against qmm_matmul_id on the GPU.

The no-allocation entry point runs the same routes and kernels as
qmm_matmul_id with its routing table in the library's per-GPU scratch
array instead of a caller workspace, so its output must equal
qmm_matmul_id's bit for bit (each output element is the same fixed-order
sum whatever the tile order), and lie within the tolerance of the oracle.
Two calls in a row, the second with a smaller input, check that the scratch
left by the first call does not leak into the second.
"""
import numpy as np
import pytest
import torch

import block_quantized_matmul_amd as qmm
from block_quantized_matmul_amd import synth
import oracle.qmm_oracle as O
from gpu_util import assert_bitwise, dev, say

pytestmark = pytest.mark.gpu

Q4 = qmm.QMM_TYPE_Q4_0


def _case(E, rows, k, n_tokens, n_ids, x_slots, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    nb1 = synth.dense_row_bytes(Q4, k)
    Wn = synth.make_weights(Q4, E * rows, k, nb1, rng)
    Xn = synth.make_activations(n_tokens * x_slots, k, rng).reshape(n_tokens, x_slots, k)
    ids = np.stack([rng.permutation(E)[:n_ids] for _ in range(n_tokens)]).astype(np.int32)
    ids[0, 0] = E + 3  # one invalid id: a NaN row
    return Wn, Xn, ids, nb1


def _both(Wn, Xn, ids, E, rows, k, nb1):
    W = dev(Wn).view(E, rows, nb1)
    X, I = dev(Xn), dev(ids)
    Ya = torch.full((ids.shape[0], ids.shape[1], rows), 7.0, dtype=torch.float32, device="cuda")
    Yb = torch.full_like(Ya, -7.0)
    qmm.qmm_matmul_id(W, Q4, k, X, I, Y=Ya)
    qmm.qmm_matmul_id_noalloc(W, Q4, k, X, I, Y=Yb)
    torch.cuda.synchronize()
    return Ya.cpu().numpy(), Yb.cpu().numpy()


def _check(Ya, Yb, Wn, Xn, ids, E, rows, k, nb1, what):
    assert_bitwise(Yb, Ya, what)
    y_ref, s = O.matmul_id(Wn.reshape(E, rows * nb1), Q4, E, rows, k, nb1, rows * nb1, Xn, ids)
    ok = O.within_tolerance(Yb, y_ref, s)
    assert ok.all(), f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance"


# (experts, rows, k, [(tokens, n_ids, x_slots) first call, second smaller call]):
# the 128-pair matrix-core tiles, the decode tiles and the per-pair route
ROUTES = [
    ("gemm", 8, 256, 512, [(200, 2, 1), (40, 2, 2)]),
    ("tiles", 8, 256, 512, [(8, 2, 1), (4, 2, 2)]),
    ("per_pair", 8, 128, 256, [(3, 2, 1), (1, 2, 1)]),
]


@pytest.mark.parametrize("name,E,rows,k,calls", ROUTES, ids=[r[0] for r in ROUTES])
def test_noalloc_matches_workspace_entry_point(name, E, rows, k, calls):
    for i, (n, n_ids, xs) in enumerate(calls):
        say(f"noalloc {name} call {i}: experts={E} rows={rows} k={k} tokens={n} ids={n_ids} x_slots={xs}")
        Wn, Xn, ids, nb1 = _case(E, rows, k, n, n_ids, xs, 900 + 10 * i + len(name))
        Ya, Yb = _both(Wn, Xn, ids, E, rows, k, nb1)
        _check(Ya, Yb, Wn, Xn, ids, E, rows, k, nb1, f"{name} call {i}")


def test_noalloc_refuses_oversized_call_without_launch():
    say("noalloc oversized call")
    E, rows, k = 8, 16, 64
    nb1 = synth.dense_row_bytes(Q4, k)
    n = 200000
    W = torch.zeros((E, rows, nb1), dtype=torch.uint8, device="cuda")
    X = torch.zeros((n, 1, k), dtype=torch.float32, device="cuda")
    ids = torch.zeros((n, 2), dtype=torch.int32, device="cuda")
    Y = torch.full((n, 2, rows), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_matmul_id_noalloc(W, Q4, k, X, ids, Y=Y)
    assert e.value.status == qmm.QMM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all())  # nothing was written
