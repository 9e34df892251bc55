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
Q4, Q41, Q8 = O.TYPE_Q4_0, O.TYPE_Q4_1, O.TYPE_Q8_0
Q50, Q51 = O.TYPE_Q5_0, O.TYPE_Q5_1


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


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("layout", ["stream", "general"])
@pytest.mark.parametrize("shared_x", [False, True])
@pytest.mark.parametrize("n_tokens", [1, 3, 9])
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
    if n_tokens == 9:  # 18 pairs over 8 experts: bucketed into decode tiles of 4 pairs
        import block_quantized_matmul_amd as qmm
        assert qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0
    say(f"matmul_id {layout} type={qtype} tokens={n_tokens} x_slots={X.shape[1]} ids={ids.tolist()}")
    Y = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset)
    y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
    _check(Y, y_ref, s, f"matmul_id {layout}")


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("n_tokens,n_experts", [(2, 2), (5, 4), (8, 4), (12, 8), (8, 1)])
@pytest.mark.parametrize("shared_x", [False, True])
def test_matmul_id_decode_tiles(qtype, n_tokens, n_experts, shared_x):
    """Decode-sized calls with several pairs per expert: the pairs are
    bucketed by expert and the streaming decode kernel runs tiles of 2, 4 or
    8 pairs of one expert, with repeated experts and one id that names none.
    The same call on a padded layout takes the per-pair route. Both against
    the oracle."""
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([509, qtype, n_tokens, n_experts, int(shared_x)]))
    n_ids, rows, k = 2, 136, 512
    assert qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0, "not a grouped route"
    dense = synth.dense_row_bytes(qtype, k)
    xs = 1 if shared_x else n_ids
    X = synth.make_activations(n_tokens * xs, k, rng, np.float32).reshape(n_tokens, xs, k)
    ids = rng.integers(0, n_experts, size=(n_tokens, n_ids)).astype(np.int32)
    ids[0, 1] = -3
    for nb1, nb2, offset, what in ((dense, rows * dense, 0, "tiles"),
                                   (dense + 2, rows * (dense + 2), 2, "per-pair")):
        W = _stack(qtype, n_experts, rows, k, nb1, nb2, rng)
        say(f"matmul_id decode {what} type={qtype} tokens={n_tokens} experts={n_experts} x_slots={xs}")
        Y = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset)
        y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
        _check(Y, y_ref, s, f"matmul_id decode {what}")


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


def _skewed_ids(rng, n_tokens, n_ids, n_experts):
    """Routing with an uneven load: expert 1 takes about half the pairs (more
    than one 128-pair tile at 300 tokens), expert n_experts - 1 none, and
    two ids name no expert."""
    ids = rng.integers(0, n_experts - 1, size=(n_tokens, n_ids)).astype(np.int32)
    ids[rng.random((n_tokens, n_ids)) < 0.5] = 1
    ids[0, 0] = -1
    ids[n_tokens - 1, n_ids - 1] = n_experts
    return ids


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("layout", ["aligned", "padded"])
@pytest.mark.parametrize("shared_x", [False, True])
@pytest.mark.parametrize("n_tokens,n_experts", [(9, 4), (300, 8)])
def test_matmul_id_grouped(qtype, layout, shared_x, n_tokens, n_experts):
    """More tokens than the decode kernels take: pairs bucketed by expert,
    matrix-core tiles. Every token is checked at 9 tokens; a sample at 300."""
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([503, qtype, n_tokens, int(shared_x), len(layout)]))
    n_ids, rows, k = 2, 200, 544   # 17 blocks: an odd block count, a ragged row tile
    assert qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0, "not the grouped path"
    dense = synth.dense_row_bytes(qtype, k)
    if layout == "aligned":
        nb1, nb2, offset = dense, rows * dense + 64, 0
    else:                    # 2-byte-aligned stack and rows: the halfword weight loads
        nb1, nb2, offset = dense + 2, rows * (dense + 2) + 6, 2
    W = _stack(qtype, n_experts, rows, k, nb1, nb2, rng)
    xs = 1 if shared_x else n_ids
    X = synth.make_activations(n_tokens * xs, k, rng, np.float32).reshape(n_tokens, xs, k)
    ids = _skewed_ids(rng, n_tokens, n_ids, n_experts)
    say(f"matmul_id grouped {layout} type={qtype} tokens={n_tokens} x_slots={xs}")
    Y = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset)
    sample = np.arange(n_tokens) if n_tokens <= 16 else \
        np.unique(np.concatenate([[0, 1, n_tokens - 1], rng.integers(0, n_tokens, 40)]))
    y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X[sample], ids[sample])
    _check(Y[sample], y_ref, s, f"matmul_id grouped {layout}")


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_matmul_id_grouped_repeatable_and_agrees_with_decode(qtype):
    """The bucket order inside an expert varies from run to run; the results
    must not (bitwise). Each token's rows also agree, within tolerance, with
    the same token routed alone through the decode kernels."""
    rng = np.random.Generator(np.random.PCG64([504, qtype]))
    n_experts, n_ids, rows, k, n_tokens = 16, 4, 256, 1024, 200
    nb1 = synth.dense_row_bytes(qtype, k)
    nb2 = rows * nb1
    W = _stack(qtype, n_experts, rows, k, nb1, nb2, rng)
    X = synth.make_activations(n_tokens * n_ids, k, rng, np.float32).reshape(n_tokens, n_ids, k)
    ids = rng.integers(0, n_experts, size=(n_tokens, n_ids)).astype(np.int32)
    import block_quantized_matmul_amd as qmm
    assert qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0, "not the grouped path"
    say(f"matmul_id grouped twice type={qtype} tokens={n_tokens}")
    Y1 = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
    Y2 = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
    assert np.array_equal(Y1.view(np.uint32), Y2.view(np.uint32)), "grouped MUL_MAT_ID is not repeatable"
    for t in (0, 77, n_tokens - 1):
        Yd = _run(W, qtype, n_experts, rows, k, nb1, nb2, X[t:t + 1], ids[t:t + 1])
        y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X[t:t + 1], ids[t:t + 1])
        _check(Yd, y_ref, s, "decode route")
        _check(Y1[t:t + 1], y_ref, s, "grouped route")


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("layout", ["aligned", "padded"])
@pytest.mark.parametrize("shared_x", [False, True])
def test_matmul_id_two_group_tiles(qtype, layout, shared_x):
    """Enough 128-row tiles x tile pairs to fill the 256 CUs (4096 rows, 512
    tokens, 2 of 8 experts): the two-group routed kernel, two 160-pair tiles
    of the routing table per workgroup. Skewed routing gives an expert of
    several tiles, the last one partial, one id names no expert; every
    element against the oracle, NaN rows exact, and bitwise repeatable."""
    rng = np.random.Generator(np.random.PCG64([507, qtype, len(layout), int(shared_x)]))
    n_experts, n_ids, rows, k, n_tokens = 8, 2, 4096, 256, 512
    dense = synth.dense_row_bytes(qtype, k)
    if layout == "aligned":
        nb1, nb2, offset = dense, rows * dense, 0
    else:  # 2-byte-aligned rows: the unaligned staging
        nb1, nb2, offset = dense + 2, rows * (dense + 2) + 2, 2
    W = _stack(qtype, n_experts, rows, k, nb1, nb2, rng)
    slots = 1 if shared_x else n_ids
    X = synth.make_activations(n_tokens * slots, k, rng, np.float32).reshape(n_tokens, slots, k)
    ids = _skewed_ids(rng, n_tokens, n_ids, n_experts)
    ids[3, 1] = n_experts
    say(f"matmul_id two-group type={qtype} layout={layout} shared_x={shared_x}")
    Y = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset)
    y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
    _check(Y, y_ref, s, "two-group routed")
    Y2 = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset)
    assert np.array_equal(Y.view(np.uint32), Y2.view(np.uint32)), "not repeatable"


@pytest.mark.parametrize("qtype,layout", [(Q4, "aligned"), (Q4, "padded"), (Q51, "aligned"), (Q8, "aligned")])
def test_matmul_id_two_group_tile_edges(qtype, layout):
    """Pair counts at the two-group kernel's tile edges (160 pairs per tile):
    161 (a full tile and a one-pair tile), 160, 129, 1, 300 (160 + 140), 150,
    123 and 0 pairs for experts 0..7, 9 tiles in all, so one workgroup's
    second group is empty. Every element against the oracle, and the same
    bits as the one-group kernel (128-pair tiles, chosen by a workspace
    without room for the fp16 activations)."""
    import torch
    import block_quantized_matmul_amd as qmm
    from gpu_util import place_weights
    rng = np.random.Generator(np.random.PCG64([512, qtype, len(layout)]))
    n_experts, n_ids, rows, k, n_tokens = 8, 2, 4096, 256, 512
    counts = [161, 160, 129, 1, 300, 150, 123, 0]
    assert sum(counts) == n_tokens * n_ids
    ids = rng.permutation(np.repeat(np.arange(n_experts, dtype=np.int32), counts)).reshape(n_tokens, n_ids)
    dense = synth.dense_row_bytes(qtype, k)
    if layout == "aligned":
        nb1, nb2, offset = dense, rows * dense, 0
    else:
        nb1, nb2, offset = dense + 2, rows * (dense + 2) + 2, 2
    W = _stack(qtype, n_experts, rows, k, nb1, nb2, rng)
    X = synth.make_activations(n_tokens, k, rng, np.float32).reshape(n_tokens, 1, k)
    say(f"matmul_id two-group tile edges type={qtype} layout={layout}")
    Y = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset)
    y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
    _check(Y, y_ref, s, "two-group tile edges")
    _keep, Wd = place_weights(W, offset)
    ws = torch.empty(qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens), dtype=torch.uint8,
                     device="cuda")
    Y1 = qmm.qmm_matmul_id(Wd, qtype, k, dev(X), dev(ids), n_experts=n_experts, n_rows=rows, row_stride_bytes=nb1,
                           expert_stride_bytes=nb2, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(Y.view(np.uint32), Y1.cpu().numpy().view(np.uint32)), "two-group != one-group kernel"


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_matmul_id_mixtral_prefill_sampled(qtype):
    """512 tokens through 8 experts of 14336 x 4096, 2 selected per token
    (the probe's batch at a routed-FFN shape, the grouped bench case);
    sampled (token, slot, row) outputs against the oracle."""
    import torch
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([505, qtype]))
    n_experts, rows, k, n_ids, n_tokens = 8, 14336, 4096, 2, 512
    nb1 = synth.dense_row_bytes(qtype, k)
    Wn = synth.make_weights(qtype, n_experts * rows, k, nb1, rng)
    X = synth.make_activations(n_tokens, k, rng, np.float32).reshape(n_tokens, 1, k)
    ids = np.stack([rng.permutation(n_experts)[:n_ids] for _ in range(n_tokens)]).astype(np.int32)
    say(f"matmul_id prefill experts={n_experts} rows={rows} k={k} tokens={n_tokens} type={qtype}")
    W = dev(Wn.reshape(n_experts, rows, nb1))
    Y = qmm.qmm_matmul_id(W, qtype, k, dev(X), dev(ids))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    for t in (0, 255, 511):
        rsamp = np.unique(np.concatenate([[0, 127, 128, rows - 1], rng.integers(0, rows, 60)]))
        for i in range(n_ids):
            e = ids[t, i]
            We = Wn[e * rows:(e + 1) * rows]
            y_ref, s = O.matmul_sampled(We, qtype, rows, k, nb1, X[t], np.zeros_like(rsamp), rsamp)
            ok = O.within_tolerance(Y[t, i, rsamp], y_ref, s)
            assert ok.all(), f"token {t} expert {e}: {int((~ok).sum())} sampled rows outside tolerance"


@pytest.mark.parametrize("qtype", [Q4, Q8])
def test_matmul_id_mixtral_batched_decode_sampled(qtype):
    """8 tokens through 8 experts of 14336 x 4096, 2 selected per token (the
    bench's batched-decode case, grouped decode tiles of 2 pairs); every
    (token, slot) pair's sampled rows against the oracle."""
    import torch
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([510, qtype]))
    n_experts, rows, k, n_ids, n_tokens = 8, 14336, 4096, 2, 8
    assert qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0, "not a grouped route"
    nb1 = synth.dense_row_bytes(qtype, k)
    Wn = synth.make_weights(qtype, n_experts * rows, k, nb1, rng)
    X = synth.make_activations(n_tokens, k, rng, np.float32).reshape(n_tokens, 1, k)
    ids = np.stack([rng.permutation(n_experts)[:n_ids] for _ in range(n_tokens)]).astype(np.int32)
    say(f"matmul_id batched decode experts={n_experts} rows={rows} k={k} tokens={n_tokens} type={qtype}")
    W = dev(Wn.reshape(n_experts, rows, nb1))
    Y = qmm.qmm_matmul_id(W, qtype, k, dev(X), dev(ids))
    torch.cuda.synchronize()
    Y = Y.cpu().numpy()
    for t in range(n_tokens):
        rsamp = np.unique(np.concatenate([[0, 15, 16, rows - 1], rng.integers(0, rows, 24)]))
        for i in range(n_ids):
            e = ids[t, i]
            We = Wn[e * rows:(e + 1) * rows]
            y_ref, s = O.matmul_sampled(We, qtype, rows, k, nb1, X[t], np.zeros_like(rsamp), rsamp)
            ok = O.within_tolerance(Y[t, i, rsamp], y_ref, s)
            assert ok.all(), f"token {t} expert {e}: {int((~ok).sum())} sampled rows outside tolerance"


@pytest.mark.parametrize("n_experts,n_tokens", [(64, 256), (64, 512), (64, 513), (65, 256), (64, 100), (65, 100)])
def test_matmul_id_routing_kernel_sizes(n_experts, n_tokens):
    """Both routing kernels: up to 64 experts and 1024 pairs take the
    one-wavefront kernel, more of either the workgroup kernel; the grouped
    GEMM (256 to 513 tokens: 8 to 16 pairs per expert) and decode tiles (100
    tokens: about 3) on each side of the boundary, with ids that name no
    expert, against the oracle."""
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([511, n_experts, n_tokens]))
    qtype, n_ids, rows, k = Q4, 2, 40, 256
    ids = rng.integers(0, n_experts, size=(n_tokens, n_ids)).astype(np.int32)
    ids[0, 0] = -1
    ids[n_tokens - 1, 1] = n_experts
    assert qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0, "not a grouped route"
    dense = synth.dense_row_bytes(qtype, k)
    W = _stack(qtype, n_experts, rows, k, dense, rows * dense, rng)
    X = synth.make_activations(n_tokens, k, rng, np.float32).reshape(n_tokens, 1, k)
    say(f"matmul_id routing experts={n_experts} tokens={n_tokens}")
    Y = _run(W, qtype, n_experts, rows, k, dense, rows * dense, X, ids)
    y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, dense, rows * dense, X, ids)
    _check(Y, y_ref, s, f"routing experts={n_experts} tokens={n_tokens}")


@pytest.mark.parametrize("n_experts,n_ids,n_tokens", [(256, 8, 128), (4096, 8, 2048), (4097, 2, 16)])
def test_matmul_id_many_experts(n_experts, n_ids, n_tokens):
    """Many small experts: 256 and 4096 (the most the grouped route counts in
    LDS) take the grouped path, 4097 the per-pair one; sampled tokens against
    the oracle."""
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([506, n_experts, n_ids]))
    rows, k = 40, 64
    nb1 = synth.dense_row_bytes(Q4, k)
    nb2 = rows * nb1
    W = _stack(Q4, n_experts, rows, k, nb1, nb2, rng)
    X = synth.make_activations(n_tokens, k, rng).reshape(n_tokens, 1, k)
    ids = rng.integers(0, n_experts, size=(n_tokens, n_ids)).astype(np.int32)
    ids[1, :] = n_experts - 1
    grouped = qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0
    assert grouped == (n_experts <= 4096)
    say(f"matmul_id experts={n_experts} n_ids={n_ids} tokens={n_tokens} grouped={grouped}")
    Y = _run(W, Q4, n_experts, rows, k, nb1, nb2, X, ids)
    sample = np.unique(np.concatenate([[0, 1, n_tokens - 1], rng.integers(0, n_tokens, 30)]))
    y_ref, s = O.matmul_id(W, Q4, n_experts, rows, k, nb1, nb2, X[sample], ids[sample])
    _check(Y[sample], y_ref, s, f"matmul_id experts={n_experts}")


@pytest.mark.parametrize("n_experts", [0, 4])
def test_matmul_id_grouped_no_valid_id(n_experts):
    """Grouped path where no id names an expert (or there are none): every
    output row is NaN, and nothing else is written."""
    import torch
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([507, n_experts]))
    rows, k, n_ids, n_tokens = 24, 64, 2, 40
    nb1 = synth.dense_row_bytes(Q4, k)
    nb2 = rows * nb1
    W = _stack(Q4, max(n_experts, 1), rows, k, nb1, nb2, rng)
    X = synth.make_activations(n_tokens, k, rng).reshape(n_tokens, 1, k)
    ids = np.full((n_tokens, n_ids), n_experts, np.int32)
    ids[::3, 0] = -7
    assert n_experts == 0 or qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0
    say(f"matmul_id no valid id experts={n_experts}")
    from gpu_util import place_weights
    _keep, Wd = place_weights(W)
    Y = torch.zeros((n_tokens + 1, n_ids, rows), dtype=torch.float32, device="cuda")
    qmm.qmm_matmul_id(Wd, Q4, k, dev(X), dev(ids), n_experts=n_experts, n_rows=rows, row_stride_bytes=nb1,
                      expert_stride_bytes=nb2, Y=Y[:n_tokens])
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy()
    assert np.isnan(Yh[:n_tokens]).all()
    assert (Yh[n_tokens] == 0).all()


def test_matmul_id_graph_replay_with_new_routing():
    """Decode and grouped MUL_MAT_ID captured in one graph and replayed with
    new routing written into the captured ids buffers between replays (as a
    serving loop would), with eager work in between: every replay equals an
    eager call on the same routing."""
    import torch
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64(508))
    n_experts, rows, k, n_ids = 8, 136, 256, 2
    nb1 = synth.dense_row_bytes(Q4, k)
    W = dev(_stack(Q4, n_experts, rows, k, nb1, rows * nb1, rng).reshape(n_experts, rows, nb1))
    Xd = dev(synth.make_activations(1, k, rng).reshape(1, 1, k))
    Xp = dev(synth.make_activations(300, k, rng).reshape(300, 1, k))
    ids_d = torch.zeros((1, n_ids), dtype=torch.int32, device="cuda")
    ids_p = torch.zeros((300, n_ids), dtype=torch.int32, device="cuda")
    Yd = torch.empty((1, n_ids, rows), dtype=torch.float32, device="cuda")
    Yp = torch.empty((300, n_ids, rows), dtype=torch.float32, device="cuda")
    ws = torch.empty(qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, 300), dtype=torch.uint8, device="cuda")

    def work():
        qmm.qmm_matmul_id(W, Q4, k, Xd, ids_d, Y=Yd)
        qmm.qmm_matmul_id(W, Q4, k, Xp, ids_p, Y=Yp, workspace=ws)

    def routing(n):
        return torch.from_numpy(np.stack([rng.permutation(n_experts)[:n_ids] for _ in range(n)]).astype(np.int32))

    say("matmul_id graph capture")
    work()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        ids_d.copy_(routing(1).cuda())
        ids_p.copy_(routing(300).cuda())
        Yd.fill_(float("nan"))
        Yp.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_d, got_p = Yd.clone(), Yp.clone()
        work()  # eager, same routing
        torch.cuda.synchronize()
        assert torch.equal(got_d, Yd), f"decode replay {rep} differs"
        assert torch.equal(got_p, Yp), f"grouped replay {rep} differs"
        _ = (Xp * 2).sum().item()  # unrelated eager work between replays


@pytest.mark.parametrize("seed", range(4))
def test_matmul_id_random_sweep(seed):
    """Seeded random MUL_MAT_ID cases: type, expert count, slots, tokens
    (every route), shared or per-slot activations, padded or streaming
    layouts, and a few ids that name no expert."""
    import block_quantized_matmul_amd as qmm
    rng = np.random.Generator(np.random.PCG64([601, seed]))
    for case in range(4):
        qtype = int(rng.choice([Q4, Q41, Q50, Q51, Q8]))
        n_experts = int(rng.integers(1, 20))
        n_ids = int(rng.integers(1, 5))
        n_tokens = int(rng.choice([1, 4, 8, 12, 40]))
        rows = int(rng.integers(1, 300))
        k = 256 * int(rng.integers(1, 4))
        dense = synth.dense_row_bytes(qtype, k)
        padded = rng.random() < 0.5
        nb1 = dense + (2 if padded else 0)
        nb2 = rows * nb1 + (6 if padded else 0)
        offset = 2 if padded else 0
        W = _stack(qtype, n_experts, rows, k, nb1, nb2, rng)
        xs = 1 if rng.random() < 0.5 else n_ids
        X = synth.make_activations(n_tokens * xs, k, rng).reshape(n_tokens, xs, k)
        ids = rng.integers(0, n_experts, size=(n_tokens, n_ids)).astype(np.int32)
        ids[rng.random((n_tokens, n_ids)) < 0.05] = n_experts
        grouped = qmm.qmm_matmul_id_workspace_bytes(n_experts, n_ids, n_tokens) > 0
        say(f"matmul_id sweep {seed}.{case} type={qtype} experts={n_experts} ids={n_ids} tokens={n_tokens} "
            f"rows={rows} k={k} padded={padded} grouped={grouped}")
        Y = _run(W, qtype, n_experts, rows, k, nb1, nb2, X, ids, offset)
        y_ref, s = O.matmul_id(W, qtype, n_experts, rows, k, nb1, nb2, X, ids)
        _check(Y, y_ref, s, f"matmul_id sweep {seed}.{case}")
