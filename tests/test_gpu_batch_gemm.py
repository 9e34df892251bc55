"""Many-token MUL_MATs of one shape in a shared two-group launch
(qmm_matmul_batch) and with the last round of tiles split in k
(qmm_matmul_batch_ws, and qmm_matmul_ws for one matrix): element by element
against the oracle within |y - y_ref| <= 1e-3 * sum|w x| + 1e-5 for every
item of the launch, with ragged rows and tokens; the split tiles' counters
back at zero after each call, bitwise repetition with the same workspace,
the workspace errors, a mixed batch (decode-sized, fp32, other shapes and
more same-shape items than one launch holds), graph replay, and the
ffn_gate + ffn_up pair of 11008 x 4096 at 2048 tokens, sampled."""
import numpy as np
import pytest
import torch

import block_quantized_matmul_amd as qmm
import oracle.qmm_oracle as O
from block_quantized_matmul_amd import synth
from gpu_util import assert_bitwise, assert_close_to_oracle, dev, say

pytestmark = pytest.mark.gpu
Q4, Q8, Q51, QK = O.TYPE_Q4_0, O.TYPE_Q8_0, O.TYPE_Q5_1, O.TYPE_Q4_K
TILE_ROWS, TILE_TOKENS = 128, 256


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _tiles(rows, n):
    return -(-rows // TILE_ROWS) * -(-n // TILE_TOKENS)


def _mats(qtype, rows, k, n, count, seed, extra=0, xdt=np.float16):
    rng = np.random.Generator(np.random.PCG64([seed, qtype, rows, k, n, count, 5]))
    nb1 = synth.dense_row_bytes(qtype, k) + extra
    return [(synth.make_weights(qtype, rows, k, nb1, rng), synth.make_activations(n, k, rng, xdt))
            for _ in range(count)]


def _items(qtype, k, mats):
    out = []
    for W, X in mats:
        Y = torch.full((X.shape[0], W.shape[0]), float("nan"), dtype=torch.float32, device="cuda")
        out.append((dev(W), qtype, k, dev(X), Y))
    return out


def _run(items, ws="auto"):
    """ws: "auto" (qmm_matmul_batch_ws with a fresh zeroed workspace of the
    size it needs, None if 0), "plain" (qmm_matmul_batch) or a workspace."""
    if isinstance(ws, str) and ws == "plain":
        qmm.qmm_matmul_batch(items)
        ws = None
    else:
        if isinstance(ws, str):
            need = qmm.qmm_matmul_batch_workspace_bytes(items)
            ws = torch.zeros(need, dtype=torch.uint8, device="cuda") if need else None
        qmm.qmm_matmul_batch_ws(items, ws)
    torch.cuda.synchronize()
    return [it[4].cpu().numpy() for it in items], ws


def _gate_up_like_rows(items_count, k_stages=64):
    """Rows (ragged) whose tiles, over `items_count` items at 2000 tokens,
    fill whole rounds on the CUs plus a last round of at most half of them."""
    cus = _cus()
    per_item_tok = -(-2000 // TILE_TOKENS)
    for rt in range(1, 400):
        T = items_count * rt * per_item_tok
        if T > cus and 0 < T % cus <= cus // 2 and 4 * T >= 3 * (-(-T // cus)) * cus:
            return TILE_ROWS * rt - 29
    raise AssertionError("no shape")


@pytest.mark.parametrize("qtype,count", [(Q4, 2), (Q4, 3), (Q8, 2), (Q51, 4)])
def test_merged_launch_with_split_last_round(qtype, count):
    rows, k, n = _gate_up_like_rows(count), 4096, 2000
    T = count * _tiles(rows, n)
    mats = _mats(qtype, rows, k, n, count, 1)
    items = _items(qtype, k, mats)
    need = qmm.qmm_matmul_batch_workspace_bytes(items)
    tail = T % _cus()
    assert need == (4 * tail + 255) // 256 * 256 + tail * 2 * (128 << 10), (need, T, tail)
    say(f"merged split type={qtype} items={count} rows={rows} k={k} n={n} tiles={T} workspace={need}")
    Ys, ws = _run(items)
    for i, ((W, X), Y) in enumerate(zip(mats, Ys)):
        assert_close_to_oracle(Y, W, qtype, k, X, f"item {i}")
    assert torch.count_nonzero(ws[:4 * tail]).item() == 0, "split counters not back at zero"
    Ys2, _ = _run(items, ws)
    for Y, Y2 in zip(Ys, Ys2):
        assert_bitwise(Y2, Y, "second call, same workspace")
    # without the workspace: whole tiles only, within the tolerance of the split
    Ys3, _ = _run(items, "plain")
    for (W, X), Y3 in zip(mats, Ys3):
        assert_close_to_oracle(Y3, W, qtype, k, X, "unsplit merged launch")


@pytest.mark.parametrize("qtype", [Q4, QK])
def test_merged_launch_whole_tiles(qtype):
    """Items whose shared launch needs no split (k too short to split, or
    Q4_K): the two-group kernel over all items' tiles; the workspace form
    gives the same bits."""
    rows, k, n = 6 * TILE_ROWS - 50, 512, 8 * TILE_TOKENS - 77   # 48 tiles per item, 192 for 4
    mats = _mats(qtype, rows, k, n, 4, 2, extra=16)
    items = _items(qtype, k, mats)
    assert qmm.qmm_matmul_batch_workspace_bytes(items) == 0
    say(f"merged whole type={qtype} rows={rows} k={k} n={n}")
    Ys, _ = _run(items, "plain")
    for i, ((W, X), Y) in enumerate(zip(mats, Ys)):
        assert_close_to_oracle(Y, W, qtype, k, X, f"item {i}")
    Ys2, _ = _run(items, "auto")
    for Y, Y2 in zip(Ys, Ys2):
        assert_bitwise(Y2, Y, "batch_ws without a split")


def test_mixed_batch():
    """Decode-sized, fp32 many-token, other-shape and five same-shape fp16
    items (four share a launch, the fifth runs alone) in one call."""
    k = 4096
    rows = _gate_up_like_rows(4)
    same = _mats(Q4, rows, k, 2000, 5, 3)
    dec = _mats(Q8, 300, k, 3, 1, 4, xdt=np.float32)
    f32 = _mats(Q4, 500, k, 300, 1, 5, xdt=np.float32)
    other = _mats(Q4, 700, 1024, 600, 1, 6)
    mats = [(same[0], Q4, k), (dec[0], Q8, k), (same[1], Q4, k), (f32[0], Q4, k), (same[2], Q4, k),
            (other[0], Q4, 1024), (same[3], Q4, k), (same[4], Q4, k)]
    items = []
    for (W, X), qt, kk in mats:
        items += _items(qt, kk, [(W, X)])
    say(f"mixed batch of {len(items)}, same-shape rows={rows}")
    Ys, ws = _run(items)
    assert ws is not None
    for i, (((W, X), qt, kk), Y) in enumerate(zip(mats, Ys)):
        assert_close_to_oracle(Y, W, qt, kk, X, f"mixed item {i}")
    tail = 4 * _tiles(rows, 2000) % _cus()
    assert torch.count_nonzero(ws[:4 * tail]).item() == 0


def test_batch_ws_errors():
    rows, k, n = _gate_up_like_rows(2), 4096, 2000
    items = _items(Q4, k, _mats(Q4, rows, k, n, 2, 7))
    need = qmm.qmm_matmul_batch_workspace_bytes(items)
    assert need > 0
    say("batch_ws errors")
    for ws in (None, torch.zeros(need - 1, dtype=torch.uint8, device="cuda")):
        with pytest.raises(qmm.QmmError) as e:
            qmm.qmm_matmul_batch_ws(items, ws)
        assert e.value.status == qmm.QMM_ERR_WORKSPACE
    big = torch.zeros(need + 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_matmul_batch_ws(items, big[8:])
    assert e.value.status == qmm.QMM_ERR_ALIGN
    torch.cuda.synchronize()
    assert torch.count_nonzero(big).item() == 0, "a rejected call touched the workspace"
    assert all(torch.isnan(it[4]).all().item() for it in items), "a rejected call wrote an output"


def test_single_matrix_split_last_round():
    """qmm_matmul_ws on one matrix whose tiles fill whole rounds plus a last
    round of at most half the CUs: that round's tiles split in two."""
    rows, k, n = _gate_up_like_rows(1), 4096, 2000
    T = _tiles(rows, n)
    need = qmm.qmm_matmul_workspace_bytes(Q4, rows, k, n, qmm.QMM_X_F16)
    tail = T % _cus()
    assert need == (4 * tail + 255) // 256 * 256 + tail * 2 * (128 << 10)
    (W, X), = _mats(Q4, rows, k, n, 1, 8)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    say(f"single split last round rows={rows} tiles={T}")
    Y = qmm.qmm_matmul_ws(dev(W), Q4, k, dev(X), ws, n_rows=rows, row_stride_bytes=W.shape[1], n_tokens=n)
    torch.cuda.synchronize()
    assert_close_to_oracle(Y.cpu().numpy(), W, Q4, k, X, "single split")
    assert torch.count_nonzero(ws[:4 * tail]).item() == 0


def test_merged_split_graph_replay():
    rows, k, n = _gate_up_like_rows(2), 4096, 2000
    items = _items(Q4, k, _mats(Q4, rows, k, n, 2, 9))
    ws = torch.zeros(qmm.qmm_matmul_batch_workspace_bytes(items), dtype=torch.uint8, device="cuda")
    say("merged split graph replay")
    ref, _ = _run(items, ws)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qmm.qmm_matmul_batch_ws(items, ws)
    for rep in range(3):
        for it in items:
            it[4].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for it, r in zip(items, ref):
            assert_bitwise(it[4].cpu().numpy(), r, f"replay {rep}")


def test_gate_up_pair_full_size_sampled():
    """ffn_gate and ffn_up of the Llama-7B layer, 11008 x 4096 Q4_0 at 2048
    fp16 tokens, in one launch with its last round split: sampled outputs of
    both against the oracle, repeat bit for bit."""
    rows, k, n = 11008, 4096, 2048
    mats = _mats(Q4, rows, k, n, 2, 10)
    items = _items(Q4, k, mats)
    say("gate+up 11008x4096 at 2048 tokens")
    Ys, ws = _run(items)
    rng = np.random.default_rng(11)
    for (W, X), Y in zip(mats, Ys):
        rr = np.concatenate([np.arange(rows - 200, rows), rng.integers(0, rows, 6000)])
        tt = np.concatenate([np.full(200, n - 1), rng.integers(0, n, 6000)])
        y_ref, s = O.matmul_sampled(W, Q4, rows, k, W.shape[1], X, tt, rr)
        assert O.within_tolerance(Y[tt, rr], y_ref, s).all()
    Ys2, _ = _run(items, ws)
    for Y, Y2 in zip(Ys, Ys2):
        assert_bitwise(Y2, Y, "repeat")
