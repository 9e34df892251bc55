"""The matrix-core MUL_MAT with k split across workgroups (qmm_matmul_ws) on
the GPU: element by element against the oracle within
|y - y_ref| <= 1e-3 * sum|w x| + 1e-5 with 2, 3 and 4 parts per tile (equal
and unequal stage ranges), ragged rows and tokens, every 32-weight type and
both load layouts; bitwise repetition, counters left at zero, workspace
reuse across shapes, graph replay, non-finite scales, the workspace errors
and the shapes that do not split, and a 4096x14336 projection at 512 tokens
at full size."""
import numpy as np
import pytest
import torch

import block_quantized_matmul_amd as qmm
import oracle.qmm_oracle as O
from block_quantized_matmul_amd import synth
from gpu_util import assert_bitwise, assert_close_to_oracle, dev, place_weights, run_matmul, say

pytestmark = pytest.mark.gpu
Q4, Q41, Q8 = O.TYPE_Q4_0, O.TYPE_Q4_1, O.TYPE_Q8_0
Q50, Q51 = O.TYPE_Q5_0, O.TYPE_Q5_1
F16 = qmm.QMM_X_F16
TILE_ROWS, TILE_TOKENS = 128, 256


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _tiles(rows, n):
    return -(-rows // TILE_ROWS) * -(-n // TILE_TOKENS)


def _inputs(qtype, rows, k, n, extra=0, seed=0):
    rng = np.random.Generator(np.random.PCG64([seed, qtype, rows, k, n, extra, 7]))
    nb1 = synth.dense_row_bytes(qtype, k) + extra
    W = synth.make_weights(qtype, rows, k, nb1, rng, 0.001, 0.05)
    X = synth.make_activations(n, k, rng, np.float16)
    return W, X


def _need(qtype, rows, k, n):
    return qmm.qmm_matmul_workspace_bytes(qtype, rows, k, n, F16)


def _run_ws(Wnp, qtype, k, Xnp, ws=None, w_offset=0):
    rows, nb1 = Wnp.shape
    n = Xnp.shape[0]
    _buf, W = place_weights(Wnp, w_offset)
    X = dev(Xnp)
    need = _need(qtype, rows, k, n)
    if ws is None and need > 0:
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    Y = qmm.qmm_matmul_ws(W, qtype, k, X, ws, n_rows=rows, row_stride_bytes=nb1, n_tokens=n)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), ws


def _counters_zero(ws, rows, n):
    assert torch.count_nonzero(ws[:4 * _tiles(rows, n)]).item() == 0, "split counters not back at zero"


# (rows, k, n, extra, offset): 6 tiles in 4 parts of 32 stages, and of 32 or
# 33 stages (k = 8256), with 4-byte and 2-byte aligned rows; 16 tiles in 4
# parts with ragged rows and tokens and padded rows.
SHAPES = [(300, 8192, 300, 0, 0), (300, 8256, 300, 0, 0), (300, 8256, 300, 2, 2), (1000, 8192, 700, 4, 0)]


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("rows,k,n,extra,offset", SHAPES)
def test_split_parity(qtype, rows, k, n, extra, offset):
    assert _tiles(rows, n) * 4 <= _cus()
    W, X = _inputs(qtype, rows, k, n, extra)
    need = _need(qtype, rows, k, n)
    assert need > 0, "the shape should take the split"
    say(f"split type={qtype} rows={rows} k={k} n={n} nb1={W.shape[1]} offset={offset} workspace={need}")
    Y, ws = _run_ws(W, qtype, k, X, w_offset=offset)
    assert_close_to_oracle(Y, W, qtype, k, X, f"split rows={rows} k={k} n={n}")
    _counters_zero(ws, rows, n)
    Y2, _ = _run_ws(W, qtype, k, X, ws, w_offset=offset)
    assert_bitwise(Y2, Y, "second call, same workspace")


@pytest.mark.parametrize("parts", [2, 3])
def test_split_two_and_three_parts(parts):
    """Tiles split in two parts (the workgroup that completes a tile adds the
    other part to its own registers) and in three (k order, read back); the
    oracle on sampled outputs, the whole output against the unsplit kernel
    within the tolerance, bitwise repetition."""
    cus = _cus()
    t = cus // parts                       # tiles giving `parts` parts each
    rows, n = TILE_ROWS * (t // 2) - 37, 2 * TILE_TOKENS - 100
    k = 64 * 32 * parts
    assert _tiles(rows, n) == 2 * (t // 2) and min(4, cus // _tiles(rows, n)) == parts
    W, X = _inputs(Q4, rows, k, n)
    assert _need(Q4, rows, k, n) == (4 * _tiles(rows, n) + 255) // 256 * 256 + _tiles(rows, n) * parts * (128 << 10)
    say(f"split {parts} parts rows={rows} k={k} n={n}")
    Y, ws = _run_ws(W, Q4, k, X)
    rng = np.random.default_rng(parts)
    r_s, t_s = rng.integers(0, rows, 4096), rng.integers(0, n, 4096)
    y_ref, s = O.matmul_sampled(W, Q4, rows, k, W.shape[1], X, t_s, r_s)
    assert O.within_tolerance(Y[t_s, r_s], y_ref, s).all()
    Y0 = run_matmul(W, Q4, k, X)
    assert np.all(np.abs(Y - Y0) <= 2e-3 * np.abs(Y0).max())
    _counters_zero(ws, rows, n)
    assert_bitwise(_run_ws(W, Q4, k, X, ws)[0], Y, "repeat")


def test_workspace_reuse_across_shapes():
    """One workspace serves calls of different shapes in a row (every call
    leaves the counters at zero); results repeat bitwise."""
    a = _inputs(Q4, 300, 8192, 300)
    b = _inputs(Q8, 1000, 8192, 700)
    size = max(_need(Q4, 300, 8192, 300), _need(Q8, 1000, 8192, 700))
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    say("workspace reuse")
    ya, _ = _run_ws(a[0], Q4, 8192, a[1], ws)
    yb, _ = _run_ws(b[0], Q8, 8192, b[1], ws)
    ya2, _ = _run_ws(a[0], Q4, 8192, a[1], ws)
    assert_bitwise(ya2, ya, "shape a after shape b")
    assert_close_to_oracle(yb, b[0], Q8, 8192, b[1], "shape b")
    _counters_zero(ws, 1000, 700)


def test_split_nonfinite_scales():
    rows, k, n = 300, 8192, 300
    W, X = _inputs(Q4, rows, k, n)
    W[3, 0:2] = [0x00, 0x7E]                  # NaN scale, first block of row 3 (part 0)
    W[7, 18 * 200:18 * 200 + 2] = [0x00, 0x7C]  # +inf scale, block 200 of row 7 (part 3)
    say("split non-finite scales")
    Y, _ = _run_ws(W, Q4, k, X)
    assert np.all(np.isnan(Y[:, 3]))
    assert not np.any(np.isfinite(Y[:, 7]))
    others = np.delete(np.arange(rows), [3, 7])
    assert np.all(np.isfinite(Y[:, others]))
    assert_close_to_oracle(Y[:, others], W[others], Q4, k, X, "finite rows")


def test_workspace_errors_and_unsplit_shapes():
    rows, k, n = 300, 8192, 300
    W, X = _inputs(Q4, rows, k, n)
    _buf, Wd = place_weights(W)
    Xd = dev(X)
    need = _need(Q4, rows, k, n)
    say("workspace errors")
    for ws in (None, torch.zeros(need - 1, dtype=torch.uint8, device="cuda")):
        with pytest.raises(qmm.QmmError) as e:
            qmm.qmm_matmul_ws(Wd, Q4, k, Xd, ws, n_rows=rows, row_stride_bytes=W.shape[1], n_tokens=n)
        assert e.value.status == qmm.QMM_ERR_WORKSPACE
    big = torch.zeros(need + 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(qmm.QmmError) as e:
        qmm.qmm_matmul_ws(Wd, Q4, k, Xd, big[8:], n_rows=rows, row_stride_bytes=W.shape[1], n_tokens=n)
    assert e.value.status == qmm.QMM_ERR_ALIGN
    assert torch.count_nonzero(big).item() == 0, "a rejected call touched the workspace"
    # shapes the split does not take need no workspace and give qmm_matmul_path's bits
    cus = _cus()
    for qt, r, kk, nn, xdt in ((Q4, 300, 8192, 8, np.float16), (Q4, 300, 8192, 300, np.float32),
                               (O.TYPE_Q4_K, 300, 8192, 300, np.float16), (Q4, 300, 8224, 300, np.float16),
                               (Q4, 300, 8192, 200, np.float16), (Q4, 300, 4096, 300, np.float16),
                               (Q4, TILE_ROWS * (cus // 4) + 1, 8192, 512, np.float16)):
        xt = F16 if xdt == np.float16 else qmm.QMM_X_F32
        assert qmm.qmm_matmul_workspace_bytes(qt, r, kk, nn, xt) == 0, (qt, r, kk, nn, xdt)
        Wq, Xq = _inputs(qt, r, kk, nn)
        Xq = Xq.astype(xdt)
        _b, Wqd = place_weights(Wq)
        y = qmm.qmm_matmul_ws(Wqd, qt, kk, dev(Xq), None, n_rows=r, row_stride_bytes=Wq.shape[1], n_tokens=nn)
        torch.cuda.synchronize()
        assert_bitwise(y.cpu().numpy(), run_matmul(Wq, qt, kk, Xq), f"unsplit shape {(qt, r, kk, nn)}")


def test_split_graph_replay():
    """Split calls captured in a graph and replayed, with eager work between
    replays, give the eager bits every time."""
    cases = [_inputs(Q4, 1000, 8192, 700), _inputs(Q51, 300, 8256, 300)]
    dev_in = []
    size = max(_need(Q4, 1000, 8192, 700), _need(Q51, 300, 8256, 300))
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for (W, X), qt, k in zip(cases, (Q4, Q51), (8192, 8256)):
        _b, Wd = place_weights(W)
        Xd = dev(X)
        Y = torch.empty((X.shape[0], W.shape[0]), dtype=torch.float32, device="cuda")
        dev_in.append((_b, Wd, Xd, Y, qt, k, W.shape))

    def work():
        for _b, Wd, Xd, Y, qt, k, shp in dev_in:
            qmm.qmm_matmul_ws(Wd, qt, k, Xd, ws, n_rows=shp[0], row_stride_bytes=shp[1], n_tokens=Xd.shape[0], Y=Y)

    say("split graph capture")
    work()
    torch.cuda.synchronize()
    ref = [d[3].clone() for d in dev_in]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        for d in dev_in:
            d[3].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for d, r in zip(dev_in, ref):
            assert torch.equal(d[3], r), f"replay {rep} differs"
        _ = (dev_in[0][2].float() * 2).sum().item()  # unrelated eager work between replays


def test_long_k_projection_512_tokens():
    """A 4096-row projection over k = 14336 at the 512-token batch (64 tiles,
    four parts each), the shape the split is for: sampled outputs against
    the oracle, the whole output against the unsplit kernel within the
    tolerance, and the 512-token workload shapes, which do not split."""
    rows, k, n = 4096, 14336, 512
    W, X = _inputs(Q4, rows, k, n, seed=3)
    assert _need(Q4, rows, k, n) > 0
    say("4096x14336 at 512 tokens, split")
    Y, ws = _run_ws(W, Q4, k, X)
    rng = np.random.default_rng(14336)
    r_s, t_s = rng.integers(0, rows, 4096), rng.integers(0, n, 4096)
    y_ref, s = O.matmul_sampled(W, Q4, rows, k, W.shape[1], X, t_s, r_s)
    assert O.within_tolerance(Y[t_s, r_s], y_ref, s).all()
    Y0 = run_matmul(W, Q4, k, X)
    assert np.all(np.abs(Y - Y0) <= 2e-3 * np.abs(Y0).max())
    _counters_zero(ws, rows, n)
    for case in synth.config_cases()[4]:
        assert _need(case.qtype, case.rows, case.k, case.n_tokens) == 0, case.name
