"""MUL_MAT parity on the GPU: the decode kernel (GEMV) and the matrix-core
kernel (GEMM) against the oracle, element by element, within
|y - y_ref| <= 1e-3 * sum|w x| + 1e-5, plus closed-form invariants that hold
bitwise, and the configured workloads at their full sizes."""
import numpy as np
import pytest

import block_quantized_matmul_amd as qmm
import oracle.qmm_oracle as O
from block_quantized_matmul_amd import synth
import gpu_util
import torch
from gpu_util import assert_bitwise, assert_close_to_oracle, run_matmul, say

pytestmark = pytest.mark.gpu
Q4, Q41, Q8 = O.TYPE_Q4_0, O.TYPE_Q4_1, O.TYPE_Q8_0
Q50, Q51 = O.TYPE_Q5_0, O.TYPE_Q5_1
GEMV, GEMM, AUTO = qmm.QMM_PATH_GEMV, qmm.QMM_PATH_GEMM, qmm.QMM_PATH_AUTO


def _inputs(qtype, rows, k, n, extra=0, seed=0, xdt=np.float32, d_lo=0.001, d_hi=0.05):
    rng = np.random.Generator(np.random.PCG64([seed, qtype, rows, k, n, extra]))
    nb1 = synth.dense_row_bytes(qtype, k) + extra
    W = synth.make_weights(qtype, rows, k, nb1, rng, d_lo, d_hi)
    X = synth.make_activations(n, k, rng, xdt)
    return W, X


def _parity(W, qtype, k, X, path, offset=0, what=""):
    say(f"matmul {what} type={qtype} rows={W.shape[0]} k={k} nb1={W.shape[1]} n={X.shape[0]} "
        f"x={X.dtype} path={path} offset={offset}")
    Y = run_matmul(W, qtype, k, X, path, offset)
    return assert_close_to_oracle(Y, W, qtype, k, X, what)


# ------------------------------------------------------------ small shapes, every kernel variant
@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 7, 8])
def test_gemv_ragged(qtype, xdt, n):
    for rows, k, extra, offset in ((1, 32, 0, 0), (37, 96, 0, 0), (37, 96, 2, 2), (300, 512, 4, 0),
                                   (300, 512, 16, 0), (17, 4096, 256, 0), (33, 11008, 0, 2), (17, 11008, 0, 0),
                                   (45, 2048, 0, 4)):
        W, X = _inputs(qtype, rows, k, n, extra, xdt=xdt)
        _parity(W, qtype, k, X, GEMV, offset, f"gemv rows={rows} k={k}")


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("n", [5, 8])
def test_gemv_multi_row_group_workgroups(qtype, xdt, n):
    """Decode calls with 5 to 8 tokens on launches of more 16-row groups than
    CUs: each workgroup covers two row groups with one set of staged
    activations; 4112 rows make the last workgroup's second group fall past
    the matrix, and padded rows keep the streaming layout. Every element
    against the oracle, and the same outputs bitwise from the matrix written
    as a dense copy and from a run with the rows permuted."""
    rows, k = 4112, 512
    assert (rows + 15) // 16 > 256
    W, X = _inputs(qtype, rows, k, n, 16 * 3, xdt=xdt)
    y = run_matmul(W, qtype, k, X, GEMV)
    say(f"gemv two row groups per workgroup type={qtype} n={n} x={np.dtype(xdt).name}")
    assert_close_to_oracle(y, W, qtype, k, X, "gemv 2 row groups")
    dense = synth.dense_row_bytes(qtype, k)
    assert_bitwise(run_matmul(np.ascontiguousarray(W[:, :dense]), qtype, k, X, GEMV), y, "dense copy")
    perm = np.random.default_rng(11).permutation(rows)
    assert_bitwise(run_matmul(W[perm], qtype, k, X, GEMV), y[:, perm], "row permutation")


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("n", [1, 9, 16, 37, 128, 200])
def test_gemm_ragged(qtype, xdt, n):
    for rows, k, extra, offset in ((1, 32, 0, 0), (37, 96, 2, 2), (130, 160, 0, 0), (300, 512, 4, 0),
                                   (129, 4096, 256, 2)):
        W, X = _inputs(qtype, rows, k, n, extra, xdt=xdt)
        _parity(W, qtype, k, X, GEMM, offset, f"gemm rows={rows} k={k}")


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("xdt", [np.float16, np.float32])
def test_gemm_full_size_tiles(qtype, xdt):
    """More 128-row tiles than CUs: the 128-row tile variant (the ragged
    tests above are small enough to take the 64-row one), with ragged rows
    and tokens and an odd block count (rows only 2-byte aligned for the
    18-, 22- and 34-byte blocks), every element against the oracle."""
    rows, k, n = 4230, 288, 1030
    assert ((rows + 127) // 128) * ((n + 127) // 128) > 256
    W, X = _inputs(qtype, rows, k, n, xdt=xdt)
    say(f"gemm 128-row tiles type={qtype} x={np.dtype(xdt).name}")
    _parity(W, qtype, k, X, GEMM, 0, "gemm 128-row tiles")


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("rows,k,n,extra,offset", [(2000, 320, 4000, 0, 0), (2048, 256, 4096, 0, 2),
                                                   (3000, 384, 4000, 2, 0), (11003, 320, 505, 0, 0)])
def test_gemm_two_group_tiles(qtype, rows, k, n, extra, offset):
    """fp16 activations with 128 x 256 tiles for at least 2/3 of the CUs (172
    tiles, one round; 256 and 384 tiles on the 256 CUs): the two-group
    kernel, with ragged rows and tokens,
    an odd number of 64-wide stages (k = 320), 2-byte-aligned weights and
    padded rows (the unaligned staging), every element against the oracle,
    and bitwise the same as the fp32 copy of the activations (the one-group
    kernel, which adds the same products in the same order)."""
    assert ((rows + 127) // 128) * ((n + 255) // 256) in (172, 256, 384)
    W, X = _inputs(qtype, rows, k, n, extra, xdt=np.float16)
    say(f"gemm two-group tiles type={qtype} rows={rows} k={k} n={n} nb1={W.shape[1]} offset={offset}")
    Y = run_matmul(W, qtype, k, X, GEMM, offset)
    assert_close_to_oracle(Y, W, qtype, k, X, "gemm two-group tiles")
    say("fp32 copy of the activations")
    assert_bitwise(run_matmul(W, qtype, k, X.astype(np.float32), GEMM, offset), Y, "one-group vs two-group kernel")


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
def test_dispatch_and_cross_check(qtype):
    """AUTO picks GEMV up to 8 tokens; for n = 1..16 both kernels agree with
    the oracle (and therefore with each other) on the same inputs."""
    for n in range(1, 17):
        W, X = _inputs(qtype, 200, 1024, n, seed=n)
        ya = run_matmul(W, qtype, 1024, X, AUTO)
        yg = run_matmul(W, qtype, 1024, X, GEMM)
        expect = run_matmul(W, qtype, 1024, X, GEMV) if n <= 8 else yg
        assert_bitwise(ya, expect, f"auto n={n}")
        assert_close_to_oracle(yg, W, qtype, 1024, X, f"gemm n={n}")
        assert_close_to_oracle(ya, W, qtype, 1024, X, f"auto n={n}")


def _dword_aligned_copy(a: np.ndarray, dtype) -> tuple:
    """a on the GPU starting 4 bytes past a 16-byte boundary (the weakest
    alignment the boundary accepts for X, Y and out). Returns (keepalive, view)."""
    per = 4 // np.dtype(dtype).itemsize
    flat = torch.zeros(a.size + 16, dtype=torch.float32 if dtype == np.float32 else torch.float16, device="cuda")
    view = flat[per:per + a.size]
    view.copy_(torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).cuda())
    assert view.data_ptr() % 16 == 4
    return flat, view.view(a.shape)


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("xdt", [np.float32, np.float16])
@pytest.mark.parametrize("path,n", [(GEMV, 1), (GEMV, 8), (GEMM, 40)])
def test_dword_aligned_activations_and_outputs(qtype, xdt, path, n):
    """X and Y only 4-byte aligned: the same results, bit for bit, as with
    16-byte-aligned buffers, for a streamable and a general weight layout."""
    for rows, k, extra in ((64, 512, 0), (70, 1024, 10)):
        W, X = _inputs(qtype, rows, k, n, extra, xdt=xdt)
        say(f"dword-aligned X/Y type={qtype} x={np.dtype(xdt).name} path={path} n={n} rows={rows} k={k} pad={extra}")
        want = run_matmul(W, qtype, k, X, path)
        _keep, Wd = gpu_util.place_weights(W)
        _kx, Xd = _dword_aligned_copy(X, xdt)
        _ky, Yd = _dword_aligned_copy(np.zeros((n, rows), np.float32), np.float32)
        qmm.qmm_matmul_path(Wd, qtype, k, Xd, n_rows=rows, row_stride_bytes=W.shape[1], n_tokens=n, Y=Yd, path=path)
        torch.cuda.synchronize()
        got = Yd.cpu().numpy()
        assert_bitwise(got, want, "dword-aligned X/Y")
        assert_close_to_oracle(got, W, qtype, k, X, "dword-aligned X/Y")


# ------------------------------------------------------------ closed-form invariants
@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("path,n", [(GEMV, 1), (GEMV, 8), (GEMM, 24)])
def test_one_hot_activation(qtype, path, n):
    """x = e_j: every other product is an exact zero, so y equals the
    dequantised weight (decode kernel) or its fp16 rounding (matrix cores)."""
    rows, k = 70, 512
    W, _ = _inputs(qtype, rows, k, 1, 6, d_lo=-1.5, d_hi=1.5)
    cols = np.array([0, 1, 15, 16, 31, 32, 250, k - 1] * 3)[:n]
    X = np.zeros((n, k), np.float32)
    X[np.arange(n), cols] = 1.0
    say(f"one-hot type={qtype} path={path} n={n}")
    Y = run_matmul(W, qtype, k, X, path)
    w = O.dequantize(W, qtype, rows, k, W.shape[1])[:, cols].T
    if path == GEMM:
        # the matrix cores take fp16(d (q - z)) or, for Q4_1, fp16(d q + m):
        # one rounding of the exact weight (exact in fp64)
        d, q = O.block_scales_and_codes(W, qtype, rows, k, W.shape[1])
        m = O.block_mins(W, qtype, rows, k, W.shape[1])
        exact = np.repeat(d, 32, axis=1) * (q - O.ZERO_POINT[qtype]) + np.repeat(m, 32, axis=1)
        w = exact[:, cols].T.astype(np.float16).astype(np.float32)
    # a zero weight may be -0.0 (negative d times code 0); sums give +0.0
    assert_bitwise(Y + np.float32(0.0), w + np.float32(0.0), "one-hot")


@pytest.mark.parametrize("qtype", [Q4, Q41, Q50, Q51, Q8])
@pytest.mark.parametrize("path,n", [(GEMV, 3), (GEMM, 40)])
def test_zero_codes_scaling_permutation_padding_determinism(qtype, path, n):
    rows, k = 150, 1024
    W, X = _inputs(qtype, rows, k, n, 10)
    # keep |x| away from the fp16 subnormal range so fp16(4 x) == 4 fp16(x)
    X = np.where(np.abs(X) < 1e-3, np.float32(1e-3), X).astype(np.float32)
    say(f"invariants type={qtype} path={path} n={n}")
    y = run_matmul(W, qtype, k, X, path)
    # determinism
    assert_bitwise(run_matmul(W, qtype, k, X, path), y, "rerun")
    # y(2^e x) = 2^e y(x)
    assert_bitwise(run_matmul(W, qtype, k, X * np.float32(4.0), path), 4.0 * y, "scale x by 4")
    # permuting rows permutes outputs
    perm = np.random.default_rng(5).permutation(rows)
    assert_bitwise(run_matmul(W[perm], qtype, k, X, path), y[:, perm], "row permutation")
    # padding bytes are never read; a dense copy gives the same result
    W2 = W.copy()
    W2[:, -10:] ^= 0xA5
    assert_bitwise(run_matmul(W2, qtype, k, X, path), y, "padding refill")
    dense = synth.dense_row_bytes(qtype, k)
    assert_bitwise(run_matmul(np.ascontiguousarray(W[:, :dense]), qtype, k, X, path), y, "dense copy")
    # zero codes (q = z) give exactly zero
    Wz = W.copy().reshape(rows, -1)
    bpb = O.BLOCK_BYTES[qtype]
    blk = Wz[:, :dense].reshape(rows, -1, bpb)
    blk[:, :, 2:] = 0x88 if qtype == Q4 else 0  # codes equal to the zero point (and m = 0)
    if qtype == Q50:
        blk[:, :, 2:6] = 0xFF  # fifth bits set: codes 16
    Wz[:, :dense] = blk.reshape(rows, dense)
    yz = run_matmul(Wz, qtype, k, X, path)
    assert np.all(yz == 0.0)


@pytest.mark.parametrize("path,n", [(GEMV, 2), (GEMM, 20)])
def test_nonfinite_scale_propagates(path, n):
    rows, k = 20, 256
    W, X = _inputs(Q4, rows, k, n)
    W[3, 0:2] = [0x00, 0x7E]        # NaN scale, block 0 of row 3
    W[7, 18 * 2:18 * 2 + 2] = [0x00, 0x7C]  # +inf scale, block 2 of row 7
    say(f"non-finite scales path={path}")
    Y = run_matmul(W, Q4, k, X, path)
    assert np.all(np.isnan(Y[:, 3]))
    assert not np.any(np.isfinite(Y[:, 7]))
    others = np.delete(np.arange(rows), [3, 7])
    assert np.all(np.isfinite(Y[:, others]))
    assert_close_to_oracle(Y[:, others], W[others], Q4, k, X, "finite rows")


# ------------------------------------------------------------ configured workloads, full size
def _run_case(case, path=AUTO):
    W, X = case.weights(), case.activations()
    return _parity(W, case.qtype, case.k, X, path, 0, case.name)


def test_config1_single_gemv():
    for case in synth.config_cases()[1]:
        _run_case(case)


def test_config2_decode_projections():
    for case in synth.config_cases()[2]:
        _run_case(case)


def test_config3_output_projection_padded():
    cases = synth.config_cases()[3]
    W = cases[0].weights()
    for case in cases:
        X = case.activations()
        say(f"{case.name}")
        Y = run_matmul(W, case.qtype, case.k, X)
        rng = np.random.default_rng(case.n_tokens)
        rows = rng.integers(0, case.rows, 2048)
        toks = rng.integers(0, case.n_tokens, 2048)
        y_ref, s = O.matmul_sampled(W, case.qtype, case.rows, case.k, case.nb1, X, toks, rows)
        assert O.within_tolerance(Y[toks, rows], y_ref, s).all(), case.name
    # padding must be ignored: refill it and compare bitwise at n = 8
    W2 = W.copy()
    W2[:, 2304:] = 255 - W2[:, 2304:]
    X = cases[-1].activations()
    assert_bitwise(run_matmul(W2, Q4, 4096, X), run_matmul(W, Q4, 4096, X), "padding refill")


def test_config4_prefill_gemm():
    for case in synth.config_cases()[4]:
        W, X = case.weights(), case.activations()
        say(case.name)
        Y16 = run_matmul(W, case.qtype, case.k, X)        # fp16 activations (qmm_matmul_x16)
        Y32 = run_matmul(W, case.qtype, case.k, X.astype(np.float32))  # the same values as fp32
        assert_bitwise(Y32, Y16, "fp32 copy of fp16 activations")
        rng = np.random.default_rng(case.rows)
        rows = rng.integers(0, case.rows, 4096)
        toks = rng.integers(0, case.n_tokens, 4096)
        y_ref, s = O.matmul_sampled(W, case.qtype, case.rows, case.k, case.nb1, X, toks, rows)
        assert O.within_tolerance(Y16[toks, rows], y_ref, s).all(), case.name
    for c in synth.config_cases()[4]:
        _run_case(c)  # 4096 x 4096 and 11008 x 4096 element by element


def _stack_layer_sampled(n_tokens, layer, m=4096):
    for case in synth.stack_cases(n_tokens, layers=layer + 1)[7 * layer:]:
        W, X = case.weights(), case.activations()
        say(case.name)
        Y = run_matmul(W, case.qtype, case.k, X)
        rng = np.random.default_rng(case.layer * 10 + case.tensor)
        rows = rng.integers(0, case.rows, m)
        toks = rng.integers(0, case.n_tokens, m)
        y_ref, s = O.matmul_sampled(W, case.qtype, case.rows, case.k, case.nb1, X, toks, rows)
        assert O.within_tolerance(Y[toks, rows], y_ref, s).all(), case.name


@pytest.mark.parametrize("layer", range(synth.N_LAYER))
def test_config5_stack_decode_every_layer_sampled(layer):
    """Every layer's seven full-size tensors of the 32-layer stack at one
    token, in the launch configuration the benchmark times, checked on
    sampled outputs."""
    _stack_layer_sampled(1, layer)


def test_config5_stack_prefill_last_layer_sampled():
    _stack_layer_sampled(2048, synth.N_LAYER - 1)


def test_config5_stack_prefill_layer0_full():
    """Layer 0 of the stack at 2048 fp16 tokens, all seven tensors element by
    element (2048 x 4096 and 2048 x 11008 outputs)."""
    for case in synth.stack_cases(2048, layers=1):
        _run_case(case)


def test_config5_decode_batched_as_benchmarked():
    """Layers 0 and 31 of the stack at one token through qmm_matmul_batch in
    exactly the benchmark's launch groups (q+k+v, o, gate+up, down, whose
    batched launches split k by their own size), checked on sampled outputs
    of every tensor."""
    import torch
    import bench
    from gpu_util import dev
    cases = {(c.layer, c.tensor): c for c in synth.stack_cases(1) if c.layer in (0, 31)}
    for layer in (0, 31):
        for grp in bench.LAYER_GROUPS:
            items, host = [], []
            for t in grp:
                c = cases[(layer, t)]
                W, X = c.weights(), c.activations()
                items.append((dev(W), c.qtype, c.k, dev(X), torch.empty((1, c.rows), dtype=torch.float32, device="cuda")))
                host.append((c, W, X))
            say(f"decode batch layer {layer} tensors {grp}")
            qmm.qmm_matmul_batch(items)
            torch.cuda.synchronize()
            for (c, W, X), it in zip(host, items):
                rng = np.random.default_rng(1000 * layer + c.tensor)
                rows = np.unique(np.concatenate([[0, 15, 16, c.rows - 1], rng.integers(0, c.rows, 1500)]))
                y_ref, s = O.matmul_sampled(W, c.qtype, c.rows, c.k, c.nb1, X, np.zeros_like(rows), rows)
                assert O.within_tolerance(it[4].cpu().numpy()[0, rows], y_ref, s).all(), c.name


def test_config5_prefill_batched_as_benchmarked():
    """Layer 0 of the stack at 2048 fp16 tokens through qmm_matmul_batch_ws in
    the benchmark's launch groups (q+k+v in one two-group launch, o, gate+up
    in one launch whose last round is split in k, down), sampled outputs of
    every tensor against the oracle, with one workspace for all groups."""
    import torch
    import bench
    from gpu_util import dev
    cases = {c.tensor: c for c in synth.stack_cases(2048, layers=1)}
    groups = []
    for grp in bench.LAYER_GROUPS:
        items, host = [], []
        for t in grp:
            c = cases[t]
            W, X = c.weights(), c.activations()
            items.append((dev(W), c.qtype, c.k, dev(X),
                          torch.full((c.n_tokens, c.rows), float("nan"), dtype=torch.float32, device="cuda")))
            host.append((c, W, X))
        groups.append((grp, items, host))
    need = max(qmm.qmm_matmul_batch_workspace_bytes(items) for _, items, _ in groups)
    assert need > 0, "the gate+up launch should split its last round"
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for grp, items, host in groups:
        say(f"prefill batch layer 0 tensors {grp}")
        qmm.qmm_matmul_batch_ws(items, ws)
        torch.cuda.synchronize()
        for (c, W, X), it in zip(host, items):
            rng = np.random.default_rng(2000 + c.tensor)
            rows = np.concatenate([[0, 127, 128, c.rows - 1], rng.integers(0, c.rows, 3000)])
            toks = np.concatenate([[0, 255, 256, c.n_tokens - 1], rng.integers(0, c.n_tokens, 3000)])
            y_ref, s = O.matmul_sampled(W, c.qtype, c.rows, c.k, c.nb1, X, toks, rows)
            assert O.within_tolerance(it[4].cpu().numpy()[toks, rows], y_ref, s).all(), c.name
    tail = 2 * 86 * 8 % torch.cuda.get_device_properties(0).multi_processor_count   # gate+up: 1376 tiles
    assert torch.count_nonzero(ws[:4 * tail]).item() == 0, "split counters not back at zero"


# ------------------------------------------------------------ batched calls and graph replay
def _batch_specs():
    # (type, rows, k, n_tokens, x dtype): streaming-eligible, general-kernel and matrix-core entries,
    # in an order that forces several launch groups
    return [(Q4, 300, 4096, 1, np.float32), (Q4, 4096, 512, 1, np.float32), (Q4, 129, 11008, 1, np.float32),
            (Q8, 77, 1024, 1, np.float32), (Q4, 40, 96, 1, np.float32), (Q4, 33, 4096, 3, np.float32),
            (Q4, 64, 2048, 8, np.float16), (Q8, 50, 4096, 20, np.float16), (Q4, 16, 256, 2, np.float32)] + \
           [(Q4, 16 * (i + 1), 256 * (1 + i % 3), 1, np.float32) for i in range(20)]


def _batch_items(specs, seed=0):
    import torch
    from gpu_util import dev
    host, items = [], []
    for i, (qt, rows, k, n, xdt) in enumerate(specs):
        W, X = _inputs(qt, rows, k, n, seed=seed + i, xdt=xdt)
        Wd, Xd = dev(W), dev(X)
        Y = torch.full((n, rows), float("nan"), dtype=torch.float32, device="cuda")
        host.append((W, X, qt, k))
        items.append((Wd, qt, k, Xd, Y))
    return host, items


def test_batch_matches_single_calls_and_oracle():
    """Every output of a mixed batch is within the tolerance of the oracle and
    reproducible bitwise; a batch of one MUL_MAT is bitwise the single call.
    (A batched launch may split k differently from a single call of the same
    matrix, since the split follows the launch's size, so across the two only
    the tolerance is promised.)"""
    import torch
    specs = _batch_specs()
    host, items = _batch_items(specs)
    say(f"batch of {len(items)}")
    qmm.qmm_matmul_batch(items)
    torch.cuda.synchronize()
    first = [it[4].cpu().numpy() for it in items]
    for it in items:
        it[4].fill_(float("nan"))
    qmm.qmm_matmul_batch(items)
    torch.cuda.synchronize()
    for (W, X, qt, k), (_, _, _, _, Y), y0 in zip(host, items, first):
        y = Y.cpu().numpy()
        assert_bitwise(y, y0, f"batch rerun {W.shape}")
        assert_close_to_oracle(y, W, qt, k, X, f"batch {W.shape}")
        assert_close_to_oracle(run_matmul(W, qt, k, X, AUTO), W, qt, k, X, f"single {W.shape}")
    for i in (0, 1, 6):
        W, X, qt, k = host[i]
        qmm.qmm_matmul_batch([items[i]])
        torch.cuda.synchronize()
        assert_bitwise(items[i][4].cpu().numpy(), run_matmul(W, qt, k, X, AUTO), f"batch of one vs single {W.shape}")


def test_graph_replay_matches_eager():
    """A captured graph (batched call + single calls) replayed several times,
    with eager work in between, reproduces the eager results every time."""
    import torch
    host, items = _batch_items(_batch_specs()[:9], seed=100)
    W0, qt0, k0, X0, _ = items[0]
    Ys = torch.empty((X0.shape[0], W0.shape[0]), dtype=torch.float32, device="cuda")
    Yg = torch.empty((40, W0.shape[0]), dtype=torch.float32, device="cuda")
    Xg = torch.randn((40, k0), dtype=torch.float32, device="cuda")

    def work():
        qmm.qmm_matmul_batch(items)
        qmm.qmm_matmul(W0, qt0, k0, X0, Y=Ys)
        qmm.qmm_matmul(W0, qt0, k0, Xg, Y=Yg)

    say("graph capture")
    work()
    torch.cuda.synchronize()
    ref = [it[4].clone() for it in items] + [Ys.clone(), Yg.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        for t in [it[4] for it in items] + [Ys, Yg]:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        out = [it[4] for it in items] + [Ys, Yg]
        for a, b in zip(out, ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = (Xg * 2).sum().item()  # unrelated eager work between replays


def test_binding_rejects_short_buffers():
    """The binding refuses buffers smaller than the sizes it passes to the C
    ABI (which trusts them), before anything is launched."""
    rows, k = 64, 256
    W, X = _inputs(Q4, rows, k, 3)
    Wd, Xd = torch.from_numpy(W).cuda(), torch.from_numpy(X).cuda()
    with pytest.raises(ValueError):
        qmm.qmm_matmul(Wd, Q4, k, Xd, Y=torch.empty((3, rows - 1), device="cuda"))
    with pytest.raises(ValueError):
        qmm.qmm_matmul(Wd[:-1], Q4, k, Xd, n_rows=rows, row_stride_bytes=W.shape[1])
    with pytest.raises(ValueError):
        qmm.qmm_matmul(Wd, Q4, k, Xd[:2], n_tokens=3)
    with pytest.raises(ValueError):
        qmm.qmm_dequantize(Wd, Q4, k, out=torch.empty((rows, k - 1), device="cuda"))
    ids = torch.zeros(5, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        qmm.qmm_get_rows(Wd, Q4, k, ids, out=torch.empty((4, k), device="cuda"))
    with pytest.raises(ValueError):
        qmm.qmm_matmul_id(Wd.view(2, rows // 2, -1), Q4, k, Xd.view(3, 1, k),
                          torch.zeros((3, 2), dtype=torch.int32, device="cuda"),
                          Y=torch.empty((3, 2, rows // 2 - 1), device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("seed", range(6))
def test_random_layouts_sweep(seed):
    """Seeded random cases across everything the dispatch looks at: weight
    type, rows, k (odd block counts included), row padding, a 2-byte-offset
    W, token count on both sides of the decode/GEMM switch, activation type.
    Each case is compared element by element with the oracle."""
    rng = np.random.Generator(np.random.PCG64([600, seed]))
    for case in range(7):
        qtype = int(rng.choice([Q4, Q41, Q50, Q51, Q8]))
        rows = int(rng.integers(1, 700))
        k = 32 * int(rng.integers(1, 80))
        extra = 2 * int(rng.integers(0, 40))
        offset = int(rng.choice([0, 2]))
        n = int(rng.choice([1, 2, 3, 5, 8, 9, 17, 64, 130, 300]))
        xdt = np.float16 if rng.random() < 0.5 else np.float32
        W, X = _inputs(qtype, rows, k, n, extra, seed=1000 * seed + case, xdt=xdt)
        _parity(W, qtype, k, X, AUTO, offset, f"sweep {seed}.{case}")
