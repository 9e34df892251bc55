"""Benchmark: block-quantized MUL_MAT over a 32-layer Llama-7B-shaped Q4_0 stack.

One step = the whole hot path over one batch of synthetic input:
  decode  - the 224 MUL_MATs of the stack (7 per layer x 32 layers) at
            n_tokens = 1 with fp32 activations, on the decode (GEMV) kernel.
            Each layer's MUL_MATs go through qmm_matmul_batch in the groups a
            transformer layer can issue together because none needs another's
            output: {attn_q, attn_k, attn_v}, {attn_output}, {ffn_gate,
            ffn_up}, {ffn_down} - 4 launches per layer, 128 per pass. 3.64 GB
            of Q4_0 blocks are read once per pass, far more than the 256 MB
            Infinity Cache holds.
  prefill - the same 224 weights, each with a 2048-token fp16 ubatch, on the
            matrix-core (GEMM) kernel, in the same groups through
            qmm_matmul_batch_ws: the group's MUL_MATs share one two-group
            launch (q|k|v: 768 tiles, three full rounds on 256 CUs; gate|up:
            1376 tiles, whose last round of 96 is split in k over the
            workspace) - 4 launches per layer.
Each pass is captured once into a HIP graph (its launches are exactly the C
entry points' launches) and replayed; HIP events on the launch stream time
every pass. Inputs are resident in HBM before the timed region starts. With
--per-call, the decode and prefill passes with one launch per MUL_MAT
(qmm_matmul, qmm_matmul_x16) are timed after the steps as well.

Prints ONE JSON line. `value` is the decode pass's achieved HBM bandwidth:
algorithmic bytes (weight blocks + activations + outputs) per pass / pass
time. `roofline` divides the decode kernel's algorithmic bytes per launch by
its average launch duration (pass time / launches); `roofline_prefill` does
the same with 2 * rows * k * tokens flops for the GEMM kernel. `traffic` is
the HBM bytes per launch that hardware counters measured, read from the
counter summaries under profiles/ - null when the kernel's source has changed
since they were taken. The CPU oracle is timed on a bounded sample of the
same decode workload.

  python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--layers 32]
                  [--cpu-layers 4] [--no-cpu-baseline] [--per-call] [--copy-calibration]
  python bench.py --summarize-trace DIR      (rocprofv3 -f csv kernel trace)
  python bench.py --only PASS [--steps K] [--layers L] [--copy-calibration]
  python bench.py --summarize-counters DIR... (rocprofv3 -f csv --pmc runs)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Q4_0 decode GEMV HBM GB/s (% of peak); prefill GEMM TFLOP/s (% MFMA peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak
DECODE_TOKENS = 1
PREFILL_TOKENS = 2048
# Launch groups of one layer (indices into synth.LAYER_TENSORS): MUL_MATs in a
# group share no data dependency.
LAYER_GROUPS = ((0, 1, 2), (3,), (4, 5), (6,))
COPY_CAL_BYTES = 1 << 30        # size of the plain copy used to calibrate counters

CSRC = os.path.join(ROOT, "block_quantized_matmul_amd", "csrc")
KERNELS = {
    # name fragment in the kernel symbol -> sources the kernel is built from
    "gemv_stream_kernel": ("gemv_stream.hip", "gemv_common.h", "common.h", "launch.h"),
    "gemv_tall_kernel": ("gemv_stream.hip", "gemv_common.h", "common.h", "launch.h"),
    "gemm_kernel": ("gemm.hip", "common.h", "launch.h"),
    "gemm_pp_kernel": ("gemm.hip", "common.h", "launch.h"),
    "gemm_pp_routed_kernel": ("gemm.hip", "common.h", "launch.h"),
}
# Template arguments of the plain (MUL_MAT) instantiations; the expert-routed
# (MUL_MAT_ID) ones carry one more, which the demangled name shows (for
# gemm_pp_kernel that flag marks the k-split form, kept apart the same way).
KERNEL_TARGS = {"gemv_stream_kernel": 4, "gemv_tall_kernel": 3, "gemm_kernel": 3, "gemm_pp_kernel": 2,
                "gemm_pp_routed_kernel": 2}
# Kernels whose extra flag marks a k-split form of the same MUL_MAT rather
# than MUL_MAT_ID: their traffic counts every form (the stack's prefill pass
# launches both), and trace summaries list the forms apart and together.
SPLIT_FORM = {"gemm_pp_kernel"}
PROFILES = os.path.join(ROOT, "profiles")


def _code_only(text: str) -> str:
    """Source text without comments and blank lines, so that editing a
    comment does not mark the recorded counters as stale."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_hash(kernel: str) -> str:
    """Hash of the code (comments stripped) of the sources `kernel` is built from."""
    h = hashlib.sha256()
    for f in KERNELS[kernel]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-get-rows", action="store_true", help="skip the GET_ROWS (token-embedding gather) line")
    ap.add_argument("--no-matmul-id", action="store_true", help="skip the MUL_MAT_ID (routed expert FFN) lines")
    ap.add_argument("--no-other-types", action="store_true", help="skip the Q8_0 / Q4_1 / Q5_0 / Q5_1 / Q4_K lines")
    ap.add_argument("--cpu-layers", type=int, default=4, help="layers of the decode pass the oracle times")
    ap.add_argument("--per-call", action="store_true",
                    help="also time the decode and prefill passes with one launch per MUL_MAT")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"also run one plain {COPY_CAL_BYTES >> 20} MiB device copy (for counter calibration)")
    ap.add_argument("--only", choices=("decode", "decode_per_call", "prefill", "prefill_per_call",
                                       "output_projection", "prefill_512",
                                       "matmul_id"),
                    help="run just this pass (eagerly once, then --steps graph replays) and print no JSON; "
                         "for hardware-counter runs, whose per-dispatch averages must cover one pass only")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-counters", metavar="DIR", nargs="+")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- profiles

def _find(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0], newline="") as fh:
        return list(csv.DictReader(fh))


def _demangle_simple(name):
    """qmm::kernel<...> for an Itanium-mangled kernel symbol whose template
    arguments are integers and booleans (the form rocprofv3 sometimes
    reports), else the name unchanged."""
    m = re.match(r"_ZN((?:\d+[A-Za-z_]\w*?)+)I((?:L[ib]\d+E)+)EE", name)
    if not m:
        return name
    parts, rest = [], m.group(1)
    while rest:
        n = re.match(r"\d+", rest).group(0)
        parts.append(rest[len(n):len(n) + int(n)])
        rest = rest[len(n) + int(n):]
    args = [("true" if v == "1" else "false") if t == "b" else v for t, v in re.findall(r"L([ib])(\d+)E", m.group(2))]
    return "::".join(parts) + "<" + ", ".join(args) + ">"


def _short(name):
    name = _demangle_simple(name).replace("(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name).replace("void ", "")


def _routed(name, kern):
    """True for the expert-routed instantiation of `kern`: its last template
    argument (the routing flag, which a demangled name may omit when it has
    its default, false) is true."""
    m = re.search(re.escape(kern) + r"<([^>]*)>", name)
    if not m:
        return False
    args = [a.strip() for a in m.group(1).split(",")]
    return len(args) > KERNEL_TARGS[kern] and args[KERNEL_TARGS[kern]] == "true"


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def summarize_trace(d):
    """Per-kernel dispatch statistics of a rocprofv3 --kernel-trace -f csv run."""
    by = {}
    for r in _find(d, "kernel_trace.csv"):
        key = (_short(r["Kernel_Name"]), int(_col(r, "Grid_Size_X", "Grid_Size")))
        by.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"{'kernel':58s} {'grid_x':>9s} {'calls':>6s} {'avg_us':>9s} {'med_us':>9s} {'min_us':>9s} {'max_us':>9s}")
    for (k, gx), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        print(f"{k[:58]:58s} {gx:9d} {len(v):6d} {statistics.mean(v):9.2f} {statistics.median(v):9.2f} "
              f"{min(v):9.2f} {max(v):9.2f}")
    for kern in KERNELS:
        groups = {}
        for (k, _), xs in by.items():
            m = re.search(re.escape(kern) + r"<(\d+)", k)
            if m:
                groups.setdefault((int(m.group(1)), _routed(k, kern)), []).extend(xs)
        for (qt, routed), v in sorted(groups.items()):
            tag = (" split" if kern in SPLIT_FORM else " routed") if routed else ""
            print(f"ALL {kern} type {qt}{tag}: calls {len(v)} avg_us {statistics.mean(v):.3f} "
                  f"source_sha256 {source_hash(kern)}")
        if kern in SPLIT_FORM:
            for qt in sorted({q for q, _ in groups}):
                if (qt, False) in groups and (qt, True) in groups:
                    v = groups[(qt, False)] + groups[(qt, True)]
                    print(f"ALL {kern} type {qt} every form: calls {len(v)} avg_us {statistics.mean(v):.3f} "
                          f"source_sha256 {source_hash(kern)}")


def summarize_counters(dirs):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of rocprofv3 --pmc -f csv
    runs, per kernel. Each counter is scaled by the factor that makes the
    plain device copy of COPY_CAL_BYTES (run by --copy-calibration) read, or
    write, exactly that many bytes; the scaled sum is the HBM traffic per
    launch."""
    per = {}
    for d in dirs:
        for r in _find(d, "counter_collection.csv"):
            key = (_short(r["Kernel_Name"]), r["Dispatch_Id"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    agg = {}
    for (k, _, cn), v in per.items():
        agg.setdefault((k, cn), []).append(v)
    for (k, cn), v in sorted(agg.items()):
        unit = "avg_KiB" if cn in ("FETCH_SIZE", "WRITE_SIZE") else "avg"
        print(f"{k[:58]:58s} {cn:11s} dispatches {len(v):5d} {unit} {statistics.mean(v):14.1f}")
    factor = {}
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        cal = [v for (k, c), vs in agg.items() if c == cn and "copyBuffer" in k for v in vs
               if v * 1024 > COPY_CAL_BYTES / 4]
        if cal:
            factor[cn] = COPY_CAL_BYTES / (statistics.mean(cal) * 1024)
            print(f"CALIBRATION {cn}: copy of {COPY_CAL_BYTES} bytes counts {statistics.mean(cal) * 1024:.0f} "
                  f"(factor {factor[cn]:.4f}, {len(cal)} dispatches)")
    for kern in KERNELS:
        total = 0.0
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            v = [x for (k, c), xs in agg.items()
                 if kern in k and (kern in SPLIT_FORM or not _routed(k, kern)) and c == cn for x in xs]
            if not v or cn not in factor:
                total = None
                break
            total += statistics.mean(v) * 1024 * factor[cn]
            print(f"{kern} {cn}: dispatches {len(v)} avg_KiB {statistics.mean(v):.1f} scaled_bytes "
                  f"{statistics.mean(v) * 1024 * factor[cn]:.0f}")
        if total is not None:
            print(f"TRAFFIC {kern} bytes_per_launch {total:.0f} source_sha256 {source_hash(kern)}")


def traffic_from_profiles(kernel, profile):
    """HBM bytes per launch of `kernel` recorded in profiles/<profile> (a line
    'TRAFFIC <kernel> bytes_per_launch <B> source_sha256 <h>', taken on the
    workload that profile names), or None if it holds none for the current
    source."""
    h = source_hash(kernel)
    f = os.path.join(PROFILES, profile)
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        for line in fh:
            m = re.match(r"TRAFFIC (\S+) bytes_per_launch (\d+) source_sha256 (\w+)", line)
            if m and m.group(1) == kernel and m.group(3) == h:
                return int(m.group(2))
    return None


# ---------------------------------------------------------------- GET_ROWS

GET_ROWS_IDS = 2048


def time_get_rows(torch, qmm, synth, with_oracle=False):
    """GET_ROWS of one prefill ubatch (2048 token ids) from the model's
    32000x4096 Q4_0 token-embedding matrix: back-to-back launches in a graph,
    rotating over >= 1 GiB of matrix copies so the gathered rows come from
    HBM. Algorithmic bytes: the gathered rows' blocks, the ids and the fp32
    output (HBM-bound decoder)."""
    import numpy as np
    rows, k, qt = 32000, 4096, synth.TYPE_Q4_0
    nb1 = synth.dense_row_bytes(qt, k)
    rng = np.random.Generator(np.random.PCG64(4242))
    W0 = torch.from_numpy(synth.make_weights(qt, rows, k, nb1, rng)).cuda()
    copies = int(np.ceil(1.1 * 2**30 / W0.numel()))
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    ids = torch.from_numpy(rng.integers(0, rows, size=GET_ROWS_IDS).astype(np.int32)).cuda()
    out = torch.empty((GET_ROWS_IDS, k), dtype=torch.float32, device="cuda")
    reps = 4 * copies

    def run():
        for i in range(reps):
            qmm.qmm_get_rows(Ws[i % copies], qt, k, ids, out=out)

    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(5):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / reps)
    us = sorted(ts)[2]
    byts = GET_ROWS_IDS * (nb1 + 4 + 4 * k)
    gbs = byts / (us * 1e-6) / 1e9
    res = {"workload": f"{GET_ROWS_IDS} ids into a {rows}x{k} Q4_0 matrix", "us_per_launch": round(us, 3),
           "algorithmic_bytes_per_launch": byts, "GB_per_s": round(gbs, 2),
           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "kernel": "dequant_kernel", "bound": "hbm"}
    if with_oracle:
        # the oracle as it stands (it dequantises the whole matrix, then gathers), once, on the host
        import oracle.qmm_oracle as O
        Wh, idh = W0.cpu().numpy(), ids.cpu().numpy()
        t0 = time.perf_counter()
        O.get_rows(Wh, qt, rows, k, nb1, idh)
        res["cpu_oracle_us"] = round((time.perf_counter() - t0) * 1e6, 1)
    return res


# ---------------------------------------------------------------- other legacy types

def time_type(torch, qmm, synth, qt, with_oracle=False):
    """Another weight type (Q8_0, Q4_1, Q5_0, Q5_1, Q4_K) on the 11008x4096 FFN
    projection: decode (1 fp32 token) and prefill (2048 fp16 tokens),
    back-to-back launches in a graph over >= 1.1 GiB of weight copies, so
    weights come from HBM."""
    import numpy as np
    rows, k = 11008, 4096
    rng = np.random.Generator(np.random.PCG64(4100 + qt))
    Wh = synth.make_weights(qt, rows, k, None, rng)
    W0 = torch.from_numpy(Wh).cuda()
    copies = int(np.ceil(1.1 * 2**30 / W0.numel()))
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    Xh = synth.make_activations(1, k, rng)
    X1 = torch.from_numpy(Xh).cuda()
    Y1 = torch.empty((1, rows), dtype=torch.float32, device="cuda")
    reps = 4 * copies
    us = _graph_time(torch, lambda: [qmm.qmm_matmul(Ws[i % copies], qt, k, X1, Y=Y1) for i in range(reps)], reps)
    byts = W0.numel() + 4 * k + 4 * rows
    gbs = byts / (us * 1e-6) / 1e9
    T = 2048
    X2 = torch.from_numpy(synth.make_activations(T, k, rng, np.float16)).cuda()
    Y2 = torch.empty((T, rows), dtype=torch.float32, device="cuda")
    us2 = _graph_time(torch, lambda: [qmm.qmm_matmul_x16(Ws[i % copies], qt, k, X2, Y=Y2) for i in range(copies)],
                      copies)
    tfl = 2 * T * rows * k / (us2 * 1e-6) / 1e12
    res = {"workload": f"{rows}x{k} {synth.TYPE_NAMES[qt].upper()}",
           "decode": {"tokens": 1, "us_per_launch": round(us, 3), "algorithmic_bytes_per_launch": byts,
                      "GB_per_s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "kernel": "gemv_stream_kernel", "bound": "hbm"},
           "prefill": {"tokens": T, "us_per_launch": round(us2, 3), "TFLOP_per_s": round(tfl, 2),
                       "frac_of_mfma_f16_peak": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
                       "kernel": "gemm_pp_kernel", "bound": "mfma"}}
    if with_oracle:
        import oracle.qmm_oracle as O
        t0 = time.perf_counter()
        O.matmul(Wh, qt, rows, k, Wh.shape[1], Xh)
        res["decode"]["cpu_oracle_us"] = round((time.perf_counter() - t0) * 1e6, 1)
    return res


# ---------------------------------------------------------------- output projection and 512-token prefill

def _roof(achieved, peak, unit, bound):
    return {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None}


def time_output_projection(torch, qmm, synth):
    """The output-projection workload: Q4_0 32000x4096 with rows padded to
    nb1 = 2560 (256 random padding bytes per row), fp32 activations of 1, 2,
    4 and 8 tokens, on the decode kernels (the k-split kernel at 1 and 2
    tokens, the row-split one at 4 and 8). Back-to-back launches in a graph
    over >= 1.1 GiB of weight copies, so the weights come from HBM.
    Algorithmic bytes: the blocks (padding excluded), X and Y."""
    import numpy as np
    rows, k, nb1, qt = synth.N_VOCAB, synth.N_EMBD, 2560, synth.TYPE_Q4_0
    rng = np.random.Generator(np.random.PCG64(4400))
    W0 = torch.from_numpy(synth.make_weights(qt, rows, k, nb1, rng)).cuda()
    copies = int(np.ceil(1.1 * 2**30 / W0.numel()))
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    reps = 4 * copies
    out = {"workload": f"{rows}x{k} Q4_0, nb1 = {nb1} (padded rows), fp32 activations"}
    for n in (1, 2, 4, 8):
        X = torch.from_numpy(synth.make_activations(n, k, rng)).cuda()
        Y = torch.empty((n, rows), dtype=torch.float32, device="cuda")
        us = _graph_time(torch, lambda: [qmm.qmm_matmul(Ws[i % copies], qt, k, X, Y=Y) for i in range(reps)], reps)
        byts = rows * synth.dense_row_bytes(qt, k) + 4 * n * k + 4 * n * rows
        gbs = byts / (us * 1e-6) / 1e9
        # 3 to 8 tokens on this tall matrix: the row-split kernel
        out[f"n{n}"] = {"tokens": n, "us_per_launch": round(us, 3), "algorithmic_bytes_per_launch": byts,
                        "GB_per_s": round(gbs, 2), "kernel": "gemv_tall_kernel" if n >= 3 else "gemv_stream_kernel",
                        "roofline": _roof(gbs, HBM_PEAK_GBS, "GB/s", "hbm")}
    return out


def time_prefill_512(torch, qmm, synth):
    """The 512-token prefill workload: Q4_0 4096x4096 and 11008x4096 with
    fp16 activations of 512 tokens (the batch of the capability probe), on
    the matrix-core kernel; back-to-back launches in a graph over >= 1.1 GiB
    of weight copies. Flops: 2 * rows * k * tokens. Beside them, the
    4096x11008 down projection at the same batch through qmm_matmul_ws (the
    k split), with the unsplit launch's time, and a layer's three 4096x4096
    q, k, v projections in one qmm_matmul_batch call."""
    import numpy as np
    qt, k, T = synth.TYPE_Q4_0, synth.N_EMBD, 512
    rng = np.random.Generator(np.random.PCG64(4500))
    out = {"workload": f"Q4_0 4096x4096 and 11008x4096 (and the 4096x11008 down projection), {T} fp16 tokens"}
    for rows in (synth.N_EMBD, synth.N_FF):
        W0 = torch.from_numpy(synth.make_weights(qt, rows, k, None, rng)).cuda()
        copies = int(np.ceil(1.1 * 2**30 / W0.numel()))
        Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
        X = torch.from_numpy(synth.make_activations(T, k, rng, np.float16)).cuda()
        Y = torch.empty((T, rows), dtype=torch.float32, device="cuda")
        us = _graph_time(torch, lambda: [qmm.qmm_matmul_x16(Ws[i % copies], qt, k, X, Y=Y) for i in range(copies)],
                         copies)
        tfl = 2 * rows * k * T / (us * 1e-6) / 1e12
        # the library's choice: the two-group kernel when its 128 x 256 tiles
        # cover at least 2/3 of the CUs (11008 rows), else the one-group kernel
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        pp = 3 * ((rows + 127) // 128) * ((T + 255) // 256) >= 2 * cus
        out[f"{rows}x{k}"] = {"tokens": T, "us_per_launch": round(us, 3), "flops_per_launch": 2 * rows * k * T,
                              "TFLOP_per_s": round(tfl, 2), "kernel": "gemm_pp_kernel" if pp else "gemm_kernel",
                              "roofline": _roof(tfl, MFMA_F16_PEAK_TFLOPS, "TFLOP/s", "mfma")}
        del Ws, W0
    # attn_q, attn_k and attn_v of a layer at the same batch in one
    # qmm_matmul_batch call: 3 x 64 tiles share one two-group launch
    rows = synth.N_EMBD
    W0 = torch.from_numpy(synth.make_weights(qt, rows, k, None, rng)).cuda()
    groups = int(np.ceil(1.1 * 2**30 / (3 * W0.numel())))
    Ws = [W0] + [W0.clone() for _ in range(3 * groups - 1)]
    Xs = [torch.from_numpy(synth.make_activations(T, k, rng, np.float16)).cuda() for _ in range(3)]
    Ys = [torch.empty((T, rows), dtype=torch.float32, device="cuda") for _ in range(3)]
    items = [[(Ws[3 * g + j], qt, k, Xs[j], Ys[j]) for j in range(3)] for g in range(groups)]
    us = _graph_time(torch, lambda: [qmm.qmm_matmul_batch(it) for it in items], groups)
    tfl = 3 * 2 * rows * k * T / (us * 1e-6) / 1e12
    out[f"3x{rows}x{k}_batched"] = {"tokens": T, "us_per_launch": round(us, 3),
                                     "flops_per_launch": 3 * 2 * rows * k * T, "TFLOP_per_s": round(tfl, 2),
                                     "kernel": "gemm_pp_kernel (q|k|v in one qmm_matmul_batch launch)",
                                     "roofline": _roof(tfl, MFMA_F16_PEAK_TFLOPS, "TFLOP/s", "mfma")}
    del Ws, W0, items
    # the stack's down projection at the same batch: 64 tiles over k = 11008,
    # the shape qmm_matmul_ws splits in k (four parts per tile), against the
    # unsplit launch
    rows, k = synth.N_EMBD, synth.N_FF
    W0 = torch.from_numpy(synth.make_weights(qt, rows, k, None, rng)).cuda()
    copies = int(np.ceil(1.1 * 2**30 / W0.numel()))
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    X = torch.from_numpy(synth.make_activations(T, k, rng, np.float16)).cuda()
    Y = torch.empty((T, rows), dtype=torch.float32, device="cuda")
    ws = torch.zeros(qmm.qmm_matmul_workspace_bytes(qt, rows, k, T, qmm.QMM_X_F16), dtype=torch.uint8, device="cuda")
    us = _graph_time(torch, lambda: [qmm.qmm_matmul_ws(Ws[i % copies], qt, k, X, ws, Y=Y) for i in range(copies)],
                     copies)
    us0 = _graph_time(torch, lambda: [qmm.qmm_matmul_x16(Ws[i % copies], qt, k, X, Y=Y) for i in range(copies)],
                      copies)
    tfl = 2 * rows * k * T / (us * 1e-6) / 1e12
    out[f"{rows}x{k}"] = {"tokens": T, "us_per_launch": round(us, 3), "flops_per_launch": 2 * rows * k * T,
                          "TFLOP_per_s": round(tfl, 2), "kernel": "gemm_pp_kernel (k split, qmm_matmul_ws)",
                          "workspace_bytes": ws.numel(), "unsplit_us_per_launch": round(us0, 3),
                          "roofline": _roof(tfl, MFMA_F16_PEAK_TFLOPS, "TFLOP/s", "mfma")}
    del Ws, W0
    return out


# ---------------------------------------------------------------- MUL_MAT_ID

MOE_EXPERTS, MOE_ROWS, MOE_K, MOE_USED = 8, 14336, 4096, 2
MOE_PREFILL_TOKENS = 512
MOE_BATCH_TOKENS = 8


def _graph_time(torch, run, reps):
    """Median over 5 replays of a graph of `reps` launches: microseconds per launch."""
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(5):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / reps)
    return sorted(ts)[2]


def time_matmul_id(torch, qmm, synth, with_oracle=False):
    """MUL_MAT_ID on a routed FFN projection: 8 experts of 14336x4096 Q4_0,
    2 selected per token (seeded random routing), activations shared by the
    slots. Decode (1 token, per-pair decode kernel), batched decode (8
    tokens, routing kernel + decode tiles of 2 pairs) and the probe's
    512-token batch (routing kernel, fp16 copy of the activations, two-group
    matrix-core kernel on 160-pair tiles), each as back-to-back
    launches in a graph over >= 1.1 GiB of expert-stack copies, a different
    routing per launch, so the weights come from HBM."""
    import numpy as np
    E, rows, k, used, qt = MOE_EXPERTS, MOE_ROWS, MOE_K, MOE_USED, synth.TYPE_Q4_0
    nb1 = synth.dense_row_bytes(qt, k)
    rng = np.random.Generator(np.random.PCG64(4343))
    Wh = synth.make_weights(qt, E * rows, k, nb1, rng)
    W0 = torch.from_numpy(Wh).cuda().view(E, rows, nb1)
    copies = int(np.ceil(1.1 * 2**30 / W0.numel()))
    Ws = [W0] + [W0.clone() for _ in range(copies - 1)]
    res = {"workload": f"{E} experts of {rows}x{k} Q4_0, {used} selected per token"}

    def routing(n_tokens):
        return np.stack([rng.permutation(E)[:used] for _ in range(n_tokens)]).astype(np.int32)

    # decode
    reps = 4 * copies
    ids_d = [torch.from_numpy(routing(1)).cuda() for _ in range(reps)]
    Xd = torch.from_numpy(synth.make_activations(1, k, rng)).cuda().view(1, 1, k)
    Yd = torch.empty((1, used, rows), dtype=torch.float32, device="cuda")

    def run_d():
        for i in range(reps):
            qmm.qmm_matmul_id(Ws[i % copies], qt, k, Xd, ids_d[i], Y=Yd)

    us = _graph_time(torch, run_d, reps)
    byts = used * rows * nb1 + 4 * k + 4 * used + 4 * used * rows
    gbs = byts / (us * 1e-6) / 1e9
    res["decode"] = {"tokens": 1, "us_per_launch": round(us, 3), "algorithmic_bytes_per_launch": byts,
                     "GB_per_s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "kernel": "gemv_stream_kernel", "bound": "hbm"}
    # batched decode: a few tokens, their pairs grouped into decode tiles so
    # an expert selected by several tokens is read once
    Tb = MOE_BATCH_TOKENS
    ids_b = [torch.from_numpy(routing(Tb)).cuda() for _ in range(reps)]
    Xb = torch.from_numpy(synth.make_activations(Tb, k, rng)).cuda().view(Tb, 1, k)
    Yb = torch.empty((Tb, used, rows), dtype=torch.float32, device="cuda")
    ws_b = torch.empty(max(1, qmm.qmm_matmul_id_workspace_bytes(E, used, Tb)), dtype=torch.uint8, device="cuda")

    def run_b():
        for i in range(reps):
            qmm.qmm_matmul_id(Ws[i % copies], qt, k, Xb, ids_b[i], Y=Yb, workspace=ws_b)

    us_b = _graph_time(torch, run_b, reps)
    # the distinct experts of each launch's routing are the weights it must read
    distinct = float(np.mean([len(np.unique(i.cpu().numpy())) for i in ids_b]))
    byts_b = int(distinct * rows * nb1) + 4 * Tb * k + 4 * Tb * used + 4 * Tb * used * rows
    gbs_b = byts_b / (us_b * 1e-6) / 1e9
    res["batched_decode"] = {"tokens": Tb, "mean_distinct_experts": distinct, "us_per_launch": round(us_b, 3),
                             "algorithmic_bytes_per_launch": byts_b, "GB_per_s": round(gbs_b, 2),
                             "frac_of_hbm_peak": round(gbs_b / HBM_PEAK_GBS, 4),
                             "kernel": "route_small_kernel + gemv_stream_kernel (tiles)", "bound": "hbm"}
    # prefill-sized batch
    T = MOE_PREFILL_TOKENS
    reps_p = copies
    ids_p = [torch.from_numpy(routing(T)).cuda() for _ in range(reps_p)]
    Xp = torch.from_numpy(synth.make_activations(T, k, rng)).cuda().view(T, 1, k)
    Yp = torch.empty((T, used, rows), dtype=torch.float32, device="cuda")
    ws = torch.empty(qmm.qmm_matmul_id_workspace_bytes_x16(E, used, T, k, 1), dtype=torch.uint8, device="cuda")

    def run_p():
        for i in range(reps_p):
            qmm.qmm_matmul_id(Ws[i % copies], qt, k, Xp, ids_p[i], Y=Yp, workspace=ws)

    us_p = _graph_time(torch, run_p, reps_p)
    flops = 2 * T * used * rows * k
    tfl = flops / (us_p * 1e-6) / 1e12
    res["prefill"] = {"tokens": T, "us_per_launch": round(us_p, 3), "flops_per_launch": flops,
                      "TFLOP_per_s": round(tfl, 2), "frac_of_mfma_f16_peak": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
                      "kernel": "route_small_kernel (+ fp16 copy of X) + gemm_pp_routed_kernel", "bound": "mfma"}
    if with_oracle:
        # the oracle as it stands, once, on the host: the decode call
        import oracle.qmm_oracle as O
        idh = ids_d[0].cpu().numpy()
        t0 = time.perf_counter()
        O.matmul_id(Wh.reshape(E, rows * nb1), qt, E, rows, k, nb1, rows * nb1, Xd.cpu().numpy(), idh)
        res["decode"]["cpu_oracle_us"] = round((time.perf_counter() - t0) * 1e6, 1)
    return res


# ---------------------------------------------------------------- workload

def upload_stack(torch, synth, layers, keep_host_layers):
    """Generate (seeded, on the host) and upload weights and both activation
    sets; keep the host copies of the first layers for the CPU sample."""
    dec = synth.stack_cases(DECODE_TOKENS, layers)
    pre = synth.stack_cases(PREFILL_TOKENS, layers)
    W, X1, X2, host = [], [], [], []
    workers = min(16, os.cpu_count() or 1)

    def gen(i):
        return dec[i].weights(), dec[i].activations(), pre[i].activations()

    with ThreadPoolExecutor(workers) as ex:
        for li in range(layers):
            idx = range(7 * li, 7 * li + 7)
            for i, (w, x1, x2) in zip(idx, ex.map(gen, idx)):
                W.append(torch.from_numpy(w).cuda())
                X1.append(torch.from_numpy(x1).cuda())
                X2.append(torch.from_numpy(x2).cuda())
                if li < keep_host_layers:
                    host.append((dec[i], w, x1))
            if li % 8 == 7:
                log(f"uploaded {li + 1}/{layers} layers")
    torch.cuda.synchronize()
    return dec, pre, W, X1, X2, host


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


def _oracle_legs(O, items, one_thread):
    """Time oracle.matmul over (case, W rows, X) items as it stands; with
    one_thread its BLAS is held to one thread (numpy's dequantisation runs
    on one thread either way). Returns (seconds, algorithmic bytes, flops)."""
    import contextlib
    lim = contextlib.nullcontext()
    if one_thread:
        from threadpoolctl import threadpool_limits
        lim = threadpool_limits(1)
    nbytes = flops = 0
    with lim:
        t0 = time.perf_counter()
        for c, w, x in items:
            rows = w.shape[0]
            O.matmul(w, c.qtype, rows, c.k, c.nb1, x)
            nbytes += rows * (c.w_bytes() // c.rows) + x.nbytes + rows * x.shape[0] * 4
            flops += 2 * rows * c.k * x.shape[0]
        return time.perf_counter() - t0, nbytes, flops


def cpu_baseline(O, host, pre_layer0):
    """The oracle as it stands, timed on the host beside the GPU run.

    value: the decode MUL_MATs of the first stack layers (n_tokens = 1) with
    numpy's BLAS on all its threads, GB/s of algorithmic bytes. Beside it:
    the same on one thread (layer 0 only), and one layer's prefill MUL_MATs
    at n_tokens = 2048 on a stated fraction of each tensor's rows, reported
    as the whole layer's time extrapolated by that fraction (all threads and
    one thread)."""
    threads = _blas_threads()
    dt, nbytes, _ = _oracle_legs(O, host, False)
    layers = len(host) // 7
    dt1, nb1_, _ = _oracle_legs(O, host[:7], True)
    res = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"decode MUL_MATs of layers 0..{layers - 1} of the same stack ({len(host)} matmuls, "
                     f"n_tokens=1, {nbytes / 1e6:.1f} MB algorithmic) in {dt:.2f} s; dequantisation in numpy "
                     f"on one thread, fp64 products on {threads} BLAS threads",
           "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
           "decode_one_thread": {"value": round(nb1_ / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                 "sample": f"decode MUL_MATs of layer 0 (7 matmuls) in {dt1:.2f} s"}}
    if pre_layer0:
        for key, frac, one in (("prefill", 8, False), ("prefill_one_thread", 32, True)):
            items = [(c, w[: c.rows // frac], x) for c, w, x in pre_layer0]
            dtp, _, fl = _oracle_legs(O, items, one)
            full = dtp * frac
            res[key] = {"value": round(fl * frac / full / 1e9, 3), "unit": "GFLOP/s", "cores": 1 if one else threads,
                        "layer_seconds_extrapolated": round(full, 2),
                        "sample": f"prefill MUL_MATs of layer 0 (7 matmuls, n_tokens={PREFILL_TOKENS}) on the "
                                  f"first 1/{frac} of each tensor's rows in {dtp:.2f} s; whole-layer time "
                                  f"extrapolated by {frac}x"}
    return res


def main():
    args = parse()
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): a MUL_MAT shards by weight rows "
              "(or experts) across GPUs without communication, so one GPU's throughput is what is measured",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_quantized_matmul_amd as qmm
    from block_quantized_matmul_amd import synth

    if not os.path.exists(qmm.LIB_PATH):
        raise SystemExit(f"{qmm.LIB_PATH} is missing: build it first (python -m block_quantized_matmul_amd.build)")
    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    layers = args.layers
    cpu_layers = 0 if args.no_cpu_baseline else max(1, min(args.cpu_layers, layers))

    if args.only in ("output_projection", "prefill_512", "matmul_id"):
        # one of the single-matrix workloads alone (for counter runs): its
        # timed graphs, after a plain copy of known size when calibrating
        if args.copy_calibration:
            a = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
            torch.empty_like(a).copy_(a)
            torch.cuda.synchronize()
            del a
        res = {"output_projection": time_output_projection, "prefill_512": time_prefill_512,
               "matmul_id": time_matmul_id}[args.only](torch, qmm, synth)
        log(json.dumps(res))
        return

    log(f"generating and uploading the {layers}-layer stack")
    dec, pre, W, X1, X2, host = upload_stack(torch, synth, layers, cpu_layers)
    if args.copy_calibration:  # a plain device copy of known size, for counter calibration
        a = torch.empty(COPY_CAL_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    n = len(W)
    Y1 = [torch.empty((DECODE_TOKENS, r), dtype=torch.float32, device="cuda") for _, r, _ in synth.LAYER_TENSORS]
    Y1b = [torch.empty_like(y) for y in Y1]
    Y2 = [torch.empty((PREFILL_TOKENS, r), dtype=torch.float32, device="cuda") for _, r, _ in synth.LAYER_TENSORS]
    groups = [[(W[7 * li + j], dec[7 * li + j].qtype, dec[7 * li + j].k, X1[7 * li + j], Y1[j]) for j in grp]
              for li in range(layers) for grp in LAYER_GROUPS]

    def decode_pass():
        for items in groups:
            qmm.qmm_matmul_batch(items)

    def decode_per_call_pass():
        for i in range(n):
            c = dec[i]
            qmm.qmm_matmul(W[i], c.qtype, c.k, X1[i], Y=Y1b[i % 7])

    pgroups = [[(W[7 * li + j], pre[7 * li + j].qtype, pre[7 * li + j].k, X2[7 * li + j], Y2[j]) for j in grp]
               for li in range(layers) for grp in LAYER_GROUPS]
    ws_bytes = max(qmm.qmm_matmul_batch_workspace_bytes(items) for items in pgroups)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")   # zero before first use

    def prefill_pass():
        for items in pgroups:
            qmm.qmm_matmul_batch_ws(items, ws)

    Y2b = [torch.empty_like(y) for y in Y2]

    def prefill_per_call_pass():
        for i in range(n):
            c = pre[i]
            qmm.qmm_matmul_x16(W[i], c.qtype, c.k, X2[i], Y=Y2b[i % 7])

    passes = {"decode": decode_pass, "decode_per_call": decode_per_call_pass, "prefill": prefill_pass,
              "prefill_per_call": prefill_per_call_pass}
    for extra in ("decode_per_call", "prefill_per_call"):
        if not args.per_call and args.only != extra:
            del passes[extra]
    launches = {"decode": len(groups), "decode_per_call": n, "prefill": len(pgroups), "prefill_per_call": n}
    if args.only:
        f = passes[args.only]
        f()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        log(f"ran the {args.only} pass {1 + args.steps} times ({launches[args.only]} launches each)")
        return
    # eager run (reference outputs of the last layer), then capture each pass
    for f in passes.values():
        f()
    torch.cuda.synchronize()
    outs = Y1 + (Y1b if "decode_per_call" in passes else []) + Y2 + (Y2b if "prefill_per_call" in passes else [])
    refs = [y.clone() for y in outs]
    # a batched launch may split k differently from a single call, so the
    # two agree within rounding, not bitwise
    for name, ya, yb in (("decode", Y1, Y1b), ("prefill", Y2, Y2b)):
        if f"{name}_per_call" in passes:
            for a, b in zip(ya, yb):
                if not torch.allclose(a, b, rtol=2e-3, atol=1e-4 * float(b.abs().max())):
                    raise RuntimeError(f"batched and per-call {name} outputs differ beyond rounding")
    graphs = {}
    for name, f in passes.items():
        graphs[name] = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graphs[name]):
            f()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        for g in graphs.values():
            g.replay()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record()
        graphs["decode"].replay()
        ev[s][1].record()
        graphs["prefill"].replay()
        ev[s][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span = {"decode": (0, 1), "prefill": (1, 2)}
    ms = {name: sorted(ev[s][a].elapsed_time(ev[s][b]) for s in range(K))[K // 2] for name, (a, b) in span.items()}
    for extra in ("decode_per_call", "prefill_per_call"):
        if extra in graphs:
            # timed after the steps, outside the step clock
            for s in range(K):
                ev[s][3].record()
                graphs[extra].replay()
                ev[s][4].record()
            torch.cuda.synchronize()
            ms[extra] = sorted(ev[s][3].elapsed_time(ev[s][4]) for s in range(K))[K // 2]

    for a, b in zip(outs, refs):
        if not torch.equal(a, b):
            raise RuntimeError("graph replay output differs from the eager run")

    dec_bytes = sum(c.w_bytes() + c.n_tokens * c.k * 4 + c.n_tokens * c.rows * 4 for c in dec)
    pre_flops = sum(2.0 * c.rows * c.k * c.n_tokens for c in pre)
    gbs = dec_bytes / (ms["decode"] * 1e-3) / 1e9

    tfl = pre_flops / (ms["prefill"] * 1e-3) / 1e12
    us_launch = {k: ms[k] * 1e3 / launches[k] for k in ms}

    def roof(kernel, profile, bound, per_launch, unit, peak, achieved):
        t = traffic_from_profiles(kernel, profile)
        return {"kernel": kernel, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": t,
                "algorithmic_per_launch": per_launch, "avg_launch_us": None}

    r_dec = roof("gemv_stream_kernel", "gemv_stream_kernel__llama7b_q4_0_stack_decode.txt", "hbm",
                 dec_bytes / launches["decode"], "GB/s", HBM_PEAK_GBS,
                 (dec_bytes / launches["decode"]) / (us_launch["decode"] * 1e-6) / 1e9)
    r_dec["avg_launch_us"] = round(us_launch["decode"], 3)
    r_pre = roof("gemm_pp_kernel", "gemm_pp_kernel__llama7b_q4_0_stack_prefill.txt", "mfma",
                 pre_flops / launches["prefill"], "TFLOP/s", MFMA_F16_PEAK_TFLOPS,
                 (pre_flops / launches["prefill"]) / (us_launch["prefill"] * 1e-6) / 1e12)
    r_pre["avg_launch_us"] = round(us_launch["prefill"], 3)

    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": f"{layers}-layer Llama-7B-shaped Q4_0 stack (per layer q,k,v,o 4096x4096; gate,up "
                        f"11008x4096; down 4096x11008): decode n_tokens=1 fp32 x (4 batched launches per layer) "
                        f"+ prefill ubatch n_tokens=2048 fp16 x (4 batched launches per layer, last round "
                        f"of the gate|up launch split in k)",
            "layers": layers,
            "matmuls_per_pass": n,
            "weight_bytes": sum(c.w_bytes() for c in dec),
            "decode_tokens": DECODE_TOKENS,
            "prefill_tokens": PREFILL_TOKENS,
        },
        "decode": {"ms_per_pass": round(ms["decode"], 4), "launches": launches["decode"],
                   "us_per_launch": round(us_launch["decode"], 3), "GB_per_s": round(gbs, 2),
                   "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_pass": dec_bytes},
        "prefill": {"ms_per_pass": round(ms["prefill"], 4), "launches": launches["prefill"],
                    "workspace_bytes": ws_bytes,
                    "us_per_launch": round(us_launch["prefill"], 3), "TFLOP_per_s": round(tfl, 2),
                    "frac_of_mfma_f16_peak": round(tfl / MFMA_F16_PEAK_TFLOPS, 4), "flops_per_pass": pre_flops},
        "roofline": r_dec,
        "roofline_prefill": r_pre,
    }
    if "decode_per_call" in ms:
        gbs_pc = dec_bytes / (ms["decode_per_call"] * 1e-3) / 1e9
        out["decode_per_call"] = {"ms_per_pass": round(ms["decode_per_call"], 4), "launches": n,
                                  "us_per_launch": round(us_launch["decode_per_call"], 3),
                                  "GB_per_s": round(gbs_pc, 2), "frac_of_hbm_peak": round(gbs_pc / HBM_PEAK_GBS, 4)}
    if "prefill_per_call" in ms:
        tfl_pc = pre_flops / (ms["prefill_per_call"] * 1e-3) / 1e12
        out["prefill_per_call"] = {"ms_per_pass": round(ms["prefill_per_call"], 4), "launches": n,
                                   "us_per_launch": round(us_launch["prefill_per_call"], 3),
                                   "TFLOP_per_s": round(tfl_pc, 2),
                                   "frac_of_mfma_f16_peak": round(tfl_pc / MFMA_F16_PEAK_TFLOPS, 4)}
    out["output_projection"] = time_output_projection(torch, qmm, synth)
    out["prefill_512"] = time_prefill_512(torch, qmm, synth)
    if not args.no_get_rows:
        out["get_rows"] = time_get_rows(torch, qmm, synth, with_oracle=bool(cpu_layers))
    if not args.no_matmul_id:
        out["matmul_id"] = time_matmul_id(torch, qmm, synth, with_oracle=bool(cpu_layers))
    if not args.no_other_types:
        for qt in (synth.TYPE_Q8_0, synth.TYPE_Q4_1, synth.TYPE_Q5_0, synth.TYPE_Q5_1, synth.TYPE_Q4_K):
            out[synth.TYPE_NAMES[qt]] = time_type(torch, qmm, synth, qt, with_oracle=bool(cpu_layers))
    if cpu_layers:
        import oracle.qmm_oracle as O
        log("timing the CPU oracle on a sample")
        pre0 = [(c, c.weights(), c.activations()) for c in pre[:7]]
        out["cpu_baseline"] = cpu_baseline(O, host, pre0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
