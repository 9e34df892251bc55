"""Benchmark: block-quantized MUL_MAT over a 32-layer Llama-7B-shaped Q4_0 stack.

One step = the whole hot path over one batch of synthetic input:
  decode  - 224 independent MUL_MATs (7 per layer x 32 layers), 1 token, fp32
            activations, on the decode kernel (3.64 GB of Q4_0 weights, read
            once per pass, far larger than the 256 MB Infinity Cache);
  prefill - the same 224 weights with a 2048-token fp16 ubatch each, on the
            matrix-core kernel.
Each pass is captured once into a HIP graph (the launches are exactly the C
entry points' launches) and replayed; HIP events on the launch stream time
the passes. Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line. `value` is the decode pass's achieved HBM bandwidth
(algorithmic bytes: weight blocks + activations + outputs, per pass / pass
time); the prefill pass's TFLOP/s (2 * rows * k * tokens) is reported beside
it. The CPU oracle is timed on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--layers 32] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
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


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=2, help="layers of the decode pass the oracle times")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def upload_stack(torch, synth, layers):
    """Generate (seeded, host) and upload weights and both activation sets."""
    dec = synth.stack_cases(DECODE_TOKENS, layers)
    pre = synth.stack_cases(PREFILL_TOKENS, layers)
    W, X1, X2 = [], [], []
    workers = min(16, os.cpu_count() or 1)

    def gen(i):
        return dec[i].weights(), dec[i].activations(), pre[i].activations()

    with ThreadPoolExecutor(workers) as ex:
        for li in range(layers):
            idx = range(7 * li, 7 * li + 7)
            for w, x1, x2 in ex.map(gen, idx):
                W.append(torch.from_numpy(w).cuda())
                X1.append(torch.from_numpy(x1).cuda())
                X2.append(torch.from_numpy(x2).cuda())
            if li % 8 == 7:
                log(f"uploaded {li + 1}/{layers} layers")
    torch.cuda.synchronize()
    return dec, pre, W, X1, X2


def cpu_baseline(synth, O, layers_for_sample):
    """Time the oracle (as it stands) on the decode MUL_MATs of the first
    layers of the same stack; report GB/s of algorithmic bytes."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cases = [c for c in synth.stack_cases(DECODE_TOKENS, layers_for_sample)]
    inputs = [(c, c.weights(), c.activations()) for c in cases]
    nbytes = 0
    t0 = time.perf_counter()
    for c, w, x in inputs:
        O.matmul(w, c.qtype, c.rows, c.k, c.nb1, x)
        nbytes += c.w_bytes() + x.nbytes + c.rows * c.n_tokens * 4
    dt = time.perf_counter() - t0
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"decode MUL_MATs of layers 0..{layers_for_sample - 1} ({len(cases)} matmuls, n_tokens=1, "
                      f"{nbytes / 1e6:.1f} MB algorithmic) in {dt:.1f} s; numpy dequant single-threaded, "
                      f"fp64 products on {threads} BLAS threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of this "
              "path is a design, not a build", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import block_quantized_matmul_amd as qmm
    from block_quantized_matmul_amd import synth

    if not os.path.exists(qmm.LIB_PATH):
        from block_quantized_matmul_amd import build as b
        b.build()
    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    layers = args.layers

    log(f"generating and uploading the {layers}-layer stack")
    dec, pre, W, X1, X2 = upload_stack(torch, synth, layers)
    n = len(W)
    Y1 = [torch.empty((DECODE_TOKENS, r), dtype=torch.float32, device="cuda") for _, r, _ in synth.LAYER_TENSORS]
    Y2 = [torch.empty((PREFILL_TOKENS, r), dtype=torch.float32, device="cuda") for _, r, _ in synth.LAYER_TENSORS]

    def decode_pass():
        for i in range(n):
            c = dec[i]
            qmm.qmm_matmul(W[i], c.qtype, c.k, X1[i], Y=Y1[i % 7])

    def prefill_pass():
        for i in range(n):
            c = pre[i]
            qmm.qmm_matmul_x16(W[i], c.qtype, c.k, X2[i], Y=Y2[i % 7])

    # eager reference of the last layer's outputs, then capture both passes
    decode_pass()
    prefill_pass()
    torch.cuda.synchronize()
    ref1 = [y.clone() for y in Y1]
    ref2 = [y.clone() for y in Y2]
    g_dec, g_pre = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dec):
        decode_pass()
    with torch.cuda.graph(g_pre):
        prefill_pass()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        g_dec.replay()
        g_pre.replay()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        ev[s][0].record()
        g_dec.replay()
        ev[s][1].record()
        g_pre.replay()
        ev[s][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = sorted(ev[s][0].elapsed_time(ev[s][1]) for s in range(K))
    pre_ms = sorted(ev[s][1].elapsed_time(ev[s][2]) for s in range(K))
    dec_ms_med = dec_ms[K // 2]
    pre_ms_med = pre_ms[K // 2]

    for a, b in zip(Y1 + Y2, ref1 + ref2):
        if not torch.equal(a, b):
            raise RuntimeError("graph replay output differs from the eager run")

    dec_bytes = sum(c.w_bytes() + c.n_tokens * c.k * 4 + c.n_tokens * c.rows * 4 for c in dec)
    pre_flops = sum(2.0 * c.rows * c.k * c.n_tokens for c in pre)
    gbs = dec_bytes / (dec_ms_med * 1e-3) / 1e9
    tfl = pre_flops / (pre_ms_med * 1e-3) / 1e12
    per_launch_dec_us = dec_ms_med * 1e3 / n
    per_launch_pre_us = pre_ms_med * 1e3 / n

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
            "workload": f"{layers}-layer Llama-7B-shaped Q4_0 stack (q,k,v,o 4096x4096; gate,up 11008x4096; "
                        f"down 4096x11008): decode n_tokens=1 fp32 x + prefill ubatch n_tokens=2048 fp16 x",
            "layers": layers,
            "matmuls_per_pass": n,
            "weight_bytes": sum(c.w_bytes() for c in dec),
            "decode_tokens": DECODE_TOKENS,
            "prefill_tokens": PREFILL_TOKENS,
        },
        "decode": {"ms_per_pass": round(dec_ms_med, 4), "us_per_launch": round(per_launch_dec_us, 3),
                   "GB_per_s": round(gbs, 2), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                   "algorithmic_bytes_per_pass": dec_bytes},
        "prefill": {"ms_per_pass": round(pre_ms_med, 4), "us_per_launch": round(per_launch_pre_us, 3),
                    "TFLOP_per_s": round(tfl, 2), "frac_of_mfma_f16_peak": round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
                    "flops_per_pass": pre_flops},
        "roofline": {"kernel": "gemv_kernel (decode)", "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "roofline_prefill": {"kernel": "gemm_kernel (prefill)", "bound": "mfma", "achieved": round(tfl, 2),
                             "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tfl / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        import oracle.qmm_oracle as O
        log("timing the CPU oracle on a sample")
        out["cpu_baseline"] = cpu_baseline(synth, O, max(1, min(args.cpu_layers, layers)))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
