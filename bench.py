"""Benchmark of the dual-weight GLU projection on one MI355X.

One step is one pass of a 32-layer decode stack: 32 distinct weight sets of
M=1, K=2560, N=9216 (a 4B-class decoder MLP gate/up, 3.02 GB in total, far
beyond the 256 MB Infinity Cache), called back to back in layer order with a
per-layer hidden vector.  Inputs are seeded synthetic data already resident in
HBM when timing starts.  The metric is achieved HBM bandwidth: algorithmic
bytes (both weight matrices once, hidden and output) over time.

Prints ONE JSON line.  Extra modes (written to --extra-json, not stdout):
--workloads times the batched workloads and M=1 at their (K, N).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0


def algorithmic_bytes(M: int, N: int, K: int) -> int:
    """Both weight matrices once, hidden once, output once (bf16)."""
    return 2 * N * K * 2 + M * K * 2 + M * N * 2


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "glu_mlp_gemv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str):
    """HBM bytes per launch from committed counter runs, if taken on the current kernels."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except ValueError:
        return None
    if d.get("source_hash") != source_hash():
        return None
    ent = d.get("kernels", {}).get(kernel_key)
    return None if ent is None else ent.get("bytes_per_launch")


def make_stack(torch, inputs, layers, N, K, seed, dev):
    ws = [inputs.weights(N, K, inputs.stack_layer_seed(seed, l), device=dev) for l in range(layers)]
    hs = inputs.stack_hidden(seed, layers, K).to(dev)
    outs = torch.empty(layers, N, dtype=torch.bfloat16, device=dev)
    return ws, hs, outs


def time_region(torch, fn, steps, warmup, stream):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end)  # ms


def cpu_baseline(torch, ws, hs, layers_sample: int, min_seconds: float):
    """The oracle as it stands, on the host, over the first layers of the same stack."""
    import numpy as np
    import oracle

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    host = [(bits(ws[l][0]), bits(ws[l][1]), bits(hs[l:l + 1])) for l in range(layers_sample)]
    threads = oracle.max_threads()
    calls = 0
    t0 = time.perf_counter()
    while True:
        for wg, wu, h in host:
            oracle.dual_gemv(h, wg, wu, threads=threads)
            calls += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    N, K = host[0][0].shape
    gbs = calls * algorithmic_bytes(1, N, K) / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} oracle calls over layers 0-{layers_sample - 1} of the 32-layer "
                      f"M=1 K={K} N={N} stack, {el:.1f} s wall, {threads} OpenMP threads"}


def capture(torch, fn):
    """A HIP graph of one call of fn (captured on a side stream after a warm-up call)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def bench_workloads(torch, api, inputs, dev, reps=30):
    """Batched workloads and M=1 at the same (K, N), each over a rotation pool of >= 1.4 GB,
    one graph replay per pass over the pool."""
    res = []
    stream = torch.cuda.current_stream()
    for name in ("batch_k4096_n12288", "mfma_k5120_n17408"):
        w = inputs.WORKLOADS[name]
        per = 2 * w.N * w.K * 2
        sets = max(4, -(-1_400_000_000 // per))
        pool = [inputs.weights(w.N, w.K, 100 + i, device=dev, outlier_frac=w.outlier_frac) for i in range(sets)]
        for M in (1,) + w.Ms:
            h = inputs.hidden(M, w.K, 0, row0_scale=w.row0_scale).to(dev)
            out = torch.empty(M, w.N, dtype=torch.bfloat16, device=dev)

            def one_pass():
                for wg, wu in pool:
                    api.dual_gemv(h, wg, wu, out=out)
            g = capture(torch, one_pass)
            ms = time_region(torch, g.replay, reps, 2, stream)
            us = ms * 1e3 / (reps * sets)
            b = algorithmic_bytes(M, w.N, w.K)
            flops = 4 * M * w.N * w.K
            res.append({"workload": name, "M": M, "K": w.K, "N": w.N, "us_per_call": round(us, 3),
                        "GBs": round(b / us / 1e3, 1), "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                        "TFLOPs": round(flops / us / 1e6, 2), "kernel": api.plan(M, w.N, w.K)["kernel_name"],
                        "pool_sets": sets})
            print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
            del g
        del pool
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=5.0)
    ap.add_argument("--workloads", action="store_true", help="also time the batched workloads")
    ap.add_argument("--extra-json", default=None, help="file for the --workloads results")
    ap.add_argument("--tuning", default=None, help="JSON dict of glu_tuning fields (sweeps)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the projection shards along N with no communication: one GPU runs the same kernel on its rows). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from glu_mlp_gemv_amd import api, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = inputs.WORKLOADS["stack32_k2560_n9216"]
    M, N, K, L = 1, w.N, w.K, w.layers
    tuning = api.make_tuning(**json.loads(args.tuning)) if args.tuning else None
    plan = api.plan(M, N, K, True, tuning)

    ws, hs, outs = make_stack(torch, inputs, L, N, K, args.seed, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        for l in range(L):
            api.dual_gemv(hs[l], ws[l][0], ws[l][1], out=outs[l], tuning=tuning)

    # eager: raw C calls on precomputed device addresses (host cost per launch is minimal)
    lib = api.library()
    ptrs = [(hs[l].data_ptr(), ws[l][0].data_ptr(), ws[l][1].data_ptr(), outs[l].data_ptr())
            for l in range(L)]
    sh = stream.cuda_stream

    def step_eager():
        for p in ptrs:
            lib.glu_dual_gemv(p[0], p[1], p[2], p[3], M, N, K, sh)

    ms_eager = time_region(torch, step_eager, args.steps, args.warmup, stream)
    # the decode step as deployed: one graph replay of the 32 launches
    graph = capture(torch, step)
    ms = time_region(torch, graph.replay, args.steps, args.warmup, stream)
    ms_per_step = ms / args.steps
    bytes_call = algorithmic_bytes(M, N, K)
    bytes_step = bytes_call * L
    gbs = bytes_step / (ms_per_step * 1e-3) / 1e9
    launch_us = ms * 1e3 / (args.steps * L * plan["launches"])
    achieved = bytes_call / plan["launches"] / (launch_us * 1e-6) / 1e9

    kernel_key = f"{plan['kernel_name']}_M{M}_K{K}_N{N}"
    traffic = load_traffic(kernel_key)
    line = {
        "metric": "achieved HBM GB/s (and % of peak) for dual GEMV+SiLU·mul, M=1, K=2560, N=9216",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "glu_dual_gemv M=1 K=2560 N=9216, 32-layer decode stack (3.02 GB of "
                               "bf16 gate/up weights), layers called back to back",
                   "M": M, "K": K, "N": N, "layers": L, "bytes_per_call": bytes_call,
                   "us_per_call": round(launch_us * plan["launches"], 3),
                   "timing": "one HIP graph replay per step (32 launches); events on the launch stream",
                   "eager_ms_per_step": round(ms_eager / args.steps, 5),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": plan,
                   "accumulate": "fp32", "tuning": json.loads(args.tuning) if args.tuning else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, ws, hs, layers_sample=4, min_seconds=args.cpu_seconds)
    if args.workloads:
        extra = {"workloads": bench_workloads(torch, api, inputs, dev), "stack": line}
        path = args.extra_json or os.path.join(ROOT, "gpurun_out", "bench_workloads.json")
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            json.dump(extra, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
