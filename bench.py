"""Benchmark of the dual-weight GLU projection on one MI355X.

One step is one pass of a 32-layer decode stack: 32 distinct weight sets of
M=1, K=2560, N=9216 (a 4B-class decoder MLP gate/up, 3.02 GB in total, far
beyond the 256 MB Infinity Cache), called back to back in layer order with a
per-layer hidden vector, captured once as a HIP graph and replayed per step
(a decode step is one graph replay).  Inputs are seeded synthetic data
already resident in HBM when timing starts.  The metric is achieved HBM
bandwidth: algorithmic bytes (both weight matrices once, hidden and output)
over time.

Prints ONE JSON line.  Other modes:
  --workloads FILE     also time the batched workloads (JSON written to FILE);
                       --filter S keeps the sections whose name contains S
  --ceiling FILE       also time the streaming-read yardstick (glu_read_ceiling:
                       the GEMV's loads without its arithmetic) against the
                       GEMV: on the 32-layer stack at several launch shapes,
                       and at 12-357 MB per launch with a fit t = a + bytes/BW
                       (JSON written to FILE)
  --units FILE         also time the unit ceilings (glu_unit_ceiling): matrix-core
                       issue rate of the 16x16x32 and 32x32x16 bf16 MFMA shapes
                       and the LDS read rate, at 4, 8 and 16 waves per CU
  --calibrate-copy     run a 256 MiB device copy first (reference kernel for
                       rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE scaling)
  --summarize KIND DIR turn rocprofv3 output in DIR into the text summaries
                       kept under profiles/ (KIND: trace | trace-grid |
                       counters | counter-table); host only, no GPU
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
CALIBRATION_BYTES = 256 * 1024 * 1024
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
METRIC = "achieved HBM GB/s (and % of peak) for dual GEMV+SiLU·mul, M=1, K=2560, N=9216"
STACK = dict(M=1, K=2560, N=9216, layers=32)


def algorithmic_bytes(M: int, N: int, K: int) -> int:
    """Both weight matrices once, hidden once, output once (bf16)."""
    return 2 * N * K * 2 + M * K * 2 + M * N * 2


# the sources the headline kernel (the VALU GEMV) is compiled from: its template, its per-M
# instantiations and dispatch, and the headers they include
HEADLINE_SOURCES = ("glu_valu", "glu_device.h", "glu_launch.h")


def source_hash() -> str:
    """Hash of the headline kernel's HIP sources: counter figures are valid only for the kernel
    they were taken on."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "glu_mlp_gemv_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.startswith(HEADLINE_SOURCES):
            continue
        h.update(f.encode())
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel_name: str):
    """HBM bytes per launch of a kernel from the committed counter summary, if current."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        d = json.load(open(TRAFFIC_JSON))
    except ValueError:
        return None
    if d.get("source_hash") != source_hash():
        return None
    ent = d.get("kernels", {}).get(kernel_name)
    return None if ent is None else ent.get("bytes_per_launch")


# ---------------------------------------------------------------- timing ----

def capture(torch, fn):
    """A HIP graph of one call of fn, captured on a side stream after a warm-up call."""
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


def warm(torch, fn, seconds):
    """Replays fn, untimed, for at least `seconds`: the first ~10 ms of replays of a freshly
    captured graph run up to 20 % slower than the steady state."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        fn()
        torch.cuda.synchronize()


def time_region(torch, fn, steps, warmup, stream):
    """Milliseconds for `steps` calls of fn, events on the launch stream, synchronised both sides."""
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
    return start.elapsed_time(end)


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(torch, ws, hs, layers_sample: int, min_seconds: float):
    """The oracle as it stands, on the host, over the first layers of the same stack: once with all
    the OpenMP threads it takes by default (the reported value) and once on one thread."""
    import numpy as np
    import oracle

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    host = [(bits(ws[l][0]), bits(ws[l][1]), bits(hs[l:l + 1])) for l in range(layers_sample)]
    N, K = host[0][0].shape

    def timed(threads):
        calls = 0
        t0 = time.perf_counter()
        while True:
            for wg, wu, h in host:
                oracle.dual_gemv(h, wg, wu, threads=threads)
                calls += 1
                if time.perf_counter() - t0 >= min_seconds:
                    break
            el = time.perf_counter() - t0
            if el >= min_seconds:
                return calls, el

    threads = oracle.max_threads()
    calls, el = timed(threads)
    calls1, el1 = timed(1)
    per = algorithmic_bytes(1, N, K)
    return {"value": round(calls * per / el / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "single_thread_value": round(calls1 * per / el1 / 1e9, 3),
            "cpu_model": host_cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{calls} oracle calls ({threads} OpenMP threads, {el:.1f} s wall) and {calls1} calls "
                      f"(1 thread, {el1:.1f} s) over layers 0-{layers_sample - 1} of the 32-layer "
                      f"M=1 K={K} N={N} stack; seconds per call {el / calls:.4f} and {el1 / calls1:.4f}"}


BATCHED_ROUNDS = 6  # interleaved timing rounds of the batched workloads
BATCHED_WARM_SECONDS = 0.5  # untimed replays first: the first ~10 ms after capture run up to 20 % slower
WORKLOAD_WARM_SECONDS = 0.2  # the same for each graph of the other workloads


def bench_workloads(torch, api, inputs, dev, reps=30, only=None):
    """Batched workloads and M=1 at the same (K, N), each over a rotation pool of >= 1.4 GB,
    one graph replay per pass over the pool.  ``only``: run the sections whose name contains it
    (batched, prefill, backward, rows, grouped)."""
    res = []
    stream = torch.cuda.current_stream()

    def want(section):
        return only is None or only in section
    for name in (("batch_k4096_n12288", "mfma_k5120_n17408") if want("batched") else ()):
        w = inputs.WORKLOADS[name]
        per = 2 * w.N * w.K * 2
        sets = max(4, -(-1_400_000_000 // per))
        pool = [inputs.weights(w.N, w.K, 100 + i, device=dev, outlier_frac=w.outlier_frac) for i in range(sets)]
        # every M's graph is built first, then timed in interleaved rounds (median per M), so that
        # the ratios to M = 1 do not depend on the order or on the clock drifting during the run
        # (M, tuning, label): the planner's default for every M, and where hidden is staged in K-slices
        # above 8 rows also the 8-row kernel's block-by-block K walk, for comparison
        cases = [(M, None, "default") for M in (1,) + w.Ms]
        cases += [(M, api.make_tuning(rows_per_wave=8, mfma_order=1), "block_by_block") for M in w.Ms
                  if M > 8 and M * w.K * 2 > 65536]
        graphs = []
        for M, t, _ in cases:
            h = inputs.hidden(M, w.K, 0, row0_scale=w.row0_scale).to(dev)
            out = torch.empty(M, w.N, dtype=torch.bfloat16, device=dev)

            def one_pass(h=h, out=out, t=t):
                for wg, wu in pool:
                    api.dual_gemv(h, wg, wu, out=out, tuning=t)
            graphs.append((capture(torch, one_pass), h, out))
        per_round = max(1, reps // BATCHED_ROUNDS)
        times = [[] for _ in cases]
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < BATCHED_WARM_SECONDS:  # untimed, interleaved as below
            for g, _, _ in graphs:
                g.replay()
            torch.cuda.synchronize()
        for _ in range(BATCHED_ROUNDS):
            for i, (g, _, _) in enumerate(graphs):
                times[i].append(time_region(torch, g.replay, per_round, 1, stream) * 1e3 / (per_round * sets))
        for (M, t, label), ts in zip(cases, times):
            us = statistics.median(ts)
            b = algorithmic_bytes(M, w.N, w.K)
            flops = 4 * M * w.N * w.K
            res.append({"workload": name, "M": M, "K": w.K, "N": w.N, "us_per_call": round(us, 3),
                        "us_rounds": [round(t, 2) for t in ts],
                        "GBs": round(b / us / 1e3, 1), "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                        "TFLOPs": round(flops / us / 1e6, 2),
                        "mfma_frac": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 5),
                        "kernel": api.plan(M, w.N, w.K, True, t)["kernel_symbol"], "variant": label,
                        "pool_sets": sets})
            print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
        del graphs
        del pool
        torch.cuda.empty_cache()
    # large batches (prefill-like): the default plan (the slice-major 8-row MFMA kernel in launches of
    # 64 rows up to M = 64, the tiled GEMM above) and the alternatives beside it
    for (K, N), Ms in ((((5120, 17408), (48, 64, 128, 256, 512, 1024)), ((2560, 9216), (48, 64, 256, 1024)))
                       if want("prefill") else ()):
        per = 2 * N * K * 2
        sets = max(4, -(-1_400_000_000 // per))
        pool = [inputs.weights(N, K, 500 + i, device=dev) for i in range(sets)]
        for M in Ms:
            h = inputs.hidden(M, K, 0).to(dev)
            out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            variants = [("default", None)]
            if M <= 64:
                variants.append(("gemm", api.make_tuning(kernel=api.KERNEL_GEMM)))
                variants.append(("mfma_32_row_launches", api.make_tuning(kernel=api.KERNEL_MFMA, rows_per_wave=8,
                                                                         mfma_order=2)))
            elif M <= 256:
                variants.append(("mfma_64_row_launches", api.make_tuning(kernel=api.KERNEL_MFMA)))
            for kname, t in variants:
                def one_pass():
                    for wg, wu in pool:
                        api.dual_gemv(h, wg, wu, out=out, tuning=t)
                g = capture(torch, one_pass)
                r = max(3, reps // max(1, M // 64))
                warm(torch, g.replay, WORKLOAD_WARM_SECONDS)
                ms = time_region(torch, g.replay, r, 1, stream)
                us = ms * 1e3 / (r * sets)
                b = algorithmic_bytes(M, N, K)
                flops = 4 * M * N * K
                res.append({"workload": f"prefill_k{K}_n{N}", "M": M, "K": K, "N": N, "us_per_call": round(us, 3),
                            "GBs": round(b / us / 1e3, 1), "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                            "TFLOPs": round(flops / us / 1e6, 2),
                            "mfma_frac": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                            "kernel": api.plan(M, N, K, True, t)["kernel_symbol"], "variant": kname,
                            "pool_sets": sets})
                print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
                del g
            # yardstick, not this library's path: the two products alone on the platform's GEMM
            # library (torch.mm, G and U written in bf16, no epilogue) on the same pools, replayed
            # from a graph like the rows above (eager if the library refuses the capture)
            gy = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            uy = torch.empty_like(gy)

            def lib_pass():
                for wg, wu in pool:
                    torch.mm(h, wg.t(), out=gy)
                    torch.mm(h, wu.t(), out=uy)
            try:
                lib_run, launch = capture(torch, lib_pass).replay, "graph"
            except RuntimeError:
                torch.cuda.synchronize()
                lib_run, launch = lib_pass, "eager"
            r = max(3, reps // max(1, M // 64))
            warm(torch, lib_run, WORKLOAD_WARM_SECONDS)
            us = time_region(torch, lib_run, r, 1, stream) * 1e3 / (r * sets)
            flops = 4 * M * N * K
            res.append({"workload": f"prefill_k{K}_n{N}", "M": M, "K": K, "N": N, "us_per_call": round(us, 3),
                        "TFLOPs": round(flops / us / 1e6, 2),
                        "mfma_frac": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                        "kernel": "torch.mm x2 (library GEMM, no epilogue)", "variant": "library_gemm_yardstick",
                        "launch": launch, "pool_sets": sets})
            print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
            del gy, uy, lib_run
        del pool
        torch.cuda.empty_cache()
    # backward: gradients of hidden and both weights (reads Wg, Wu once more, writes dWg, dWu)
    for (K, N), Ms in ((((2560, 9216), (1, 4, 16, 64, 512)), ((4096, 12288), (1, 2, 8))) if want("backward") else ()):
        per = 4 * N * K * 2  # weights and their gradients per set
        sets = max(4, -(-1_400_000_000 // per))
        pool = [(*inputs.weights(N, K, 600 + i, device=dev),
                 torch.empty(N, K, dtype=torch.bfloat16, device=dev),
                 torch.empty(N, K, dtype=torch.bfloat16, device=dev)) for i in range(sets)]
        # yardstick for this read/write mix: device copies of both weights into the gradient buffers
        # (every byte the backward must move at M = 1, read once and written once)

        def copy_pass():
            for wg, wu, dwg, dwu in pool:
                dwg.copy_(wg)
                dwu.copy_(wu)
        g = capture(torch, copy_pass)
        warm(torch, g.replay, WORKLOAD_WARM_SECONDS)
        ms = time_region(torch, g.replay, reps, 2, stream)
        us = ms * 1e3 / (reps * sets)
        b = 8 * N * K
        res.append({"workload": f"backward_k{K}_n{N}", "M": 0, "K": K, "N": N, "us_per_call": round(us, 3),
                    "GBs": round(b / us / 1e3, 1), "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                    "kernel": "device copy of Wg and Wu (torch copy_)", "pool_sets": sets})
        print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
        del g
        # the same copy streamed like the GEMV reads, with nontemporal stores (glu_copy_ceiling)

        def stream_pass():
            for wg, wu, dwg, dwu in pool:
                api.copy_ceiling(wg, wu, dwg, dwu)
        g = capture(torch, stream_pass)
        warm(torch, g.replay, WORKLOAD_WARM_SECONDS)
        ms = time_region(torch, g.replay, reps, 2, stream)
        us = ms * 1e3 / (reps * sets)
        res.append({"workload": f"backward_k{K}_n{N}", "M": 0, "K": K, "N": N, "us_per_call": round(us, 3),
                    "GBs": round(b / us / 1e3, 1), "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                    "kernel": "streaming copy of Wg and Wu (glu_copy_ceiling: the read/write yardstick)",
                    "pool_sets": sets})
        print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
        del g
        for M in Ms:
            h = inputs.hidden(M, K, 0).to(dev)
            go = inputs.grad_out(M, N, 0).to(dev)
            dh = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
            ws = torch.empty(api.backward_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)

            def one_pass():
                for wg, wu, dwg, dwu in pool:
                    api.dual_gemv_backward(h, wg, wu, go, dh, dwg, dwu, workspace=ws)
            g = capture(torch, one_pass)
            warm(torch, g.replay, WORKLOAD_WARM_SECONDS)
            ms = time_region(torch, g.replay, reps, 2, stream)
            us = ms * 1e3 / (reps * sets)
            b = 8 * N * K + 4 * M * K + 2 * M * N
            flops = 12 * M * N * K  # G and U again, dh, and both weight gradients
            res.append({"workload": f"backward_k{K}_n{N}", "M": M, "K": K, "N": N, "us_per_call": round(us, 3),
                        "GBs": round(b / us / 1e3, 1), "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                        "TFLOPs": round(flops / us / 1e6, 2),
                        "mfma_frac": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 5),
                        "kernel": "backward", "pool_sets": sets})
            print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
            del g
        del pool
        torch.cuda.empty_cache()
    # row-strided operands: gate and up as the two column halves of one fused
    if want("rows"):
        # [N, 2K] block (each keeps the fused row stride 2K), at the decode shape
        N, K = STACK["N"], STACK["K"]
        sets = max(4, -(-1_400_000_000 // (2 * N * K * 2)))
        fused = [torch.cat(inputs.weights(N, K, 300 + i, device=dev), dim=1) for i in range(sets)]
        for layout in ("packed", "fused"):
            # the same weights, as two packed copies or as the two halves of the fused block
            ops = ([(f[:, :K].contiguous(), f[:, K:].contiguous()) for f in fused] if layout == "packed"
                   else [(f[:, :K], f[:, K:]) for f in fused])
            for M in (1, 4):
                h = inputs.hidden(M, K, 0).to(dev)
                out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)

                def one_pass():
                    for wg, wu in ops:
                        api.dual_gemv(h, wg, wu, out=out)
                g = capture(torch, one_pass)
                warm(torch, g.replay, WORKLOAD_WARM_SECONDS)
                ms = time_region(torch, g.replay, reps, 2, stream)
                us = ms * 1e3 / (reps * sets)
                b = algorithmic_bytes(M, N, K)
                res.append({"workload": f"rows_{layout}_k2560_n9216", "M": M, "K": K, "N": N,
                            "us_per_call": round(us, 3), "GBs": round(b / us / 1e3, 1),
                            "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4), "row_stride": ops[0][0].stride(0),
                            "kernel": api.plan(M, N, K)["kernel_name"], "pool_sets": sets})
                print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
                del g
            del ops
        del fused
        torch.cuda.empty_cache()
    # grouped GEMV: n projections of one hidden, weights read in place
    for name, Ns in ((("grouped_qkv_like_k2560", (4096, 1024, 1024)), ("grouped_gdn_like_k2560", (8192, 4096, 32, 32)))
                     if want("grouped") else ()):
        K = STACK["K"]
        rows = sum(Ns)
        per = rows * K * 2
        sets = max(4, -(-1_400_000_000 // per))
        pool = [[inputs.weights(n_i, K, 400 + 10 * i + t, device=dev)[0] for t, n_i in enumerate(Ns)]
                for i in range(sets)]
        # (M, tuning, label): the planner's default, and above 8 rows the same call with hidden read
        # from L2 per stage instead of staged whole into every workgroup's LDS first
        cases = [(M, None, "default") for M in (1, 4, 16, 32, 48, 64)]
        # 33..64 rows in one launch: stages of 4 segments (64 KiB ring) against the default 8 (128 KiB)
        cases += [(M, api.make_tuning(mfma_hidden=3, mfma_segments=4), "k_slices_stages_of_4") for M in (48, 64)]
        cases += [(M, api.make_tuning(mfma_hidden=2), "hidden_from_l2") for M in (16, 32)]
        # and with K-slices of hidden streamed under the weights, one, two or three blocks of 4 groups
        # of 8 rows per workgroup
        blocks = -(-rows // 32)
        cases += [(M, api.make_tuning(mfma_hidden=3, grid=-(-blocks // jb)), f"k_slices_{jb}")
                  for M in (16, 32) for jb in (1, 2, 3)]
        for M, t, label in cases:
            h = inputs.hidden(M, K, 0).to(dev)
            outs = [torch.empty(M, n_i, dtype=torch.bfloat16, device=dev) for n_i in Ns]

            def one_pass():
                for ws in pool:
                    api.grouped_gemv(h, ws, outs=outs, tuning=t)
            g = capture(torch, one_pass)
            warm(torch, g.replay, WORKLOAD_WARM_SECONDS)
            ms = time_region(torch, g.replay, reps, 2, stream)
            us = ms * 1e3 / (reps * sets)
            b = per + M * K * 2 + M * rows * 2
            res.append({"workload": name, "M": M, "K": K, "N": list(Ns), "us_per_call": round(us, 3),
                        "GBs": round(b / us / 1e3, 1), "hbm_frac": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                        "kernel": api.grouped_plan(M, K, rows, tuning=t, mult8=all(n_i % 8 == 0 for n_i in Ns))["kernel_symbol"],
                        "variant": label,
                        "pool_sets": sets})
            print(f"[workloads] {res[-1]}", file=sys.stderr, flush=True)
            del g
        del pool
        torch.cuda.empty_cache()
    return res


PREWARM_SECONDS = 0.5     # untimed replays of the headline graph before its timed trials
TRIALS = 5                # timed trials of the headline (Olympic average reported)


def olympic(xs):
    """Mean without the smallest and the largest value (of 3 or more)."""
    s = sorted(xs)
    return sum(s[1:-1]) / (len(s) - 2) if len(s) >= 3 else sum(s) / len(s)


CEILING_ROUNDS = 5        # interleaved timing rounds of the yardstick comparisons (median reported)
CEILING_ROWS = (1200, 2400, 4608, 9216, 18432, 34880)  # rows of K = 2560: 12-357 MB per launch
CEILING_SHAPES = (        # (kernel, label, tuning fields) timed on the 32-layer stack
    ("gemv", "default", {}),
    ("ceiling", "default", {}),
    ("ceiling", "xcd_bands", {"xcd_bands": 1}),
    ("ceiling", "rows2", {"rows_per_wave": 2}),
    ("ceiling", "grid256x4", {"grid": 256, "waves_per_block": 4}),
    ("ceiling", "grid512x2", {"grid": 512, "waves_per_block": 2}),
    ("ceiling", "rows2_grid256x4", {"rows_per_wave": 2, "grid": 256, "waves_per_block": 4}),
    ("ceiling", "rows2_grid128x4", {"rows_per_wave": 2, "grid": 128, "waves_per_block": 4}),
    ("gemv", "rows2", {"rows_per_wave": 2}),
    ("gemv", "rows2_grid256x4", {"rows_per_wave": 2, "grid": 256, "waves_per_block": 4}),
    ("gemv", "rows2_grid128x4", {"rows_per_wave": 2, "grid": 128, "waves_per_block": 4}),
    ("gemv", "rows2_grid512x2", {"rows_per_wave": 2, "grid": 512, "waves_per_block": 2}),
    ("gemv", "grid256x4", {"grid": 256, "waves_per_block": 4}),
)


def interleaved(torch, graphs, reps, stream, rounds=CEILING_ROUNDS):
    """Median microseconds per replay of each graph, timed in interleaved rounds after 0.3 s of
    untimed interleaved replays."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
    times = [[] for _ in graphs]
    for _ in range(rounds):
        for i, g in enumerate(graphs):
            times[i].append(time_region(torch, g.replay, reps, 1, stream) * 1e3 / reps)
    return [statistics.median(t) for t in times], times


def fit_latency_bandwidth(points):
    """Least-squares t = a + bytes / BW over (bytes, us) points: (a in us, BW in GB/s)."""
    n = len(points)
    xs = [b / 1e6 for b, _ in points]  # MB
    ys = [t for _, t in points]
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    slope = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx  # us per MB
    a = my - slope * mx
    return a, 1e3 / slope


def bench_ceiling(torch, api, inputs, dev, ws, hs, reps=20, shapes=CEILING_SHAPES, sizes=True):
    """The streaming-read yardstick against the GEMV: (1) the 32-layer stack at several launch shapes
    of the yardstick, (2) both kernels at 12-357 MB per launch, fitted to t = a + bytes/BW."""
    stream = torch.cuda.current_stream()
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    L = len(ws)
    N, K = ws[0][0].shape
    out = {"stack": [], "sizes": []}
    outs = torch.empty(L, N, dtype=torch.bfloat16, device=dev)
    graphs, labels = [], []
    for kind, label, fields in shapes:
        t = api.make_tuning(**fields) if fields else None
        if kind == "gemv":
            def stack(t=t):
                for l in range(L):
                    api.dual_gemv(hs[l], ws[l][0], ws[l][1], out=outs[l], tuning=t)
            plan = api.plan(1, N, K, True, t)
        else:
            def stack(t=t):
                for l in range(L):
                    api.read_ceiling(ws[l][0], ws[l][1], sink, tuning=t)
            plan = api.read_ceiling_plan(N, 2 * K, t)
        graphs.append(capture(torch, stack))
        labels.append((kind, label, fields, plan))
    med, rounds = interleaved(torch, graphs, reps, stream)
    b = algorithmic_bytes(1, N, K)
    for (kind, label, fields, plan), us, ts in zip(labels, med, rounds):
        per = us / L
        out["stack"].append({"kernel": kind, "shape": label, "tuning": fields,
                             "grid": plan["grid"], "block": plan["block"], "us_per_launch": round(per, 3),
                             "GBs": round(b / per / 1e3, 1), "hbm_frac": round(b / per / 1e3 / HBM_PEAK_GBS, 4),
                             "rounds_us_per_launch": [round(x / L, 3) for x in ts]})
        print(f"[ceiling] {out['stack'][-1]}", file=sys.stderr, flush=True)
    del graphs
    torch.cuda.synchronize()
    for rows in (CEILING_ROWS if sizes else ()):
        per_set = 2 * rows * K * 2
        sets = max(4, -(-1_400_000_000 // per_set))
        pool = [inputs.weights(rows, K, 700 + i, device=dev) for i in range(sets)]
        h = inputs.hidden(1, K, 0).to(dev)
        o = torch.empty(1, rows, dtype=torch.bfloat16, device=dev)

        def gemv_pool():
            for wg, wu in pool:
                api.dual_gemv(h, wg, wu, out=o)

        def ceil_pool():
            for wg, wu in pool:
                api.read_ceiling(wg, wu, sink)
        gs = [capture(torch, gemv_pool), capture(torch, ceil_pool)]
        med, _ = interleaved(torch, gs, max(2, reps // 4), stream)
        b = algorithmic_bytes(1, rows, K)
        ent = {"rows": rows, "K": K, "bytes_per_launch": b, "pool_sets": sets,
               "gemv_us": round(med[0] / sets, 3), "ceiling_us": round(med[1] / sets, 3),
               "gemv_grid": api.plan(1, rows, K)["grid"], "ceiling_grid": api.read_ceiling_plan(rows, 2 * K)["grid"]}
        ent["gemv_GBs"] = round(b / ent["gemv_us"] / 1e3, 1)
        ent["ceiling_GBs"] = round(b / ent["ceiling_us"] / 1e3, 1)
        out["sizes"].append(ent)
        print(f"[ceiling] {ent}", file=sys.stderr, flush=True)
        del gs, pool
        torch.cuda.empty_cache()
    for kind in (("gemv", "ceiling") if sizes else ()):
        a, bw = fit_latency_bandwidth([(e["bytes_per_launch"], e[kind + "_us"]) for e in out["sizes"]])
        out[kind + "_fit"] = {"a_us": round(a, 3), "BW_GBs": round(bw, 1),
                              "at_94MB_frac": round(b94 / (a + b94 / bw / 1e3) / 1e3 / HBM_PEAK_GBS, 4)
                              if (b94 := algorithmic_bytes(1, N, K)) else None}
    return out


UNIT_NAMES = {1: "mfma_16x16x32_bf16", 2: "mfma_32x32x16_bf16", 3: "lds_read_b128"}
UNIT_WAVES = (4, 8, 16)  # waves per compute unit: 1, 2 and 4 per SIMD
CLOCK_GHZ = 2.4          # MI355X peak engine clock, published


def bench_units(torch, api, dev, reps=3):
    """The unit ceilings: matrix-core issue rate of the two bf16 MFMA shapes and LDS read rate, one
    workgroup per compute unit, a launch of ~0.2-1 s of work per point, median of `reps` launches."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.zeros(64, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    out = []
    for unit in (1, 2, 3):
        for waves in UNIT_WAVES:
            iters = 20000 if unit != 3 else 4000
            api.unit_ceiling(unit, waves, cus, 100, sink)  # warm
            ts = sorted(time_region(torch, lambda: api.unit_ceiling(unit, waves, cus, iters, sink), 1, 0, stream)
                        for _ in range(reps))
            ms = ts[len(ts) // 2]
            work = api.unit_ceiling_work(unit, waves, cus, iters)
            ent = {"unit": UNIT_NAMES[unit], "waves_per_cu": waves, "cus": cus, "iterations": iters,
                   "ms": round(ms, 4)}
            if unit == 3:
                ent["bytes_per_clk_per_cu"] = round(work / (ms * 1e-3) / (CLOCK_GHZ * 1e9) / cus, 1)
            else:
                ent["tflops"] = round(work / (ms * 1e-3) / 1e12, 1)
                ent["frac_of_bf16_peak"] = round(ent["tflops"] / MFMA_BF16_PEAK_TFLOPS, 4)
            out.append(ent)
            print(f"[units] {ent}", file=sys.stderr, flush=True)
    return out


def run(args):
    import torch
    from glu_mlp_gemv_amd import api, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        a = torch.ones(CALIBRATION_BYTES // 2, dtype=torch.bfloat16, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    M, N, K, L = STACK["M"], STACK["N"], STACK["K"], STACK["layers"]
    tuning = api.make_tuning(**json.loads(args.tuning)) if args.tuning else None
    plan = api.plan(M, N, K, True, tuning)

    ws = [inputs.weights(N, K, inputs.stack_layer_seed(args.seed, l), device=dev) for l in range(L)]
    hs = inputs.stack_hidden(args.seed, L, K).to(dev)
    outs = torch.empty(L, N, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def step():
        for l in range(L):
            api.dual_gemv(hs[l], ws[l][0], ws[l][1], out=outs[l], tuning=tuning)

    graph = capture(torch, step)
    # the first ~10 ms of replays of a fresh graph run slower: replay it untimed for PREWARM_SECONDS
    # first (reported), then time TRIALS regions of exactly `steps` replays, each after `warmup`
    # untimed ones, and take the Olympic average (drop the fastest and the slowest, mean of the rest)
    warm(torch, graph.replay, args.prewarm)
    trials = [time_region(torch, graph.replay, args.steps, args.warmup, stream) for _ in range(TRIALS)]
    ms = olympic(trials)
    ms_per_step = ms / args.steps
    bytes_call = algorithmic_bytes(M, N, K)
    gbs = bytes_call * L / (ms_per_step * 1e-3) / 1e9
    launches = args.steps * L * plan["launches"]
    launch_us = ms * 1e3 / launches
    achieved = bytes_call / plan["launches"] / (launch_us * 1e-6) / 1e9

    # the same step launched eagerly, one C call per layer on precomputed addresses
    ms_eager = None
    if tuning is None:
        lib = api.library()
        ptrs = [(hs[l].data_ptr(), ws[l][0].data_ptr(), ws[l][1].data_ptr(), outs[l].data_ptr())
                for l in range(L)]
        sh = stream.cuda_stream

        def step_eager():
            for p in ptrs:
                lib.glu_dual_gemv(p[0], p[1], p[2], p[3], M, N, K, sh)
        ms_eager = time_region(torch, step_eager, args.steps, args.warmup, stream)

    kernel = plan["kernel_symbol"]
    line = {
        "metric": METRIC,
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
        "config": {"workload": "glu_dual_gemv M=1 K=2560 N=9216, 32-layer decode stack (3.02 GB of bf16 "
                               "gate/up weights), one HIP graph replay of the 32 launches per step",
                   "M": M, "K": K, "N": N, "layers": L, "bytes_per_call": bytes_call,
                   "us_per_call": round(launch_us * plan["launches"], 3),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                   "timing": {"prewarm_s": args.prewarm, "trials": TRIALS, "average": "olympic",
                              "trial_ms_per_step": [round(t / args.steps, 5) for t in trials],
                              "median_ms_per_step": round(statistics.median(trials) / args.steps, 5),
                              "min_ms_per_step": round(min(trials) / args.steps, 5)},
                   "eager_ms_per_step": None if ms_eager is None else round(ms_eager / args.steps, 5),
                   "kernel": kernel, "plan": plan, "accumulate": "fp32",
                   "tuning": json.loads(args.tuning) if args.tuning else None},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(kernel)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, ws, hs, layers_sample=4, min_seconds=args.cpu_seconds)
    if args.ceiling:
        shapes = [tuple(s) for s in json.loads(args.shapes)] if args.shapes else CEILING_SHAPES
        res = bench_ceiling(torch, api, inputs, dev, ws, hs, shapes=shapes, sizes=not args.no_sizes)
        os.makedirs(os.path.dirname(os.path.abspath(args.ceiling)), exist_ok=True)
        with open(args.ceiling, "w") as f:
            json.dump(res, f, indent=1)
    if args.units:
        res = bench_units(torch, api, dev)
        os.makedirs(os.path.dirname(os.path.abspath(args.units)), exist_ok=True)
        with open(args.units, "w") as f:
            json.dump(res, f, indent=1)
    if args.workloads:
        extra = {"workloads": bench_workloads(torch, api, inputs, dev, only=args.filter), "stack": line}
        os.makedirs(os.path.dirname(os.path.abspath(args.workloads)), exist_ok=True)
        with open(args.workloads, "w") as f:
            json.dump(extra, f, indent=1)
    print(json.dumps(line), flush=True)


# ------------------------------------------------------- profile summaries ----

def _rows(pattern):
    out = []
    for p in sorted(glob.glob(pattern, recursive=True)):
        with open(p) as f:
            out.extend(csv.DictReader(f))
    return out


def summarize_trace(d: str):
    """Kernel-trace statistics (rocprofv3 --kernel-trace --stats -f csv) as a markdown table."""
    stats = _rows(os.path.join(d, "**", "*kernel_stats.csv"))
    if not stats:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    lines = ["| kernel | calls | total ns | average ns | min ns | max ns | % |",
             "|---|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:100]}` | {r['Calls']} | {r['TotalDurationNs']} | "
                     f"{float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | {float(r['Percentage']):.2f} |")
    return "\n".join(lines)


def short_kernel_name(name: str) -> str:
    """A demangled kernel name without its argument list, return type or anonymous namespace (which
    would otherwise cut the name at its first parenthesis)."""
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()


def summarize_trace_grid(d: str):
    """Per-dispatch kernel trace grouped by (kernel, grid size): a kernel run at several shapes gets
    one row per shape (the grid tells them apart), average and median duration."""
    rows = _rows(os.path.join(d, "**", "*kernel_trace.csv"))
    if not rows:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    groups = {}
    for r in rows:
        name = r["Kernel_Name"]
        if not name.startswith(("glu::", "void glu::")):
            continue
        key = (short_kernel_name(name), int(r["Grid_Size_X"]), int(r["LDS_Block_Size"]))
        groups.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines = ["| kernel | grid (threads) | LDS bytes | dispatches | average ns | median ns | min ns |",
             "|---|---|---|---|---|---|---|"]
    for (name, grid, lds), ts in sorted(groups.items()):
        ts.sort()
        lines.append(f"| `{name}` | {grid} | {lds} | {len(ts)} | {sum(ts) / len(ts):.0f} | {ts[len(ts) // 2]} | {ts[0]} |")
    return "\n".join(lines)


def summarize_counter_table(d: str):
    """Mean of each collected counter per (kernel, grid) from rocprofv3 --pmc csv output."""
    rows = _rows(os.path.join(d, "**", "*counter_collection.csv"))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name", "")
        if not name.startswith(("glu::", "void glu::")):
            continue
        key = (short_kernel_name(name), int(r.get("Grid_Size", r.get("Grid_Size_X", 0)) or 0), r["Counter_Name"])
        # a dispatch may report several rows of one counter (per dimension): sum them per dispatch
        disp = (r.get("Dispatch_Id") or r.get("Correlation_Id"))
        acc.setdefault(key, {}).setdefault(disp, 0.0)
        acc[key][disp] += float(r["Counter_Value"])
    lines = ["| kernel | grid (threads) | counter | dispatches | mean per dispatch |", "|---|---|---|---|---|"]
    for (name, grid, cname), per in sorted(acc.items()):
        vals = list(per.values())
        lines.append(f"| `{name}` | {grid} | {cname} | {len(vals)} | {sum(vals) / len(vals):.2f} |")
    return "\n".join(lines)


def summarize_counters(d: str, command: str):
    """FETCH_SIZE / WRITE_SIZE per dispatch, scaled by the calibration copy of known size.

    ``d`` is one directory or several separated by commas (one counter per run)."""
    rows = []
    for one in d.split(","):
        rows.extend(_rows(os.path.join(one, "**", "*counter_collection.csv")))
    if not rows:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    per = {}
    for r in rows:
        per.setdefault((r["Kernel_Name"], r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    cal_kib = CALIBRATION_BYTES / 1024
    scale = {}
    for cname in ("FETCH_SIZE", "WRITE_SIZE"):
        cal = [v for (k, c), vs in per.items() if c == cname and "copyBuffer" in k for v in vs
               if v > 0.25 * cal_kib]
        if cal:
            scale[cname] = cal_kib / max(cal)
    kernels = {}
    for (k, c), vs in per.items():
        if "glu::" not in k:
            continue
        short = short_kernel_name(k)
        ent = kernels.setdefault(short, {})
        ent[c + "_kib_per_dispatch"] = round(sum(vs) / len(vs), 2)
        ent["dispatches"] = len(vs)
    for ent in kernels.values():
        have = [c for c in ("FETCH_SIZE", "WRITE_SIZE") if c + "_kib_per_dispatch" in ent and c in scale]
        ent["bytes_per_launch"] = (round(sum(ent[c + "_kib_per_dispatch"] * scale[c] * 1024 for c in have))
                                   if len(have) == 2 else None)
    return {"source_hash": source_hash(), "calibration": {"copy_bytes": CALIBRATION_BYTES, "scale": scale},
            "command": command, "kernels": kernels}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=5.0)
    ap.add_argument("--prewarm", type=float, default=PREWARM_SECONDS,
                    help="seconds of untimed replays of the headline graph before its timed trials")
    ap.add_argument("--workloads", default=None, metavar="FILE", help="also time the batched workloads")
    ap.add_argument("--filter", default=None, help="with --workloads: only the sections whose name contains this "
                                                   "(batched, prefill, backward, rows, grouped)")
    ap.add_argument("--tuning", default=None, help="JSON dict of glu_tuning fields")
    ap.add_argument("--ceiling", default=None, metavar="FILE",
                    help="also time the streaming-read yardstick against the GEMV")
    ap.add_argument("--shapes", default=None, help="with --ceiling: JSON list of [kernel ('gemv' or 'ceiling'), "
                                                   "label, tuning fields] timed on the stack")
    ap.add_argument("--no-sizes", action="store_true", help="with --ceiling: skip the 12-357 MB size sweep")
    ap.add_argument("--units", default=None, metavar="FILE",
                    help="also time the unit ceilings (MFMA shapes, LDS reads) into FILE")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize", nargs=2, metavar=("KIND", "DIR"))
    ap.add_argument("--command", default="", help="the profiled command, recorded in counter summaries")
    args = ap.parse_args()
    if args.summarize:
        kind, d = args.summarize
        if kind == "trace":
            print(summarize_trace(d))
        elif kind == "trace-grid":
            print(summarize_trace_grid(d))
        elif kind == "counter-table":
            print(summarize_counter_table(d))
        else:
            print(json.dumps(summarize_counters(d, args.command), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (the projection shards "
              "along N with no communication: one GPU runs the same kernel on its rows). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
