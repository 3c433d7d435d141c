#!/usr/bin/env python3
"""Benchmark: fused block-quantized GEMV on one MI355X.

Default workload — one "step" is the TinyLlama-1.1B-shaped Q4_K_M decode-step
weight pass at batch 1: for each of 22 layers q (Q4_K 2048x2048), k (Q4_K
256x2048), v (Q6_K 256x2048), o (Q4_K 2048x2048), gate and up (Q4_K
5632x2048), down (Q6_K 2048x5632), then lm_head (Q6_K 32000x2048): 155
GEMVs, 667,152,384 bytes of packed weights, every tensor distinct and
resident in HBM. The GEMVs run as one qk_gemv_batch per dependency stage
(q/k/v, o, gate/up, down per layer, then lm_head: 89 launches),
each stage with its own seeded fp32 N(0,1) x. The same pass is also timed as
155 single qk_gemv calls and as one persistent launch (qk_gemv_pass), each
eager and from a graph.

Reported (one JSON line): weight GB/s over the whole pass (value), decode
steps/s, % of the 8 TB/s HBM peak, the roofline of the dominant kernel
(timed with HIP events on the launch stream) and the CPU oracle on a bounded
sample of the same workload.

Other single-matrix workloads (--workload cfg0|cfg1|cfg2q8|cfg2q4|lmhead|gate,
cfg4gate:M|cfg4down:M for the multi-token path; down7b|down8b|down8b_q6k|
downqwen7b for the wide down projections of 7B-8B models and gate7b|o7b|v7b
for their 4096-column projections; tp8gate|tp8down|
tp8head for one GPU's share of the 1.1B shapes at 8-way tensor parallelism)
time one GEMV/GEMM over >= 1 GiB of rotating copies so that the data comes
from HBM and not from the 256 MB Infinity Cache; tall_q4k|tall_q6k|
tall_q6k2048|tall_q4k5632|tall_q8_0|tall_q4_0|tall_q6k11008|tall_q4k11008|
tall_q6k14336|tall_q4k14336|tall_q4k4096|tall_q6k4096 (and tall_q5k|tall_q2k|tall_q3k|tall_q5_1|
tall_q8_0h for the ggml formats, at 2048 columns or, with the suffix 5632, at
5632) time one GEMV over a single matrix of >= 1 GiB (sustained streaming);
tall_*/N over a matrix of N MiB instead. dequant_q6k and dequant_q6k_big time
qk_dequantize_row (Q6_K, 2^20 and 2^28 weights per call). --workload step[:P] times one whole decode step
(norms, RoPE, KV cache, attention, SwiGLU and every GEMV of the 1.1B model)
at position P from one HIP graph; step7b[:P] the same at Llama-2-7B shapes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused K-quant GEMV weight GB/s & % HBM peak; 1.1B-shape decode steps/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4


def synth_qk(t):
    from block_quantized_weight_gemv_amd import synth

    return synth.BLOCK_ELEMS[t]


def kernel_name(group):
    """Name (as rocprofv3 lists it) of the GEMV kernel that one batch of
    same-width tensors runs: formats <first, second>, prefetch depth 2,
    whether rows are split over waves (more than 64 units), whether a row
    slot has 16 or more lanes (more than 8 units), and the 16-byte pieces per
    thread of a row group when rows are streamed through LDS (launches of
    >= 128 MiB whose rows one wave covers, not q4_0), else 0; and the input
    transform (0: x as given)."""
    types = {t for _, t, _, _ in group}
    cols = group[0][3]
    # (a launch that mixes Q4_K and Q6_K takes Q6_K first, q4_0 before q8_0)
    first = next(t for t in (Q6_K, Q4_K, Q4_0, Q8_0, *range(5, 10)) if t in types)
    second = {Q6_K: Q4_K, Q4_0: Q8_0}.get(first, first) if len(types) > 1 else first
    unit = 64 if synth_qk(first) == 256 else 32
    units = cols // unit
    split = "true" if units > 64 else "false"
    wide = "true" if units > 8 else "false"  # row slots of 16 or more lanes
    from block_quantized_weight_gemv_amd import synth

    spl = 0
    rbs = [synth.row_bytes(t, cols) for _, t, _, _ in group]
    nbytes = sum(r * rb for (_, _, r, _), rb in zip(group, rbs))
    if units <= 64 and first != Q4_0 and nbytes >= 128 << 20 and all(
            (r * rb) % 16 == 0 for (_, _, r, _), rb in zip(group, rbs)):
        lanes = 1 << max(0, (units - 1).bit_length())
        rg = 4 * (64 // lanes)  # rows per group: 4 waves of 64 / lanes row slots
        np_ = max((rg * rb + 159) // 16 for rb in rbs)
        spl = -(-np_ // 256)
    return f"gemv_kernel<{first}, {second}, 2, {split}, {wide}, {spl}, 0>"  # last: no input transform

# TinyLlama-1.1B shapes (rows = out, cols = in): 22 layers, hidden 2048,
# 4 KV heads x 64 = 256, FFN 5632, vocab 32000.
LAYER = [("q", Q4_K, 2048, 2048), ("k", Q4_K, 256, 2048), ("v", Q6_K, 256, 2048), ("o", Q4_K, 2048, 2048),
         ("gate", Q4_K, 5632, 2048), ("up", Q4_K, 5632, 2048), ("down", Q6_K, 2048, 5632)]
N_LAYERS = 22
LM_HEAD = ("lm_head", Q6_K, 32000, 2048)


def decode_pass_tensors():
    out = []
    for l in range(N_LAYERS):
        for name, t, r, c in LAYER:
            out.append((f"blk.{l}.{name}", t, r, c))
    out.append(LM_HEAD)
    return out


def fail(msg: str) -> None:
    print(msg, file=sys.stderr)
    sys.exit(2)


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except Exception:
        return None
    from block_quantized_weight_gemv_amd.rocprof import source_sha

    e = data.get(f"{workload}:{kernel}")
    if not e or e.get("source_sha") != source_sha():
        return None
    return e.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------- CPU baseline

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_pass_rate(tensors, jobs, budget_s: float, threads: int):
    """Whole decode passes of the oracle over `threads` host threads (ctypes
    releases the GIL in the C oracle), repeated until about budget_s seconds
    have passed (at least one pass): (passes, seconds)."""
    import concurrent.futures as cf

    import oracle

    orc = oracle.get()

    def run(job):
        t, r, c, Wj, xj = job
        orc.gemv(t, Wj, r, c, xj)

    passes = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        while True:
            list(ex.map(run, sorted(jobs, key=lambda j: -j[3].nbytes)))
            passes += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    return passes, time.perf_counter() - t0


def cpu_prefill_rate(seed: int, threads: int, rows: int = 512):
    """The oracle's GEMM (fp64 sums) at M = 512 on `rows` rows of the 5632 x
    2048 Q4_K gate matrix, rows spread over `threads` host threads: GFLOP/s
    counted as 2*M*rows*cols."""
    import concurrent.futures as cf

    import oracle
    from block_quantized_weight_gemv_amd import synth

    orc = oracle.get()
    M, cols = 512, 2048
    W = synth.matrix(Q4_K, rows, cols, seed, stream=Q4_K)
    X = synth.bf16_matrix(M, cols, seed)
    rb = synth.row_bytes(Q4_K, cols)
    chunks = [(a, min(a + 16, rows)) for a in range(0, rows, 16)]

    def run(ch):
        a, b = ch
        orc.gemm(Q4_K, W[a * rb:b * rb], b - a, cols, X, M)

    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(run, chunks))
    dt = time.perf_counter() - t0
    return 2.0 * M * rows * cols / dt / 1e9, dt


def cpu_baseline(tensors, xs, seed, budget_s: float):
    """The oracle (plain C, fp64 sums) on the same workload, on this host:
    whole decode-step weight passes with one thread (the parity reference as
    the tests run it) and with every core of the process's affinity set; the
    prefill GEMM rate at M = 512 on a sample of rows. A reported baseline,
    not a target."""
    from block_quantized_weight_gemv_amd import synth

    jobs = [(t, r, c, synth.matrix(t, r, c, seed, stream=i), xs[i]) for i, (_, t, r, c) in enumerate(tensors)]
    total_bytes = sum(j[3].nbytes for j in jobs)
    cores = len(os.sched_getaffinity(0))
    p1, t1 = cpu_pass_rate(tensors, jobs, budget_s, 1)
    pn, tn = cpu_pass_rate(tensors, jobs, budget_s, cores)
    gflops, tg = cpu_prefill_rate(seed, cores)
    return {
        "value": round(pn * total_bytes / tn / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"whole decode-step weight passes (155 tensors, {total_bytes / 1e6:.1f} MB each, the same seeded "
                  f"bytes as the GPU run), plain C oracle with fp64 sums, tensors spread over {cores} host threads: "
                  f"{pn} passes in {tn:.1f} s; one thread: {p1} passes in {t1:.1f} s; prefill: the oracle GEMM at "
                  f"M = 512 on 512 rows of the 5632 x 2048 Q4_K matrix over {cores} threads in {tg:.3f} s",
        "decode_steps_per_s": round(pn / tn, 4),
        "single_thread_GB_per_s": round(p1 * total_bytes / t1 / 1e9, 4),
        "single_thread_decode_steps_per_s": round(p1 / t1, 4),
        "prefill_m512_GFLOP_per_s": round(gflops, 3),
        "cpu_model": cpu_model(),
        "affinity_cores": cores,
    }


# ---------------------------------------------------------------- GPU

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--seed", type=int, default=3)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of CPU oracle work")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--modes", default="grouped,single,chained_grouped,chained_pass",
                    help="launch plans of the decode pass to time (grouped is always timed: value is its rate)")
    args = ap.parse_args()
    if args.gpus != 1:
        fail("this benchmark runs on exactly one GPU: the GEMV path is single-GPU "
             "(multi-GPU row/K sharding is a design note only); run with --gpus 1")

    import torch

    if not torch.cuda.is_available():
        fail("no GPU visible")
    from block_quantized_weight_gemv_amd import qk, synth

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.workload.split(":")[0] in ("step", "step7b"):
        return bench_step(args, torch, qk)
    if args.workload != "decode":
        return bench_single(args, torch, qk, synth)

    tensors = decode_pass_tensors()
    total_bytes = sum(synth.row_bytes(t, c) * r for _, t, r, c in tensors)
    assert total_bytes == 667152384, total_bytes
    Ws = []
    for i, (_, t, r, c) in enumerate(tensors):
        Ws.append(torch.from_numpy(synth.matrix(t, r, c, args.seed, stream=i)).to("cuda"))
    ys = [torch.empty(r, dtype=torch.float32, device="cuda") for _, _, r, _ in tensors]
    # One x per dependency stage of each layer (q/k/v read one normed x, o the
    # attention output, gate/up one normed x, down the SwiGLU product) and one
    # for lm_head: distinct seeded N(0,1) vectors of the stage's width.
    stage_of = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
    stages, xs_host, xs_dev = [], [], []
    for i, (name, t, r, c) in enumerate(tensors):
        key = (name.split(".")[1], stage_of[name.split(".")[2]]) if name != "lm_head" else ("head", 0)
        if not stages or stages[-1][0] != key:
            xs_host.append(synth.vector(c, args.seed, stream=3000 + len(stages)))
            xs_dev.append(torch.from_numpy(xs_host[-1]).to("cuda"))
            stages.append((key, []))
        stages[-1][1].append(i)
    x_of = {}
    for si, (_, idx) in enumerate(stages):
        for i in idx:
            x_of[i] = si
    assert len(stages) == 4 * N_LAYERS + 1
    torch.cuda.synchronize()

    def item(i):
        _, t, r, c = tensors[i]
        return (t, Ws[i], r, c, xs_dev[x_of[i]], ys[i])

    grouped = [qk.make_gemv_batch([item(i) for i in idx]) for _, idx in stages]
    single = [item(i) for i in range(len(tensors))]

    def step_grouped():
        for d in grouped:
            qk.qk_gemv_batch(d)

    def step_single():
        for (t, W, r, c, x, y) in single:
            qk.qk_gemv(t, W, r, c, x, y)

    def capture(fn):
        if args.no_graph:
            return None
        try:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            torch.cuda.synchronize()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            return g
        except Exception as e:  # graph capture unavailable: eager only
            print(f"graph capture failed: {e}", file=sys.stderr)
            return None

    def timed(fn, k):
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k, (time.perf_counter() - w0) * 1e3 / k

    # The chained model of the step: each stage's x computed from the
    # outputs of the stage before by the step's glue (q/k/v: RMSNorm of the
    # previous layer's down output with weights, layer 0: the stage's N(0,1)
    # x; o: RMSNorm(q), standing in for the attention output; gate/up:
    # RMSNorm(o); down: SwiGLU(gate, up); lm_head: RMSNorm(the last down)),
    # run as 89 transformed-input launches (qk_gemv_batch_input) and as one
    # persistent launch (qk_gemv_pass) in which each stage waits on the
    # device for the outputs it reads.
    eps = 1e-5
    nw = torch.from_numpy(np.abs(synth.vector(2048, args.seed, stream=4000)) + np.float32(0.5)).to("cuda")
    ones = {c: torch.ones(c, device="cuda") for c in (2048, 5632)}
    zeros = {c: torch.zeros(c, device="cuda") for c in (2048, 5632)}
    ych = [torch.empty(r, dtype=torch.float32, device="cuda") for _, _, r, _ in tensors]
    name_of = {n: i for i, (n, _, _, _) in enumerate(tensors)}
    chain, chain_in, chain_src = [], [], []
    for si, (key, idx) in enumerate(stages):
        lay, kind = key
        if lay == "head":
            src = ("norm", name_of[f"blk.{N_LAYERS - 1}.down"])
        elif kind == 0:
            src = ("x",) if lay == "0" else ("norm_w", name_of[f"blk.{int(lay) - 1}.down"])
        elif kind == 1:
            src = ("norm", name_of[f"blk.{lay}.q"])
        elif kind == 2:
            src = ("norm", name_of[f"blk.{lay}.o"])
        else:
            src = ("swiglu", name_of[f"blk.{lay}.gate"], name_of[f"blk.{lay}.up"])
        x = xs_dev[si] if src[0] == "x" else ych[src[1]]
        chain.append([(tensors[i][1], Ws[i], tensors[i][2], tensors[i][3], x, ych[i]) for i in idx])
        chain_src.append(src)
        if src[0] == "x":
            chain_in.append(None)
        elif src[0] == "swiglu":
            chain_in.append((qk.QK_PASS_IN_SWIGLU, ych[src[2]], None, 0.0))
        else:
            chain_in.append((qk.QK_PASS_IN_RMSNORM, None, nw if src[0] == "norm_w" else None, eps))
    x_out = {c: torch.empty(c, device="cuda") for c in (2048, 5632)}
    chain_launch = []
    for st, src in zip(chain, chain_src):
        d = qk.make_gemv_batch(st)
        c = st[0][3]
        if src[0] == "x":
            inp = qk.make_gemv_input(qk.QK_INPUT_PLAIN)
        elif src[0] == "swiglu":
            inp = qk.make_gemv_input(qk.QK_INPUT_SWIGLU, aux=ych[src[2]])
        else:
            inp = qk.make_gemv_input(qk.QK_INPUT_ADD_RMSNORM, aux=zeros[c], norm_w=nw if src[0] == "norm_w" else ones[c],
                                     eps=eps, x_out=x_out[c])
        chain_launch.append((d, inp))

    def step_chained_grouped():
        for d, inp in chain_launch:
            qk.qk_gemv_batch_input(d, inp)

    gpass = qk.GemvPass(chain, chain_in)

    def step_chained_pass():
        gpass.run()

    results = {}
    # Every mode is timed eager (host launches in the timed loop) and from a
    # captured graph; the three launch plans compute the same 155 products.
    want = set(args.modes.split(",")) | {"grouped"}
    modes = [(m, f) for m, f in (("grouped", step_grouped), ("single", step_single),
                                 ("chained_grouped", step_chained_grouped), ("chained_pass", step_chained_pass))
             if m in want]
    for mode, fn in modes:
        for _ in range(args.warmup):
            fn()
        r = {}
        r["eager_ms"], r["eager_wall_ms"] = timed(fn, args.steps)
        g = capture(fn)
        if g is not None:
            for _ in range(args.warmup):
                g.replay()
            r["graph_ms"] = timed(g.replay, args.steps)[0]
        elif "eager_ms" not in r:
            r["eager_ms"], r["eager_wall_ms"] = timed(fn, args.steps)
        r["ms"] = r.get("graph_ms", r.get("eager_ms"))
        results[mode] = r
    ms = results["grouped"]["ms"]

    # Per-kernel time: the launches of one grouped step that run the same
    # kernel, back to back in step order (replayed as one graph like the step
    # itself), timed with HIP events on the launch stream; events around
    # single launches of a few microseconds would distort them. A kernel with
    # few launches per step (lm_head: one) has its sequence repeated inside
    # the graph to at least 20 launches, so that the cost of starting a graph
    # replay is spread as it is over the step's 89 launches.
    by_kernel = {}
    for si, (_, idx) in enumerate(stages):
        by_kernel.setdefault(kernel_name([tensors[i] for i in idx]), []).append(si)
    per_kernel = {}
    kt_steps = max(5, min(args.steps, 20))
    for kname, sis in by_kernel.items():
        reps = -(-20 // len(sis))

        def only(sis=sis, reps=reps):
            for _ in range(reps):
                for si in sis:
                    qk.qk_gemv_batch(grouped[si])

        only()
        gk = capture(only)
        ms_k, _ = timed(gk.replay if gk is not None else only, kt_steps)
        nbytes = sum(synth.row_bytes(tensors[i][1], tensors[i][3]) * tensors[i][2] for si in sis for i in stages[si][1])
        per_kernel[kname] = {"launches": len(sis), "us": ms_k * 1e3 / reps, "bytes": nbytes}
    dom = max(per_kernel, key=lambda n: per_kernel[n]["us"])
    d = per_kernel[dom]
    stream_us = d["us"] / d["launches"]
    avg_bytes = d["bytes"] / d["launches"]

    # Average launch duration of the dominant kernel: its launches of one
    # step replayed back to back as one graph, timed with HIP events on the
    # launch stream (kernel time plus the dispatch gap after each launch).
    avg_us = stream_us
    achieved = avg_bytes / (avg_us * 1e-6) / 1e9
    traffic = load_traffic(dom, "decode")

    # parity spot check of the timed outputs, oracle on sampled rows
    step_grouped()
    torch.cuda.synchronize()
    parity = spot_check(tensors, ys, [xs_host[x_of[i]] for i in range(len(tensors))], args.seed)

    # achievable streaming-read and copy rates on this device, same run
    probe, copy_probe = hbm_probe(torch, qk)

    gbs = total_bytes / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": "TinyLlama-1.1B-shaped Q4_K_M decode-step weight pass, batch 1: 22 x {q,k,o,gate,up Q4_K; "
                        "v,down Q6_K} + lm_head Q6_K 32000x2048; 155 weight matrices, 667152384 packed weight "
                        "bytes; one qk_gemv_batch per dependency stage (q/k/v, o, gate/up, down, lm_head)",
            "launches_per_step": sum(v["launches"] for v in per_kernel.values()),
            "timing": "hipGraph replay" if "graph_ms" in results["grouped"] else "eager launches",
            "seed": args.seed,
        },
        "decode_steps_per_s": round(1e3 / ms, 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "modes": {m: {k: (round(v, 5) if v is not None else None) for k, v in r.items()} for m, r in results.items()},
        "per_kernel": {n: {"launches_per_step": v["launches"],
                           "avg_us": round(v["us"] / v["launches"], 3),
                           "bytes_per_launch": round(v["bytes"] / v["launches"]),
                           "GB_per_s": round(v["bytes"] / (v["us"] * 1e-6) / 1e9, 1)} for n, v in per_kernel.items()},
        "hbm_read_probe_GB_per_s": probe,
        "hbm_copy_probe_GB_per_s": copy_probe,
        "pct_of_read_probe": round(100.0 * gbs / probe, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                     "algorithmic_bytes_per_launch": round(avg_bytes), "avg_launch_us": round(avg_us, 3),
                     "launches_timed": d["launches"] * kt_steps},
        "parity": parity,
    }
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(tensors, [xs_host[x_of[i]] for i in range(len(tensors))], args.seed,
                                           args.cpu_budget)
    if "single" in results:
        res["single_155_calls_eager_GB_per_s"] = round(total_bytes / (results["single"]["eager_ms"] * 1e-3) / 1e9, 2)
        res["single_155_calls_eager_steps_per_s"] = round(1e3 / results["single"]["eager_ms"], 2)
    for m in ("chained_grouped", "chained_pass"):
        if m in results:
            res[f"{m}_GB_per_s"] = round(total_bytes / (results[m]["ms"] * 1e-3) / 1e9, 2)
    if "chained_pass" in results:
        res["chained_pass_grid"] = gpass.grid
        if gpass.gave_up():
            fail("the persistent pass gave up a wait")
        # the chained outputs of the last run against the oracle, on the
        # oracle's transform of the outputs each stage read
        step_chained_pass()
        torch.cuda.synchronize()
        res["chained_parity"] = chained_spot_check(tensors, ych, chain_src, xs_host, nw.cpu().numpy(), eps, args.seed)
    print(json.dumps(res), flush=True)


def hbm_probe(torch, qk, nbytes=2 << 30, reps=10):
    """Plain streaming read of 2 GiB (qk_probe_read) and plain copy of 512 MiB
    (qk_probe_copy), best of `reps` each. The copy is also the known-size
    kernel that calibrates the HBM byte counters (rocprof harness)."""
    def best_rate(fn, moved):
        fn()
        torch.cuda.synchronize()
        best = 0.0
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = max(best, moved / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        return round(best, 1)

    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(256 * 8, dtype=torch.int32, device="cuda")
    read = best_rate(lambda: qk.qk_probe_read(buf, nbytes, out), nbytes)
    half = 512 << 20
    src, dst = buf[:half], buf[half:2 * half]
    copy = best_rate(lambda: qk.qk_probe_copy(src, dst, half), 2 * half)
    del buf, src, dst
    return read, copy


def spot_check(tensors, ys, xs, seed):
    import oracle
    from block_quantized_weight_gemv_amd import synth

    orc = oracle.get()
    worst = 0.0
    idx = [0, 1, 2, 3, 4, 6, len(tensors) - 1]
    for i in idx:
        _, t, r, c = tensors[i]
        W = synth.matrix(t, r, c, seed, stream=i)
        rows = sorted(set([0, r - 1] + list(synth.rng(seed, 77 + i).integers(0, r, 16))))
        yr, a = orc.gemv_rows(t, W, c, xs[i], rows)
        yg = ys[i].cpu().numpy()[rows]
        ok, w = oracle.within_tolerance(yg, yr, a)
        if not ok:
            fail(f"parity failure on {tensors[i][0]}: worst ratio {w}")
        worst = max(worst, w)
    return {"checked": [tensors[i][0] for i in idx], "worst_err_over_tol": round(worst, 6)}


def chained_spot_check(tensors, ych, chain_src, xs_host, nw, eps, seed):
    """Sampled rows of the chained pass's q, o, gate and down of layers 0 and
    1 and of lm_head against the oracle applied to the oracle's transform
    (RMSNorm, SwiGLU) of the outputs each stage read."""
    import oracle
    from block_quantized_weight_gemv_amd import synth

    orc = oracle.get()
    stage_of_kind = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3}
    t_stage, s, prev = [], -1, None
    for n, _, _, _ in tensors:
        key = (n.split(".")[1], stage_of_kind[n.split(".")[2]]) if n != "lm_head" else ("head", 0)
        if key != prev:
            s, prev = s + 1, key
        t_stage.append(s)
    worst, checked = 0.0, []
    for i in [0, 3, 4, 6, 7, 10, len(tensors) - 1]:
        _, t, r, c = tensors[i]
        src = chain_src[t_stage[i]]
        if src[0] == "x":
            x = xs_host[t_stage[i]]
        elif src[0] == "swiglu":
            x = orc.swiglu(ych[src[1]].cpu().numpy(), ych[src[2]].cpu().numpy()).astype(np.float32)
        else:
            v = ych[src[1]].cpu().numpy()
            x = orc.rmsnorm(v, nw if src[0] == "norm_w" else np.ones(v.size, np.float32), eps)
        W = synth.matrix(t, r, c, seed, stream=i)
        rows = sorted(set([0, r - 1] + list(synth.rng(seed, 177 + i).integers(0, r, 16))))
        yr, a = orc.gemv_rows(t, W, c, x, rows)
        ok, w = oracle.within_tolerance(ych[i].cpu().numpy()[rows], yr, a)
        if not ok:
            fail(f"chained parity failure on {tensors[i][0]}: worst ratio {w}")
        worst = max(worst, w)
        checked.append(tensors[i][0])
    return {"checked": checked, "worst_err_over_tol": round(worst, 6)}


def bench_single(args, torch, qk, synth):
    """One GEMV (cfg0, cfg1, cfg2q8, cfg2q4) or GEMM (cfg4gate/cfg4down at
    --m) over rotating copies covering >= 1 GiB."""
    spec = {"cfg0": (Q4_K, 512, 2048, 0), "cfg1": (Q6_K, 2048, 5632, 1), "cfg2q8": (Q8_0, 5632, 2048, 2),
            "cfg2q4": (Q4_0, 5632, 2048, 2), "cfg2q8s": (Q8_0, 2048, 2048, 2), "cfg2q4s": (Q4_0, 2048, 2048, 2),
            # GGUF's Q8_0 (34-byte blocks, fp16 scale) at the gate shape
            "cfg2q8h": (5, 5632, 2048, 2),
            # the other ggml formats at the gate / down shapes
            "gate_q5k": (7, 5632, 2048, 3), "gate_q2k": (8, 5632, 2048, 3), "down_q3k": (9, 2048, 5632, 3),
            "gate_q5_1": (6, 5632, 2048, 3),
            "lmhead": (Q6_K, 32000, 2048, 3), "gate": (Q4_K, 5632, 2048, 3),
            # down projections of 7B-8B models (wide rows; 11008 = 43 Q6_K blocks)
            "down7b": (Q6_K, 4096, 11008, 3), "down8b": (Q4_K, 4096, 14336, 3), "down8b_q6k": (Q6_K, 4096, 14336, 3),
            "downqwen7b": (Q6_K, 3584, 18944, 3),
            # the other 7B projections (4096 columns)
            "gate7b": (Q4_K, 11008, 4096, 3), "o7b": (Q4_K, 4096, 4096, 3), "v7b": (Q6_K, 4096, 4096, 3),
            # one GPU's share at 8-way tensor parallelism of the 1.1B shapes
            "tp8gate": (Q4_K, 704, 2048, 3), "tp8down": (Q6_K, 2048, 768, 3), "tp8head": (Q6_K, 4000, 2048, 3),
            "cfg4gate": (Q4_K, 5632, 2048, 4), "cfg4down": (Q6_K, 2048, 5632, 4)}
    # sustained streaming: one matrix of >= 1 GiB per call (rows computed)
    tall = {"tall_q4k": (Q4_K, 2048), "tall_q6k": (Q6_K, 5632), "tall_q6k2048": (Q6_K, 2048),
            "tall_q4k5632": (Q4_K, 5632), "tall_q8_0": (Q8_0, 2048), "tall_q4_0": (Q4_0, 2048),
            "tall_q5k": (7, 2048), "tall_q2k": (8, 2048), "tall_q3k": (9, 2048), "tall_q5_1": (6, 2048),
            "tall_q8_0h": (5, 2048), "tall_q5k5632": (7, 5632), "tall_q2k5632": (8, 5632),
            "tall_q3k5632": (9, 5632), "tall_q5_1_5632": (6, 5632), "tall_q8_0h5632": (5, 5632),
            "tall_q6k11008": (Q6_K, 11008), "tall_q4k14336": (Q4_K, 14336), "tall_q6k14336": (Q6_K, 14336),
            "tall_q4k11008": (Q4_K, 11008), "tall_q4k4096": (Q4_K, 4096), "tall_q6k4096": (Q6_K, 4096)}
    name = args.workload.split(":")[0]
    M = int(args.workload.split(":")[1]) if ":" in args.workload else 1
    if name.startswith("dequant"):
        return bench_dequant(args, torch, qk, synth, name)
    mib = 1024
    if "/" in name:  # tall_*/N: a matrix of N MiB (rotating copies still cover >= 1 GiB)
        name, mib = name.split("/")[0], int(name.split("/")[1])
    if name in tall:
        t, c = tall[name]
        rb = synth.row_bytes(t, c)
        r = -(-(mib << 20) // rb)
        r += r % 2  # an even row count (odd Q6_K/Q3_K block counts are fused only then)
        # a seeded 64 MiB block of whole rows, tiled to the full matrix (the
        # kernels have no data-dependent control flow: content does not change
        # their speed)
        base_rows = min(r, (64 << 20) // rb)
        blk = torch.from_numpy(synth.matrix(t, base_rows, c, 5, stream=t)).to("cuda")
        W = torch.empty(r * rb, dtype=torch.uint8, device="cuda")
        for off in range(0, r * rb, blk.numel()):
            n = min(blk.numel(), r * rb - off)
            W[off:off + n].copy_(blk[:n])
        del blk
        if mib >= 1024:
            Ws, ncopies = [W] * 4, 4
        else:
            ncopies = max(2, -(-1024 // mib))
            Ws = [W] + [W.clone() for _ in range(ncopies - 1)]
        seed = 5
        Wn = np.empty(r * rb, dtype=np.uint8)  # only its size is used below
    elif name in spec:
        t, r, c, seed = spec[name]
        Wn = synth.matrix(t, r, c, seed, stream=t)
        ncopies = max(2, int(np.ceil((1 << 30) / Wn.nbytes)))
        base = torch.from_numpy(Wn).to("cuda")
        Ws = [base.clone() for _ in range(ncopies)]
    else:
        fail(f"unknown workload {args.workload}")
    if M == 1:
        x = torch.from_numpy(synth.vector(c, seed)).to("cuda")
        y = torch.empty(r, device="cuda")
        fn = lambda W: qk.qk_gemv(t, W, r, c, x, y)
    else:
        X = torch.from_numpy(synth.bf16_matrix(M, c, seed).view(np.int16)).to("cuda")
        y = torch.empty(M * r, device="cuda")
        fn = lambda W: qk.qk_gemm_prefill(t, W, r, c, X, M, y)
    # One graph replays one call per copy (rotating through >= 1 GiB, so the
    # weights come from HBM), another the same number of calls on one copy
    # (cache-resident when it fits the 256 MB Infinity Cache).
    def graph_of(seq):
        for W in seq[:2]:
            fn(W)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for W in seq:
                fn(W)
        torch.cuda.synchronize()
        return g

    def time_graph(g, calls):
        """Per-call time of each of >= 20 replays (HIP events around each),
        after >= 200 ms of replays: from an idle start the rate of a
        sustained read runs high for ~2 ms, dips by a third around 4 ms and
        settles after ~25 ms (1 GiB Q4_K: 5.4, 3.6, then 5.4-5.8 TB/s), so
        the timed replays see the settled state."""
        t_end = time.time() + 0.2
        n = 0
        while n < max(1, args.warmup // 4) or time.time() < t_end:
            g.replay()
            torch.cuda.synchronize()
            n += 1
        times = []
        for _ in range(max(20, args.steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / calls)
        return sorted(times)

    ts = time_graph(graph_of(Ws), ncopies)
    hot = time_graph(graph_of([Ws[0]] * ncopies), ncopies)
    us = float(np.median(ts))
    gbs = Wn.nbytes / (us * 1e-6) / 1e9
    res = {"metric": METRIC, "workload": args.workload, "type": synth.NAMES[t], "rows": r, "cols": c, "M": M,
           "weight_bytes": int(Wn.nbytes), "us_per_call": round(us, 3), "GB_per_s": round(gbs, 1),
           "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "rotating_copies": ncopies,
           "us_per_call_min": round(ts[0], 3), "us_per_call_max": round(ts[-1], 3), "repeats": len(ts),
           "GB_per_s_best": round(Wn.nbytes / (ts[0] * 1e-6) / 1e9, 1),
           "hot_us_per_call": round(float(np.median(hot)), 3),
           "timing": "hipGraph replay after >= 200 ms of replays, median of the repeats (min and max beside it)"}
    if M > 1:
        res["TFLOP_per_s"] = round(2.0 * M * r * c / (us * 1e-6) / 1e12, 2)
        res["pct_bf16_peak"] = round(100 * res["TFLOP_per_s"] / BF16_PEAK_TFLOPS, 2)
    print(json.dumps(res), flush=True)


def bench_dequant(args, torch, qk, synth, name):
    """qk_dequantize_row on Q6_K blocks: dequant_q6k dequantises the 2^20
    weights of the configuration's check per call (860,160 bytes in, 4 MiB
    out), rotating over 256 input and output copies (1 GiB of output) so
    that the writes reach HBM; dequant_q6k_big dequantises 2^28 weights (220
    MB in, 1 GiB out) per call. The roofline is write-dominated: bytes read
    plus 4 bytes written per weight, against 8 TB/s."""
    n = (1 << 28) if name == "dequant_q6k_big" else (1 << 20)
    copies = 1 if n >= (1 << 28) else 256
    src = torch.from_numpy(synth.matrix(Q6_K, 1, 1 << 20, seed=1, stream=7)).to("cuda")
    ins = [src.repeat(n >> 20).contiguous() for _ in range(min(copies, 4))]
    outs = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(copies)]
    calls = [(ins[i % len(ins)], outs[i]) for i in range(copies)]

    def run(seq):
        for a, b in seq:
            qk.qk_dequantize_row(Q6_K, a, n, b)

    run(calls[:2])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(calls)
    torch.cuda.synchronize()
    # >= 200 ms of replays first (the rate settles after ~25 ms of sustained traffic)
    t_end = time.time() + 0.2
    while time.time() < t_end:
        g.replay()
        torch.cuda.synchronize()
    times = []
    for _ in range(max(20, args.steps)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / copies)
    times.sort()
    us = float(np.median(times))
    read_b = n // 256 * 210
    moved = read_b + 4 * n
    res = {"metric": "dequantisation GB/s (bytes read + fp32 written) & % HBM peak", "workload": name,
           "type": "Q6_K", "weights": n, "bytes_read": read_b, "bytes_written": 4 * n, "us_per_call": round(us, 3),
           "us_per_call_min": round(times[0], 3), "us_per_call_max": round(times[-1], 3), "repeats": len(times),
           "GB_per_s": round(moved / (us * 1e-6) / 1e9, 1),
           "pct_hbm_peak": round(100 * moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2), "rotating_copies": copies,
           "timing": "hipGraph replay after >= 200 ms of replays, median of the repeats"}
    print(json.dumps(res), flush=True)


def bench_step(args, torch, qk):
    """One whole decode step (the token's embedding row, per layer norm,
    q/k/v, RoPE and the fp16 cache store, attention over positions 0..P,
    output projection, norm, gate/up, SwiGLU, down, then the final norm and
    the output matrix), replayed from one HIP graph at position P:
    --workload step:P at TinyLlama-1.1B shapes (22 layers, 2048 wide, 32/4
    heads, FFN 5632), step7b:P at Llama-2-7B shapes (32 layers, 4096 wide, 32
    heads of 128, FFN 11008: the down projection is a wide Q6_K row of 43
    blocks); Q4_K_M types, default P = 511 (a 512-token context). Cache rows
    0..P-1 hold seeded fp16 values; each timed step writes row P and attends
    over rows 0..P. At 7B shapes layer 0's weights are generated and every
    other layer gets device copies of them (distinct memory, 3.9 GB in all:
    the kernels' speed does not depend on the values)."""
    from block_quantized_weight_gemv_amd.step import DecodeStep, StepConfig, synthetic_weights

    name = args.workload.split(":")[0]
    P = int(args.workload.split(":")[1]) if ":" in args.workload else 511
    if name == "step7b":
        cfg = StepConfig(dim=4096, n_layers=32, n_heads=32, n_kv_heads=32, ffn=11008, vocab=32000,
                         max_pos=max(2048, P + 1))
        one = StepConfig(dim=4096, n_layers=1, n_heads=32, n_kv_heads=32, ffn=11008, vocab=32000, max_pos=1)
        w = {k: torch.from_numpy(v).to("cuda") for k, v in synthetic_weights(one, args.seed).items()}
        for l in range(1, cfg.n_layers):
            for k in [k for k in list(w) if k.startswith("0.")]:
                w[f"{l}.{k[2:]}"] = w[k].clone()
        model = "Llama-2-7B"
    else:
        cfg = StepConfig(max_pos=max(2048, P + 1))
        w = synthetic_weights(cfg, args.seed)
        model = "TinyLlama-1.1B"
    if not 0 <= P < cfg.max_pos:
        fail("position out of range")
    step = DecodeStep(cfg, w)
    g = torch.Generator(device="cuda").manual_seed(args.seed)
    for c in (step.k_cache, step.v_cache):
        c.copy_(torch.randn(c.shape, generator=g, device="cuda", dtype=torch.float16).view(torch.int16))
    step.capture()
    tok = 1234
    for _ in range(args.warmup):
        step.forward(tok, P)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step.forward(tok, P)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    weight_bytes = sum(t.numel() for k, t in step.w.items() if not k.endswith("norm") and k != "token_embd")
    kv_bytes = cfg.n_layers * (P + 1) * cfg.kv_dim * 2 * 2
    res = {"metric": f"decode step tokens/s ({model} shapes, Q4_K_M types, one sequence)",
           "workload": args.workload, "position": P, "ms_per_token": round(ms, 4),
           "tokens_per_s": round(1e3 / ms, 1), "weight_bytes_per_token": int(weight_bytes),
           "kv_bytes_per_token": int(kv_bytes), "fused": bool(step.fused),
           "weight_GB_per_s": round(weight_bytes / (ms * 1e-3) / 1e9, 1),
           "timing": "HIP events over --steps forward() calls: position write, embedding row, graph replay",
           "data": "synthetic seeded weights (block scales x0.02) and KV cache"}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
