"""rocprofv3 harness for the GEMV kernels.

Runs bench.py under rocprofv3 in separate passes and turns the CSV output into
the short text summaries kept under profiles/ plus the per-launch HBM traffic
table (profiles/traffic.json) that bench.py reports:

* a kernel trace with per-kernel statistics (rocprofv3 --kernel-trace
  --stats): calls and average/min/max duration per kernel, and the average
  time from one launch's start to the next launch's start (the stream time a
  launch occupies, which is what HIP events around back-to-back launches
  measure: the kernel's duration plus the dispatch gap after it);
* one hardware-counter pass per counter (rocprofv3 --pmc FETCH_SIZE, then
  --pmc WRITE_SIZE; each KiB of HBM traffic per dispatch), never combined
  with any trace option; for multi-token workloads also MfmaUtil (the
  matrix cores' busy cycles over GRBM_GUI_ACTIVE times the SIMD count),
  SQ_INSTS_VALU_MFMA_MOPS_BF16 (bf16 MFMA flops / 512) and VALUBusy, one
  pass each.

Counter calibration: bench.py runs qk_probe_copy, a plain copy of 512 MiB, in
the same process. Its counted bytes against the known 512 MiB read and 512 MiB
written give one factor per counter, and every GEMV kernel's count is scaled
by it.

The harness only starts rocprofv3 as a child process (cwd /tmp, TMPDIR=/tmp)
with the Python interpreter and bench.py after "--"; it never touches the GPU
itself. Usage, on a machine with the GPU:

    python -m block_quantized_weight_gemv_amd.rocprof decode --out DIR

writes DIR/decode_pass_gemv_kernels.txt, DIR/decode_pass_hbm_traffic.txt
(kept under profiles/ as decode_pass_gemv_kernels_hbm_traffic.txt) and
DIR/traffic.json.

    python -m block_quantized_weight_gemv_amd.rocprof single --workload W --out DIR

profiles one single-matrix bench workload (bench.py --workload W: a GEMV,
few-token or prefill call over rotating copies) the same way and writes
DIR/W.txt (the counters scaled with the calibration of DIR/traffic.json when
a decode run wrote one there).

    python -m block_quantized_weight_gemv_amd.rocprof step --workload step:P --out DIR

traces the whole decode step (bench.py --workload step:P) and writes the
per-kernel table DIR/decode_step_step_posP.txt.
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
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BENCH = os.path.join(ROOT, "bench.py")
COPY_KERNEL = "copy_probe_kernel"
COPY_BYTES = 512 << 20  # read and written per copy probe dispatch


def kernel_key(name: str) -> str:
    """'void qk::gemv_kernel<3, 3, 2, false>(qk::GemvWork, qk::GemvPlan)' ->
    'gemv_kernel<3, 3, 2, false>' (anonymous-namespace prefixes dropped)."""
    n = name.strip()
    n = re.sub(r"^void\s+", "", n)
    n = n.split("(")[0] if not n.startswith("(") else n.split(")::", 1)[-1].split("(")[0]
    n = re.sub(r"^(qk::|\(anonymous namespace\)::)", "", n)
    return n


# The sources the GEMV kernels are built from: a traffic entry is valid only
# for the hash of these.
GEMV_SOURCES = ("qk_gemv.hip", "qk_gemv_body.h", "qk_decode.h", "qk_formats.h", "qk_launch.h")


def source_sha() -> str:
    """Hash of the GEMV kernel sources; a traffic entry is valid only for it."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for f in GEMV_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _run(cmd: list[str], log: str, timeout: float) -> int:
    env = dict(os.environ, TMPDIR="/tmp")
    with open(log, "w") as fh:
        fh.write("$ " + " ".join(cmd) + "\n")
        fh.flush()
        try:
            p = subprocess.run(cmd, cwd="/tmp", env=env, stdout=fh, stderr=subprocess.STDOUT, timeout=timeout)
        except subprocess.TimeoutExpired:
            fh.write(f"\n[harness] killed after {timeout} s\n")
            return 124
    return p.returncode


def bench_cmd(bench_args: list[str]) -> list[str]:
    return [sys.executable, BENCH, *bench_args]


def trace_cmd(out: str, bench_args: list[str]) -> list[str]:
    return ["rocprofv3", "--kernel-trace", "--stats", "-d", out, "-o", "run", "--output-format", "csv", "--",
            *bench_cmd(bench_args)]


def pmc_cmd(counter: str, out: str, bench_args: list[str]) -> list[str]:
    return ["rocprofv3", "--pmc", counter, "-d", out, "-o", "run", "--output-format", "csv", "--",
            *bench_cmd(bench_args)]


def _find(out: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(out, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {out}")
    return hits[0]


def summarize_trace(trace_csv: str) -> dict:
    """Per kernel: calls, mean/min/max duration (us), the mean duration of
    back-to-back launches (those starting within 20 us of the previous
    launch's end: graph replays, as opposed to host-paced eager launches) and
    the mean start-to-next-start (us) over launches followed by another
    launch within 50 us; and the mean over its steady calls, those starting
    100 ms or more after its first call (a sustained read settles within
    ~25 ms of an idle start)."""
    rows = []
    with open(trace_csv) as fh:
        for r in csv.DictReader(fh):
            # grid sizes count work-items; workgroups over all three dimensions
            g = w = 1
            for ax in "XYZ":
                ws = max(int(r.get("Workgroup_Size_" + ax) or 1), 1)
                g *= -(-int(r.get("Grid_Size_" + ax) or 1) // ws)
                w *= ws
            rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), kernel_key(r["Kernel_Name"]),
                         g * w, w))
    rows.sort()
    out: dict[str, dict] = {}
    for i, (s, e, k, g, w) in enumerate(rows):
        d = out.setdefault(k, {"dur": [], "next": [], "shapes": {}, "b2b": [], "t0": s, "steady": []})
        d["dur"].append((e - s) / 1e3)
        if s - d["t0"] >= 100_000_000:
            d["steady"].append((e - s) / 1e3)
        if i > 0 and (s - rows[i - 1][1]) / 1e3 < 20.0:
            d["b2b"].append((e - s) / 1e3)
        sh = f"{g // max(w, 1)}x{w}"
        d["shapes"][sh] = d["shapes"].get(sh, 0) + 1
        if i + 1 < len(rows):
            nxt = (rows[i + 1][0] - s) / 1e3
            if nxt < 50.0:
                d["next"].append(nxt)
    res = {}
    for k, d in out.items():
        res[k] = {"calls": len(d["dur"]), "mean_us": statistics.fmean(d["dur"]), "min_us": min(d["dur"]),
                  "max_us": max(d["dur"]),
                  "back_to_back_mean_us": statistics.fmean(d["b2b"]) if d["b2b"] else None,
                  "start_to_next_start_us": statistics.fmean(d["next"]) if d["next"] else None,
                  "steady_calls": len(d["steady"]),
                  "steady_mean_us": statistics.fmean(d["steady"]) if d["steady"] else None,
                  "workgroups_x_threads": d["shapes"]}
    return res


def summarize_counter(counter_csv: str, counter: str) -> dict:
    """Per kernel: dispatches and mean counter value per dispatch."""
    vals: dict[str, list[float]] = {}
    with open(counter_csv) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(kernel_key(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: {"dispatches": len(v), "mean": statistics.fmean(v)} for k, v in vals.items()}


def _bench_json(log: str) -> dict | None:
    with open(log) as fh:
        lines = [l for l in fh if l.startswith("{")]
    return json.loads(lines[-1]) if lines else None


def decode(out: str, steps: int, warmup: int) -> int:
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    sha = source_sha()
    # the grouped launch plan only (the one the bench line's value and
    # roofline time): the other plans launch the same kernels over other
    # groupings, which would mix into the per-kernel means and counters
    trace_args = ["--steps", str(steps), "--warmup", str(warmup), "--modes", "grouped"]
    pmc_args = ["--steps", "10", "--warmup", "2", "--no-cpu", "--modes", "grouped"]
    t0 = time.time()
    # the same bench command without the profiler, for its own timings
    cmd = bench_cmd(trace_args)
    print("[harness] untraced bench:", " ".join(cmd), flush=True)
    rc = _run(cmd, os.path.join(out, "bench.log"), 600)
    print(f"[harness] untraced bench rc={rc} ({time.time() - t0:.0f} s)", flush=True)
    plain = _bench_json(os.path.join(out, "bench.log"))
    if rc != 0 or plain is None:
        return rc or 3
    cmd = trace_cmd(os.path.join(out, "trace"), trace_args)
    print("[harness] kernel trace:", " ".join(cmd), flush=True)
    rc = _run(cmd, os.path.join(out, "trace.log"), 600)
    print(f"[harness] kernel trace rc={rc} ({time.time() - t0:.0f} s)", flush=True)
    bench = _bench_json(os.path.join(out, "trace.log"))
    if rc != 0 and bench is None:
        return rc
    tr = summarize_trace(_find(os.path.join(out, "trace"), "kernel_trace.csv"))
    counters = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cmd = pmc_cmd(c, os.path.join(out, c), pmc_args)
        print(f"[harness] counter pass {c}:", " ".join(cmd), flush=True)
        rc = _run(cmd, os.path.join(out, c + ".log"), 90)
        print(f"[harness] counter pass {c} rc={rc}", flush=True)
        if rc != 0:
            return rc
        counters[c] = summarize_counter(_find(os.path.join(out, c), "counter_collection.csv"), c)
    fac = {}
    for c in counters:
        cp = counters[c].get(COPY_KERNEL)
        if not cp or cp["mean"] <= 0:
            print(f"[harness] no {COPY_KERNEL} dispatch counted for {c}", flush=True)
            return 3
        fac[c] = COPY_BYTES / (cp["mean"] * 1024.0)

    bench_cmd_txt = "python bench.py " + " ".join(trace_args)
    per_kernel = plain.get("per_kernel", {})
    lines = [
        "# Decode-step weight pass (TinyLlama-1.1B shapes, Q4_K_M, batch 1): GEMV kernels under rocprofv3",
        "",
        f"command: cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
        f"{bench_cmd_txt}",
        f"made by: python -m block_quantized_weight_gemv_amd.rocprof decode --out <dir> (GEMV kernel source {sha})",
        "",
        "kernel | calls | mean us | min us | max us | back-to-back mean us | start-to-next-start us | "
        "untraced bench avg_us per launch | launch shapes (workgroups x threads: count)",
        "---|---|---|---|---|---|---|---|---",
    ]

    def f3(v):
        return f"{v:.3f}" if v is not None else "-"

    for k in sorted(tr, key=lambda k: -tr[k]["calls"] * tr[k]["mean_us"]):
        d = tr[k]
        b = per_kernel.get(k, {}).get("avg_us")
        shapes = ", ".join(f"{s}: {n}" for s, n in sorted(d["workgroups_x_threads"].items()))
        lines.append(f"{k} | {d['calls']} | {d['mean_us']:.3f} | {d['min_us']:.3f} | {d['max_us']:.3f} | "
                     f"{f3(d['back_to_back_mean_us'])} | {f3(d['start_to_next_start_us'])} | "
                     f"{b if b is not None else '-'} | {shapes}")
    rf = plain["roofline"]
    k = rf.get("kernel")
    t = tr.get(k, {})
    lines += ["", f"roofline kernel {k}: untraced bench avg_launch_us {rf.get('avg_launch_us')} (HIP events "
              f"around graph replays of its launches: the kernel plus the dispatch gap after it) vs rocprofv3 "
              f"mean duration {f3(t.get('mean_us'))} us (back-to-back launches {f3(t.get('back_to_back_mean_us'))} "
              f"us); achieved {rf.get('achieved')} GB/s of {rf.get('peak')}.",
              f"untraced bench line: value {plain.get('value')} GB/s, ms_per_step {plain.get('ms_per_step')}, "
              f"read probe {plain.get('hbm_read_probe_GB_per_s')} GB/s."]
    if bench:
        lines += [f"traced bench line (tracing lengthens every dispatch gap): value {bench.get('value')} GB/s, "
                  f"ms_per_step {bench.get('ms_per_step')}."]
    with open(os.path.join(out, "decode_pass_gemv_kernels.txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    pmc_txt = "python bench.py " + " ".join(pmc_args)
    tl = [
        "# Decode-step weight pass: HBM bytes per GEMV launch from rocprofv3 counters",
        "",
        f"commands: cd /tmp && TMPDIR=/tmp timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE -d <dir> -o run "
        f"--output-format csv -- {pmc_txt}",
        f"          (the same with --pmc WRITE_SIZE)",
        f"made by: python -m block_quantized_weight_gemv_amd.rocprof decode --out <dir> (GEMV kernel source {sha})",
        "",
        f"calibration ({COPY_KERNEL}, {COPY_BYTES >> 20} MiB read + {COPY_BYTES >> 20} MiB written per dispatch): "
        + ", ".join(f"{c} x {fac[c]:.4f}" for c in fac),
        "",
        "kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes/launch (calibrated) | "
        "algorithmic bytes/launch | ratio",
        "---|---|---|---|---|---|---",
    ]
    traffic = {}
    for k in sorted(counters["FETCH_SIZE"]):
        if not k.startswith("gemv_kernel"):
            continue
        f = counters["FETCH_SIZE"][k]["mean"]
        w = counters["WRITE_SIZE"].get(k, {"mean": 0.0})["mean"]
        hbm = f * 1024.0 * fac["FETCH_SIZE"] + w * 1024.0 * fac["WRITE_SIZE"]
        alg = per_kernel.get(k, {}).get("bytes_per_launch")
        ratio = f"{hbm / alg:.3f}" if alg else "-"
        tl.append(f"{k} | {counters['FETCH_SIZE'][k]['dispatches']} | {f:.1f} | {w:.1f} | {hbm:.0f} | "
                  f"{alg if alg else '-'} | {ratio}")
        traffic[f"decode:{k}"] = {"source_sha": sha, "hbm_bytes_per_launch": round(hbm),
                                  "fetch_kib": f, "write_kib": w, "factors": fac}
    with open(os.path.join(out, "decode_pass_hbm_traffic.txt"), "w") as fh:
        fh.write("\n".join(tl) + "\n")
    with open(os.path.join(out, "traffic.json"), "w") as fh:
        json.dump(traffic, fh, indent=1, sort_keys=True)
    print("[harness] wrote", out, flush=True)
    return 0


def single(workload: str, out: str, steps: int, warmup: int) -> int:
    """Trace and FETCH_SIZE/WRITE_SIZE passes of bench.py --workload W."""
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    tag = workload.replace(":", "_m").replace("/", "_")
    args = ["--workload", workload, "--steps", str(steps), "--warmup", str(warmup)]
    t0 = time.time()
    cmd = bench_cmd(args)
    print("[harness] untraced bench:", " ".join(cmd), flush=True)
    rc = _run(cmd, os.path.join(out, tag + ".bench.log"), 300)
    plain = _bench_json(os.path.join(out, tag + ".bench.log"))
    print(f"[harness] untraced bench rc={rc} ({time.time() - t0:.0f} s)", flush=True)
    if rc != 0 or plain is None:
        return rc or 3
    cmd = trace_cmd(os.path.join(out, tag + ".trace"), args)
    print("[harness] kernel trace:", " ".join(cmd), flush=True)
    rc = _run(cmd, os.path.join(out, tag + ".trace.log"), 300)
    print(f"[harness] kernel trace rc={rc} ({time.time() - t0:.0f} s)", flush=True)
    if rc != 0 and _bench_json(os.path.join(out, tag + ".trace.log")) is None:
        return rc
    tr = summarize_trace(_find(os.path.join(out, tag + ".trace"), "kernel_trace.csv"))
    counters = {}
    multi = (plain.get("M") or 1) > 1
    passes = ("FETCH_SIZE", "WRITE_SIZE") + (("MfmaUtil", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "VALUBusy") if multi else ())
    for c in passes:
        cmd = pmc_cmd(c, os.path.join(out, tag + "." + c), ["--workload", workload, "--steps", "10", "--warmup", "2"])
        print(f"[harness] counter pass {c}:", " ".join(cmd), flush=True)
        rc = _run(cmd, os.path.join(out, tag + "." + c + ".log"), 90)
        print(f"[harness] counter pass {c} rc={rc}", flush=True)
        if rc != 0:
            return rc
        counters[c] = summarize_counter(_find(os.path.join(out, tag + "." + c), "counter_collection.csv"), c)
    fac = None
    tj = os.path.join(out, "traffic.json")
    if os.path.exists(tj):
        with open(tj) as fh:
            ent = next(iter(json.load(fh).values()), None)
        fac = ent["factors"] if ent else None
    # the kernel with the most time: the one the workload times
    k = max((n for n in tr if n.startswith(("gemm_", "gemv_", "dequant_"))),
            key=lambda n: tr[n]["calls"] * tr[n]["mean_us"])
    d = tr[k]
    f = counters["FETCH_SIZE"].get(k, {"mean": 0.0})["mean"]
    w = counters["WRITE_SIZE"].get(k, {"mean": 0.0})["mean"]
    # algorithmic bytes per call: the packed weights (GEMV, GEMM), or the
    # blocks read plus the fp32 written (dequantisation)
    wb = plain.get("weight_bytes") or ((plain.get("bytes_read") or 0) + (plain.get("bytes_written") or 0)) or None
    lines = [f"# bench.py --workload {workload}: {plain.get('type')} {plain.get('rows')} x {plain.get('cols')}, "
             f"M = {plain.get('M')}, under rocprofv3",
             "",
             f"command: cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
             f"python bench.py {' '.join(args)}",
             f"counters: cd /tmp && TMPDIR=/tmp timeout -s KILL 90 rocprofv3 --pmc FETCH_SIZE -d <dir> -o run "
             f"--output-format csv -- python bench.py --workload {workload} --steps 10 --warmup 2 (and "
             + ", ".join(passes[1:]) + ", one pass each)",
             f"made by: python -m block_quantized_weight_gemv_amd.rocprof single --workload {workload} --out <dir>",
             "",
             f"kernel: {k}",
             f"calls {d['calls']}, mean {d['mean_us']:.3f} us, min {d['min_us']:.3f} us, max {d['max_us']:.3f} us, "
             f"launch shapes (workgroups x threads: count) "
             + ", ".join(f"{sh}: {n}" for sh, n in sorted(d["workgroups_x_threads"].items())),
             (f"steady calls (from 100 ms after the first): {d['steady_calls']}, mean {d['steady_mean_us']:.3f} us"
              + (f" = {wb / d['steady_mean_us'] / 1e3:.1f} GB/s" + (" of packed weights" if plain.get("weight_bytes")
                                                                      else " read + written") if wb else "")
              if d.get("steady_mean_us") else "steady calls (from 100 ms after the first): none"),
             f"untraced bench: {plain.get('us_per_call')} us per call (hipGraph replay after >= 200 ms of replays, "
             f"median of {plain.get('repeats')} repeats), "
             f"{plain.get('GB_per_s')} GB/s {'of packed weights' if plain.get('weight_bytes') else 'read + written'} "
             f"({plain.get('pct_hbm_peak')} % of 8 TB/s)"
             + (f", {plain.get('TFLOP_per_s')} TFLOP/s" if plain.get("TFLOP_per_s") else ""),
             f"FETCH_SIZE {f:.1f} KiB, WRITE_SIZE {w:.1f} KiB per dispatch"]
    # kernels launched once per call beside it (the untraced time covers them too)
    for n in sorted(n for n in tr if n != k and tr[n]["calls"] == d["calls"]):
        lines.append(f"also launched once per call: {n}: mean {tr[n]['mean_us']:.3f} us, launch shapes "
                     + ", ".join(f"{sh}: {c}" for sh, c in sorted(tr[n]["workgroups_x_threads"].items())))
    if fac:
        hbm = f * 1024.0 * fac["FETCH_SIZE"] + w * 1024.0 * fac["WRITE_SIZE"]
        lines.append(f"HBM bytes per dispatch (calibrated x {fac['FETCH_SIZE']:.4f} / x {fac['WRITE_SIZE']:.4f} "
                     f"with the copy probe of the decode run): {hbm:.0f}; weight bytes {wb}; ratio "
                     f"{hbm / wb:.3f}" if wb else "")
    if multi:
        util = counters["MfmaUtil"].get(k, {"mean": 0.0})["mean"]
        mops = counters["SQ_INSTS_VALU_MFMA_MOPS_BF16"].get(k, {"mean": 0.0})["mean"]
        valu = counters["VALUBusy"].get(k, {"mean": 0.0})["mean"]
        alg = 2.0 * plain["M"] * plain["rows"] * plain["cols"]
        lines.append(f"MfmaUtil {util:.1f} % (matrix-core busy cycles / (GRBM_GUI_ACTIVE x SIMDs)), VALUBusy "
                     f"{valu:.1f} %")
        lines.append(f"bf16 MFMA flops per dispatch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) {mops * 512:.4g}; "
                     f"algorithmic 2*M*rows*cols {alg:.4g}; ratio {mops * 512 / alg:.2f}")
    with open(os.path.join(out, tag + ".txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("[harness] wrote", os.path.join(out, tag + ".txt"), flush=True)
    return 0


def step(workload: str, out: str, steps: int, warmup: int) -> int:
    """Kernel trace of bench.py --workload step:P (one whole decode step per
    call): every kernel's calls per step, mean duration and share of the
    traced time."""
    out = os.path.abspath(out)
    os.makedirs(out, exist_ok=True)
    tag = "decode_step_" + workload.replace(":", "_pos")
    args = ["--workload", workload, "--steps", str(steps), "--warmup", str(warmup)]
    t0 = time.time()
    rc = _run(bench_cmd(args), os.path.join(out, tag + ".bench.log"), 300)
    plain = _bench_json(os.path.join(out, tag + ".bench.log"))
    print(f"[harness] untraced bench rc={rc} ({time.time() - t0:.0f} s)", flush=True)
    if rc != 0 or plain is None:
        return rc or 3
    cmd = trace_cmd(os.path.join(out, tag + ".trace"), args)
    print("[harness] kernel trace:", " ".join(cmd), flush=True)
    rc = _run(cmd, os.path.join(out, tag + ".trace.log"), 300)
    print(f"[harness] kernel trace rc={rc} ({time.time() - t0:.0f} s)", flush=True)
    if rc != 0 and _bench_json(os.path.join(out, tag + ".trace.log")) is None:
        return rc
    tr = summarize_trace(_find(os.path.join(out, tag + ".trace"), "kernel_trace.csv"))
    calls_per_step = steps + warmup + 1  # timed and warm-up replays, and the eager run before the capture
    rows = [(k, d) for k, d in tr.items() if not k.startswith("at::") and "rocclr" not in k]
    total = sum(d["calls"] * d["mean_us"] for _, d in rows)
    model = "Llama-2-7B" if workload.startswith("step7b") else "TinyLlama-1.1B"
    lines = [f"# bench.py --workload {workload}: one decode step ({model} shapes) per call, under rocprofv3",
             "",
             f"command: cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats -d <dir> -o run --output-format csv -- "
             f"python bench.py {' '.join(args)}",
             f"made by: python -m block_quantized_weight_gemv_amd.rocprof step --workload {workload} --out <dir>",
             "",
             f"untraced bench: {plain.get('ms_per_token')} ms per token ({plain.get('tokens_per_s')} tokens/s) at "
             f"position {plain.get('position')}; the traced run's kernels (launch gaps excluded):",
             "",
             f"{'kernel':58s} {'per step':>8s} {'mean us':>8s} {'share':>6s}"]
    for k, d in sorted(rows, key=lambda kd: -kd[1]["calls"] * kd[1]["mean_us"]):
        share = 100.0 * d["calls"] * d["mean_us"] / total if total else 0.0
        if share < 0.2:
            continue
        lines.append(f"{k[:58]:58s} {d['calls'] / calls_per_step:8.1f} {d['mean_us']:8.2f} {share:5.1f}%")
    lines.append("")
    lines.append(f"kernel time per step (traced): {total / calls_per_step:.1f} us")
    with open(os.path.join(out, tag + ".txt"), "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("[harness] wrote", os.path.join(out, tag + ".txt"), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    d = sub.add_parser("decode", help="trace + HBM counters of the default decode bench")
    d.add_argument("--out", required=True)
    d.add_argument("--steps", type=int, default=50)
    d.add_argument("--warmup", type=int, default=10)
    g = sub.add_parser("single", help="trace + HBM counters of one bench.py --workload")
    g.add_argument("--workload", required=True)
    g.add_argument("--out", required=True)
    g.add_argument("--steps", type=int, default=30)
    g.add_argument("--warmup", type=int, default=4)
    t = sub.add_parser("step", help="kernel trace of one bench.py --workload step:P")
    t.add_argument("--workload", default="step:511")
    t.add_argument("--out", required=True)
    t.add_argument("--steps", type=int, default=20)
    t.add_argument("--warmup", type=int, default=3)
    s = sub.add_parser("summarize", help="summarize an existing kernel trace CSV")
    s.add_argument("trace_csv")
    a = ap.parse_args(argv)
    if a.cmd == "decode":
        return decode(a.out, a.steps, a.warmup)
    if a.cmd == "single":
        return single(a.workload, a.out, a.steps, a.warmup)
    if a.cmd == "step":
        return step(a.workload, a.out, a.steps, a.warmup)
    print(json.dumps(summarize_trace(a.trace_csv), indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
