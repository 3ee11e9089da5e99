"""Benchmark: one fp32 GPT-2 training step (forward + backward + AdamW) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 124m] [--gpus 1]

A step is gpt2_forward (ids already resident in HBM) + gpt2_zero_grad +
gpt2_backward + gpt2_update, enqueued on one HIP stream.  W untimed steps,
then K timed steps between two device synchronizations (`value`).  The same
number of steps is then run again with every launch bracketed by HIP events
on the step's stream (the library's per-launch timing): that gives each
kernel's average duration and the roofline fraction of the dominant kernel
without perturbing the first timing.  Last, the CPU oracle is timed on a
bounded sample of the same workload.  Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "train tokens/sec (fwd+bwd+AdamW) GPT-2 124M B=4 T=1024 fp32; % MFMA/HBM roofline"
PEAK_MFMA_FP32_TFLOPS = 157.3   # MI355X dense fp32 matrix peak
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E peak
PEAK_MFMA_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak

# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc runs
# (FETCH_SIZE, then WRITE_SIZE) of this script with --copy-calibration; the
# file records a hash of the sources that decide that kernel's launches, and
# the figure is reported only while they are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_gpt2_124m_b4_t1024.json")
# Per-kernel launch durations from a rocprofv3 --kernel-trace --stats run of
# this script (no counters, so the kernels run as in an ordinary step).
KTRACE_FILE = os.path.join(ROOT, "profiles", "kernel_trace_gpt2_124m_b4_t1024.json")
KERNEL_SOURCES = ["gemm.hip", "gemm.h", "attention.hip", "attention.h", "kernels.hip", "kernels.h", "common.h",
                  "gpt2.hip"]


def sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "transformer_lm_step_flat_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str, config: str):
    """Bytes per launch of `kernel` from the committed counter summary, or None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("kernel") != kernel or t.get("config") != config or t.get("sources_sha256") != sources_sha256():
        return None
    return t.get("hbm_bytes_per_launch")


def traced_duration(kernel: str, config: str):
    """Average launch duration (ms) of `kernel` in the committed kernel-trace
    summary, or None when it is missing or its sources have changed since."""
    try:
        with open(KTRACE_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("config") != config or t.get("sources_sha256") != sources_sha256():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k["avg_ms"]


def host_cpu():
    """CPU model, online CPUs and the CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"cpu_model": model, "nproc_online": os.cpu_count(), "affinity_cpus": affinity,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def copy_calibration(mib: int):
    """A plain elementwise copy of known size (reads and writes mib MiB each),
    for scaling the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 3 x {mib} MiB read + {mib} MiB written (elementwise mul by 1)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, T_sample: int):
    """The oracle (as it is) on one sequence of T_sample ids of the same
    workload: one full step, forward + backward + AdamW over all parameters."""
    import numpy as np
    import oracle
    from transformer_lm_step_flat_amd import synth
    oracle.build(force=False)
    tensors = synth.init_params(cfg)
    p = oracle.pack(cfg, tensors)
    del tensors
    inp, tgt = synth.batch(cfg, step=0, B=1, T=T_sample)
    R = oracle.RefModel(cfg, 1, T_sample)
    g, m, v = np.zeros_like(p), np.zeros_like(p), np.zeros_like(p)
    t0 = time.perf_counter()
    R.forward(p, inp, tgt)
    R.backward(p, g)
    oracle.adamw(p, g, m, v, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1)
    dt = time.perf_counter() - t0
    R.close()
    return dict({"value": T_sample / dt, "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
                 "sample": f"one full step (forward, backward, AdamW over all {p.size} parameters) of the same model "
                           f"on 1 sequence x {T_sample} ids of the same seeded stream, float64; {dt:.1f} s wall"},
                **host_cpu())


def _short_kernel_name(n: str) -> str:
    n = n.replace("(anonymous namespace)::", "")
    if n.startswith("void "):
        n = n[5:]
    i = n.find("(")
    return n[:i] if i > 0 else n


def pmc_summary(fetch_csv: str, write_csv: str, steps: int, copy_mib: int, command: str, config: str):
    """Summarise two rocprofv3 --pmc runs of this script (FETCH_SIZE, then
    WRITE_SIZE, each with --copy-calibration): per-kernel HBM bytes per
    dispatch scaled by what the counters read for the plain copy of known
    size, and per-kernel durations from the dispatch timestamps (counter
    collection serialises dispatches, so each is a kernel alone).  Writes
    the Markdown summary to stdout and the dominant kernel's bytes per
    launch to TRAFFIC_FILE."""
    import collections
    import csv

    def load(path, counter):
        per = collections.defaultdict(list)
        dur = collections.defaultdict(list)
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            k = _short_kernel_name(r["Kernel_Name"])
            per[k].append(float(r["Counter_Value"]))
            dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-6)
        return per, dur

    fetch, dur = load(fetch_csv, "FETCH_SIZE")
    write, _ = load(write_csv, "WRITE_SIZE")
    # the copy: the elementwise kernel with the largest write (the fill of its source writes but does not read)
    copy_kib = copy_mib * 1024.0
    cands = [k for k in write if "elementwise" in k]
    ck = max(cands, key=lambda k: max(fetch.get(k, [0])))
    f_scale = copy_kib / max(fetch[ck])
    w_scale = copy_kib / max(write[ck])
    # (the step's kernels: not the copy, the runtime's fills or the matrix-unit peak probe)
    lib_kernels = [k for k in dur if "elementwise" not in k and "rocclr" not in k and "probe" not in k]
    tot = {k: sum(dur[k]) for k in lib_kernels}
    dom = max(tot, key=tot.get)
    rows = []
    for k in sorted(lib_kernels, key=lambda k: -tot[k]):
        n = len(dur[k])
        fb = sum(fetch[k]) / n * 1024 * f_scale
        wb = sum(write.get(k, [0])) / max(1, len(write.get(k, []))) * 1024 * w_scale
        rows.append((k, n, sum(dur[k]) / n, fb, wb))
    print(f"# HBM traffic and kernel durations under counter collection: {config}\n")
    print(f"Command (each pass its own run): `{command}`\n")
    print(f"Copy calibration: {copy_mib} MiB read and written by `{ck}`; FETCH_SIZE reads "
          f"{max(fetch[ck]):.0f} KiB (scale {f_scale:.3f}), WRITE_SIZE {max(write[ck]):.0f} KiB (scale {w_scale:.3f}).\n")
    print("| kernel | dispatches | avg ms | HBM read MB / dispatch | HBM write MB / dispatch |")
    print("|---|---:|---:|---:|---:|")
    for k, n, ms, fb, wb in rows:
        print(f"| `{k}` | {n} | {ms:.4f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} |")
    k, n, ms, fb, wb = next(r for r in rows if r[0] == dom)
    out = {"kernel": dom, "config": config, "sources_sha256": sources_sha256(), "dispatches": n,
           "hbm_read_bytes_per_launch": fb, "hbm_write_bytes_per_launch": wb,
           "hbm_bytes_per_launch": fb + wb, "fetch_scale": f_scale, "write_scale": w_scale,
           "command": command}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"\nDominant kernel `{dom}`: {(fb + wb) / 1e6:.1f} MB of HBM traffic per launch "
          f"(read {fb / 1e6:.1f}, write {wb / 1e6:.1f}); written to {os.path.relpath(TRAFFIC_FILE, ROOT)}.")


def kt_summary(stats_csv: str, command: str, config: str):
    """Summarise a rocprofv3 --kernel-trace --stats run of this script
    (its kernel_stats.csv): per kernel, launches and average duration.
    Writes Markdown to stdout and the per-kernel averages to KTRACE_FILE (the
    headline configuration, whose figures the bench line uses) or, for another
    configuration, to profiles/kernel_trace_<workload>.json."""
    import csv
    rows = []
    for r in csv.DictReader(open(stats_csv)):
        name = _short_kernel_name(r["Name"])
        rows.append((name, int(r["Calls"]), float(r["TotalDurationNs"]) * 1e-6, float(r["AverageNs"]) * 1e-6,
                     float(r["MinNs"]) * 1e-6, float(r["MaxNs"]) * 1e-6))
    rows.sort(key=lambda x: -x[2])
    print(f"# Kernel durations from a kernel trace (no counters): {config}\n")
    print(f"Command: `{command}`\n")
    print("| kernel | launches | total ms | avg ms | min ms | max ms |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, n, tot, avg, mn, mx in rows:
        print(f"| `{name}` | {n} | {tot:.3f} | {avg:.4f} | {mn:.4f} | {mx:.4f} |")
    out = {"config": config, "sources_sha256": sources_sha256(), "command": command,
           "kernels": {name: {"launches": n, "avg_ms": avg, "min_ms": mn, "max_ms": mx}
                       for name, n, tot, avg, mn, mx in rows}}
    names = {"124m_b16": "gpt2_124m_b16_t1024", "xl": "gpt2_xl_b4_t1024"}
    path = KTRACE_FILE if config == "124m" else os.path.join(
        ROOT, "profiles", f"kernel_trace_{names.get(config, config)}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(f"\nPer-kernel averages written to {os.path.relpath(path, ROOT)}.")


def sq_summary(sq_csv: str, command: str, config: str):
    """Summarise a rocprofv3 --pmc run with SQ_BUSY_CYCLES, SQ_VALU_MFMA_BUSY_CYCLES,
    SQ_INSTS_MFMA, SQ_WAVES and GRBM_GUI_ACTIVE: per kernel, the share of busy
    cycles in which the SIMDs' matrix units were busy and the shader clock.
    MI355X counts: SQ_BUSY_CYCLES summed over 32 shader engines,
    SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs, GRBM_GUI_ACTIVE over 8 XCDs."""
    import collections
    import csv
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(dict)
    for r in csv.DictReader(open(sq_csv)):
        k = _short_kernel_name(r["Kernel_Name"])
        disp[k][r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
    print(f"# Matrix-unit busy share and clock under counter collection: {config}\n")
    print(f"Command: `{command}`\n")
    print("| kernel | dispatches | avg ms | clock GHz | MFMA busy / busy cycles | MFMA instr / dispatch |")
    print("|---|---:|---:|---:|---:|---:|")
    rows = []
    for k, c in acc.items():
        n = len(disp[k])
        secs = sum(disp[k].values())
        if c.get("SQ_BUSY_CYCLES", 0) <= 0 or secs <= 0:
            continue
        busy = c["SQ_BUSY_CYCLES"] / 32
        rows.append((secs, k, n, secs / n * 1e3, c["GRBM_GUI_ACTIVE"] / 8 / secs / 1e9,
                     c["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / busy, c["SQ_INSTS_MFMA"] / n))
    for _, k, n, ms, ghz, fr, mi in sorted(rows, reverse=True):
        if mi > 0:
            print(f"| `{k}` | {n} | {ms:.4f} | {ghz:.2f} | {100 * fr:.1f}% | {mi:.3g} |")


def measured_peaks(torch, gpt2, copy_mib=1024, reps=5):
    """The fp32 matrix-core rate (calibration kernel of back-to-back MFMAs on
    every CU) and the HBM copy rate (copy_mib MiB read and written) this
    device reaches, best of `reps` timed launches each."""
    out = torch.zeros(1, device="cuda")
    n = copy_mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best_mfma, best_copy = 0.0, 0.0
    gpt2.probe_mfma(out, 200)
    gpt2.probe_copy(dst, src)
    for _ in range(reps):
        e0.record()
        flops = gpt2.probe_mfma(out, 2000)
        e1.record()
        torch.cuda.synchronize()
        best_mfma = max(best_mfma, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        e0.record()
        gpt2.probe_copy(dst, src)
        e1.record()
        torch.cuda.synchronize()
        best_copy = max(best_copy, 8.0 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return {"mfma_fp32_tflops": best_mfma, "hbm_copy_gbs": best_copy, "copy_mib": copy_mib}


def decode_bench(torch, M, di, B, T, prefill, steps):
    """Greedy decoding with the key/value cache: a forward over the batch as
    the prefill, then `steps` decode steps from position `prefill`, each
    step's ids feeding the next (no host round trip).  Returns tokens/s and
    the per-kernel HBM rates of a second, event-bracketed pass."""
    M.forward(di, None)
    first = di.view(B, T)[:, prefill].contiguous()
    bufs = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(2)]

    def run():
        tok = first
        for i in range(steps):
            tok = M.decode_step(tok, prefill + i, None, bufs[i % 2])

    run()  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    M.profile_enable(True)
    run()
    prof = M.profile_read()
    M.profile_enable(False)
    by = {}
    for e in prof:
        k = e["name"].partition("|")[0]
        a = by.setdefault(k, dict(name=k, launches=0, ms=0.0, bytes=0.0))
        for f in ("launches", "ms", "bytes"):
            a[f] += e[f]
    step_bytes = sum(e["bytes"] for e in by.values()) / steps
    ev_ms = sum(e["ms"] for e in by.values()) / steps
    kernels = sorted(({"name": e["name"], "launches_per_step": e["launches"] / steps,
                       "ms_per_step": e["ms"] / steps, "GBs": e["bytes"] / e["ms"] * 1e-6,
                       "frac_hbm": e["bytes"] / e["ms"] * 1e-6 / PEAK_HBM_GBS} for e in by.values()),
                     key=lambda k: -k["ms_per_step"])
    return {"tokens_per_s": B / (ms * 1e-3), "ms_per_step": ms, "B": B, "prefill": prefill,
            "steps": steps, "sampling": "greedy",
            "algorithmic_bytes_per_step": step_bytes,
            "achieved_GBs": step_bytes / (ms * 1e-3) / 1e9, "frac_hbm": step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "kernel_ms_per_step_with_events": ev_ms, "kernels": kernels[:8]}


def bf16_bench(torch, gpt2, M, step, first, steps, warmup, B, T):
    """The same training step with bfloat16 linear-layer products (fp32
    master weights, gradients, moments and activations): tokens/s and the
    dominant kernel's rate against the dense bf16 matrix peak."""
    M.set_matmul_precision(gpt2.GPT2_BF16)
    for i in range(warmup):
        step(first + i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(steps):
        step(first + warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    M.profile_enable(True)
    for i in range(steps):
        step(first + warmup + steps + i)
    prof = M.profile_read()
    M.profile_enable(False)
    M.set_matmul_precision(gpt2.GPT2_FP32)
    by = {}
    for e in prof:
        k = e["name"].partition("|")[0]
        a = by.setdefault(k, dict(name=k, launches=0, ms=0.0, flops=0.0))
        for f in ("launches", "ms", "flops"):
            a[f] += e[f]
    bf = [e for e in by.values() if "bf16" in e["name"]]
    d = max(bf, key=lambda e: e["ms"])
    achieved = d["flops"] / d["ms"] * 1e-9
    return {"tokens_per_s": B * T / (ms * 1e-3), "ms_per_step": ms, "steps": steps,
            "bf16_gemm_ms_per_step": sum(e["ms"] for e in bf) / steps,
            "dominant": {"kernel": d["name"], "launches_per_step": d["launches"] / steps,
                         "avg_launch_ms": d["ms"] / d["launches"], "achieved_tflops": achieved,
                         "peak_tflops": PEAK_MFMA_BF16_TFLOPS, "frac": achieved / PEAK_MFMA_BF16_TFLOPS}}


def ln_sweep(C=768, rows=(4096, 16384), reps=50):
    """The LayerNorm kernels on their own: `reps` back-to-back launches of
    the library's forward and backward (accumulating; its kernel and the
    column sums of dw and db) at N rows of C, replayed from a graph and timed
    with events around the replay, against the 8 TB/s HBM peak.  Bytes
    are the algorithmic ones: forward reads x and writes y (8 N C) plus the
    row statistics; backward reads dy, x and the dx it accumulates into and
    writes dx (16 N C)."""
    import torch
    from transformer_lm_step_flat_amd import gpt2
    gpt2.lib()
    print(f"LayerNorm kernels alone, C = {C}: {reps} launches back to back, replayed from a captured graph, "
          f"HIP events around the replay:")
    print("| rows N | forward us | forward GB/s | % of 8 TB/s | backward us | backward GB/s | % of 8 TB/s |")
    print("|---:|---:|---:|---:|---:|---:|---:|")
    for N in rows:
        g = torch.Generator(device="cuda").manual_seed(N)
        x = torch.randn(N * C, device="cuda", generator=g)
        dy = torch.randn(N * C, device="cuda", generator=g)
        w = torch.randn(C, device="cuda", generator=g)
        b = torch.randn(C, device="cuda", generator=g)
        y, dx = torch.empty_like(x), torch.zeros_like(x)
        mu, rs = torch.empty(N, device="cuda"), torch.empty(N, device="cuda")
        dw, db = torch.zeros(C, device="cuda"), torch.zeros(C, device="cuda")

        def timed(fn):
            # the launches are captured in a graph and replayed, so that the
            # host's per-call cost (argument checks, ctypes) does not pace them
            fn()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                for _ in range(reps):
                    fn()
            gr.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            gr.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps * 1e3

        tf = timed(lambda: gpt2.layernorm_forward(y, mu, rs, x, w, b, N, C))
        tb = timed(lambda: gpt2.layernorm_backward(dx, dw, db, dy, x, w, mu, rs, N, C, True))
        bf, bb = 8.0 * N * C + 8.0 * N, 16.0 * N * C + 8.0 * N
        print(f"| {N} | {tf:.2f} | {bf / tf * 1e-3:.0f} | {bf / tf * 1e-3 / PEAK_HBM_GBS * 100:.1f} | {tb:.2f} | "
              f"{bb / tb * 1e-3:.0f} | {bb / tb * 1e-3 / PEAK_HBM_GBS * 100:.1f} |", flush=True)


def step_roofline_ms(sites, steps):
    """The step's roofline time in ms: each call site's launches at the slower
    of their matrix bound (FLOPs / fp32 matrix peak) and their HBM bound
    (algorithmic bytes / HBM peak), summed.  Launches at one call site share a
    shape, so the bound of their sums is the sum of their bounds."""
    return sum(max(e["flops"] / (PEAK_MFMA_FP32_TFLOPS * 1e9), e["bytes"] / (PEAK_HBM_GBS * 1e6))
               for e in sites) / steps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="124m")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-events", action="store_true", help="time the steps without per-launch events")
    ap.add_argument("--cpu-sample-tokens", type=int, default=1024)
    ap.add_argument("--decode-steps", type=int, default=64, help="greedy decode steps timed after the training steps")
    ap.add_argument("--decode-prefill", type=int, default=512)
    ap.add_argument("--bf16-steps", type=int, default=10, help="steps timed with bfloat16 linear-layer products")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run a plain copy of MIB MiB (for scaling HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs of this script and exit")
    ap.add_argument("--pmc-command", default="", help="the profiled command, quoted in the summary")
    ap.add_argument("--sq-summary", metavar="SQ_CSV", help="summarise a rocprofv3 --pmc run of SQ counters and exit")
    ap.add_argument("--kt-summary", metavar="STATS_CSV",
                    help="summarise a rocprofv3 --kernel-trace --stats run (kernel_stats.csv) and exit")
    ap.add_argument("--ln-sweep", action="store_true", help="time the LayerNorm kernels alone and exit")
    args = ap.parse_args()
    if args.ln_sweep:
        ln_sweep()
        return
    if args.kt_summary:
        kt_summary(args.kt_summary, args.pmc_command, args.config)
        return
    if args.sq_summary:
        sq_summary(args.sq_summary, args.pmc_command, args.config)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.steps, args.copy_calibration or 1024,
                    args.pmc_command, args.config)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the data-parallel path over several "
              "GPUs is designed but not built; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_lm_step_flat_amd import gpt2, synth

    cfg = synth.config(args.config)
    B, T = cfg["B"], cfg["T"]
    log(f"building {args.config}: L={cfg['L']} C={cfg['C']} NH={cfg['NH']} V={cfg['V']} B={B} T={T}")
    M = gpt2.Model(cfg, B, T, init_params=gpt2.pack_params(cfg, synth.init_params(cfg), B, T))
    nb = 4
    batches = []
    for i in range(nb):
        inp, tgt = synth.batch(cfg, step=i)
        batches.append((torch.from_numpy(inp.ravel()).cuda(), torch.from_numpy(tgt.ravel()).cuda()))
    torch.cuda.synchronize()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)

    def step(i, want_loss=False):
        di, dt = batches[i % nb]
        loss = M.forward(di, dt, want_loss=want_loss)
        M.zero_grad()
        M.backward()
        M.update(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, t=i + 1)
        return loss

    for i in range(args.warmup):
        step(i)
    M.sync()
    log(f"warmup done ({args.warmup} steps)")

    # timed region: no instrumentation but one event between steps on the step's stream
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step(args.warmup + i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    dt_s = time.perf_counter() - t0
    M.sync()
    loss = float(M.act("loss")[0].item())
    ms = dt_s / args.steps * 1e3
    tok_s = B * T * args.steps / dt_s
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    step_ms = {"mean": sum(per_step) / len(per_step), "median": per_step[len(per_step) // 2],
               "min": per_step[0], "max": per_step[-1]}
    log(f"timed {args.steps} steps: {ms:.2f} ms/step, {tok_s:.0f} tokens/s, last loss {loss:.4f} "
        f"(per step: median {step_ms['median']:.2f}, min {step_ms['min']:.2f}, max {step_ms['max']:.2f} ms)")
    peaks = measured_peaks(torch, gpt2)
    log(f"measured on this device: fp32 matrix-core {peaks['mfma_fp32_tflops']:.1f} TFLOP/s, "
        f"HBM copy {peaks['hbm_copy_gbs']:.0f} GB/s")

    # the same steps again, each launch bracketed by HIP events on the step's stream
    kernels, roofline, ms_ev, sites, losses = [], None, None, [], []
    if not args.no_events:
        M.profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            # the loss of each step (read back, so this pass also waits once per step)
            losses.append(step(args.warmup + args.steps + i, want_loss=True))
        torch.cuda.synchronize()
        ms_ev = (time.perf_counter() - t0) / args.steps * 1e3
        prof = M.profile_read()
        M.profile_enable(False)
        log(f"timed {args.steps} steps with per-launch events: {ms_ev:.2f} ms/step")
        by_kernel = {}
        for e in prof:
            k, _, site = e["name"].partition("|")
            a = by_kernel.setdefault(k, dict(name=k, launches=0, ms=0.0, flops=0.0, bytes=0.0))
            for f in ("launches", "ms", "flops", "bytes"):
                a[f] += e[f]
            sites.append(dict(e, kernel=k, site=site))
        tot = sum(e["ms"] for e in by_kernel.values())

        def rate(e):
            bound = "mfma" if e["flops"] > 0 else "hbm"
            r = (e["flops"] / e["ms"] * 1e-9) if bound == "mfma" else (e["bytes"] / e["ms"] * 1e-6)
            return bound, r, (PEAK_MFMA_FP32_TFLOPS if bound == "mfma" else PEAK_HBM_GBS)

        for e in sorted(by_kernel.values(), key=lambda e: -e["ms"]):
            bound, r, peak = rate(e)
            kernels.append({"name": e["name"], "launches_per_step": e["launches"] / args.steps,
                            "ms_per_step": e["ms"] / args.steps, "share": e["ms"] / tot, "bound": bound,
                            "achieved": r, "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": r / peak})
        log("per kernel (summed over call sites):")
        for k in kernels:
            log(f"  {k['name']:<38s} {k['launches_per_step']:6.1f}/step {k['ms_per_step']:8.3f} ms/step "
                f"{100 * k['share']:5.1f}%  {k['achieved']:9.1f} {k['unit']} ({100 * k['frac']:.1f}% of peak)")
        log("per call site:")
        for e in sorted(sites, key=lambda e: -e["ms"]):
            bound, r, peak = rate(e)
            log(f"  {e['site']:<14s} {e['kernel']:<38s} {e['launches'] / args.steps:6.1f}/step "
                f"{e['ms'] / args.steps:8.3f} ms/step {r:9.1f} {'TFLOP/s' if bound == 'mfma' else 'GB/s'} "
                f"({100 * r / peak:.1f}%)")
        d = max(by_kernel.values(), key=lambda e: e["ms"])
        bound, _, peak = rate(d)
        per_launch = (d["flops"] if bound == "mfma" else d["bytes"]) / d["launches"]
        avg_ms = d["ms"] / d["launches"]
        achieved = per_launch / (avg_ms * 1e-3) / (1e12 if bound == "mfma" else 1e9)
        all_flops = sum(e["flops"] for e in by_kernel.values()) / args.steps
        roof_ms = step_roofline_ms(sites, args.steps)
        alg_bytes = d["bytes"] / d["launches"]
        traffic = measured_traffic(d["name"], args.config)
        traced_ms = traced_duration(d["name"], args.config)
        roofline = {"bound": bound, "achieved": achieved, "peak": peak,
                    "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": achieved / peak,
                    "traffic": traffic,
                    "kernel": d["name"], "avg_launch_ms": avg_ms, "launches_per_step": d["launches"] / args.steps,
                    "algorithmic_per_launch": per_launch,
                    "algorithmic_bytes_per_launch": alg_bytes,
                    "traffic_over_algorithmic_bytes": None if traffic is None else traffic / alg_bytes,
                    "kernel_trace_avg_launch_ms": traced_ms,
                    "frac_by_kernel_trace": None if traced_ms is None else
                    per_launch / (traced_ms * 1e-3) / (1e12 if bound == "mfma" else 1e9) / peak,
                    "step_flops": all_flops,
                    "step_mfma_frac": all_flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_FP32_TFLOPS,
                    "step_roofline_ms": roof_ms, "step_roofline_frac": roof_ms / ms,
                    "frac_of_measured_peak": achieved / (peaks["mfma_fp32_tflops"] if bound == "mfma"
                                                         else peaks["hbm_copy_gbs"])}
        log(f"step roofline: {roof_ms:.2f} ms (each call site at max(FLOPs / matrix peak, bytes / HBM peak)), "
            f"{100 * roof_ms / ms:.1f}% of the measured {ms:.2f} ms/step")

    decode = None
    if args.decode_steps > 0 and args.decode_prefill + args.decode_steps <= T:
        decode = decode_bench(torch, M, batches[0][0], B, T, args.decode_prefill, args.decode_steps)
        log(f"decode: {decode['tokens_per_s']:.0f} tokens/s ({decode['ms_per_step']:.3f} ms per step of {B} tokens, "
            f"{decode['achieved_GBs']:.0f} GB/s of algorithmic traffic, {100 * decode['frac_hbm']:.1f}% of HBM peak)")
        for k in decode["kernels"]:
            log(f"  {k['name']:<34s} {k['launches_per_step']:5.1f}/step {k['ms_per_step']:7.4f} ms/step "
                f"{k['GBs']:7.0f} GB/s")

    bf16 = None
    if args.bf16_steps > 0:
        bf16 = bf16_bench(torch, gpt2, M, step, 2 * args.steps + args.warmup, args.bf16_steps, 2, B, T)
        log(f"bf16 products: {bf16['tokens_per_s']:.0f} tokens/s ({bf16['ms_per_step']:.2f} ms/step; bf16 GEMMs "
            f"{bf16['bf16_gemm_ms_per_step']:.2f} ms/step with events; {bf16['dominant']['kernel']} at "
            f"{bf16['dominant']['achieved_tflops']:.0f} TFLOP/s, {100 * bf16['dominant']['frac']:.1f}% of the bf16 peak)")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on a {args.cpu_sample_tokens}-id sample ...")
        cpu = cpu_baseline(cfg, args.cpu_sample_tokens)
        log(f"  oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    ids = "Zipf(1.1) ids" if cfg.get("tokens") == "zipf" else "uniform ids"
    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"GPT-2 {args.config} fp32 training step: L={cfg['L']} C={cfg['C']} NH={cfg['NH']} "
                               f"V={cfg['V']} (head padded to {cfg['Vp']}), B={B}, T={T}, seeded N(0,0.02) init, "
                               f"{ids}, AdamW lr 1e-4",
                   "B": B, "T": T},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "last_loss": loss,
        "losses_of_event_pass": losses,
        "step_ms": step_ms,
        "measured_peaks": peaks,
        "ms_per_step_with_events": ms_ev,
        "kernels": kernels[:16],
        "decode": decode,
        "bf16_products": bf16,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
