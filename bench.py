#!/usr/bin/env python3
"""Benchmark of libmi_attn's attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward pass (one kernel launch) over the whole workload, with
Q, K, V and the outputs resident in HBM.  The K timed steps run as 5 batches
of back-to-back launches (each batch one HIP graph replay), with a HIP event
recorded on the launch stream before the first batch and after every batch:
the timed region is exactly the K steps, `ms_per_step` is its total over K,
and `ms_per_step_median_batch` the median of the 5 batches' per-launch
times.  Host launch overhead is not in the figures; `ms_per_step_eager`
gives the plain per-call rate for context.

Prints one JSON line.  `value` is algorithmic TFLOP/s of the workload:
4 * d * Hq * (visible query/key pairs) per forward.  `roofline` relates the
kernel to the dense fp16/bf16 MFMA peak of MI355X; `traffic` (HBM bytes per
launch) and `mfma_busy` come from rocprofv3 counters committed under
profiles/ and are reported only while the kernel source still hashes to the
value recorded with them.  `cpu_baseline` times the fp64 CPU oracle on the
host cores over the same workload and also yields the parity errors of this
run's GPU output.  `memory` compares torch's peak allocation during the
calls with the inputs and outputs (the library allocates nothing, so no
Lq x Lk buffer can exist).

    python bench.py --summarize-counters DIR [--workload NAME] [--write-record]

reads the CSV files of the rocprofv3 runs listed in the summary it prints
(kernel trace, HBM read and write request counters, MFMA busy cycles) from
DIR and prints a Markdown summary; --write-record also stores the per-launch
figures in the counter record under profiles/.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6}   # MI355X dense MFMA, per GPU
PEAK_HBM_GBS = 8000.0                            # MI355X HBM3E, per GPU
# what the hot kernel is built from: its template, instantiations and flags
KERNEL_SRCS = [os.path.join(ROOT, "exact_attention_61_amd", *parts) for parts in
               (("csrc", "attn_fwd_mfma.hpp"), ("csrc", "attn_fwd_mfma_d64.hip"),
                ("csrc", "attn_fwd_mfma_d128.hip"), ("csrc", "attn_decode.hip"),
                ("csrc", "attn_fwd_mfma_drop_d64.hip"), ("csrc", "attn_fwd_mfma_drop_d128.hip"),
                ("csrc", "rotary.hip"), ("csrc", "mfma_util.hpp"), ("csrc", "common.hpp"),
                ("build.py",))]
DROPOUT_SEED = 2024                              # mask seed of the dropout workloads
SIMDS = 4 * 256                                  # MI355X: 256 CUs x 4 SIMDs
PEAK_CLOCK_HZ = 2.4e9                            # the clock the peaks are quoted at
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_mfma_counters.json")
# What the headline line is quoted on (the workload's own label otherwise).
HEADLINE_METRIC = ("attn fwd TFLOP/s + % of fp16 MFMA peak, B2 H16 N2048 d64 "
                   "causal")


def visible_pairs(w, lengths=None):
    """Number of (query, key) pairs a forward pass must combine, per head."""
    if w.varlen:
        pairs = 0
        for n in lengths:
            pairs += n * (n + 1) // 2 if w.causal else n * n
        return pairs
    lq, lk = w.lq, w.lk
    if not w.causal:
        return w.batch * lq * lk
    per = sum(min(lk, max(0, i + lk - lq + 1)) for i in range(lq))
    return w.batch * per


def algorithmic_bytes(w, inp):
    """Q, K, V read once and O, LSE written once (rotary: Q and K read and
    written once)."""
    esz = {"f16": 2, "bf16": 2, "f32": 4}
    q, k, v = inp["q"], inp["k"], inp["v"]
    if w.rotary:
        return 2 * (q.numel() + k.numel()) * esz[w.in_dtype]
    n_in = (q.numel() + k.numel() + v.numel()) * esz[w.in_dtype]
    rows = q.numel() // w.d
    return n_in + rows * w.d * esz[w.out_dtype] + rows * 4


def kernel_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_counter_record(workload):
    """Per-launch counter figures of the workload from the committed record,
    or None when there is none or the kernel has changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    return rec.get("workloads", {}).get(workload) or None


def load_traffic(workload):
    """HBM bytes per launch from the committed counter record, or None."""
    ent = load_counter_record(workload)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def metric_label(w):
    """The metric string of a workload's line."""
    import workloads
    if w.name == workloads.HEADLINE:
        return HEADLINE_METRIC
    if w.decode:
        return (f"attn decode GB/s (HBM roofline), B{w.batch} Hq{w.hq} Hkv{w.hkv} "
                f"Lq{w.lq} Lk{w.lk} d{w.d} {w.in_dtype}")
    if w.rotary:
        return (f"rotary embedding of Q and K in place, GB/s (HBM roofline), B{w.batch} "
                f"Hq{w.hq} Hkv{w.hkv} L{w.lq} d{w.d} {w.in_dtype}")
    shape = (f"varlen B{w.batch} H{w.hq} max L{w.lq}" if w.varlen else
             f"B{w.batch} Hq{w.hq} Hkv{w.hkv} Lq{w.lq} Lk{w.lk}")
    drop = f" dropout {w.dropout}" if w.dropout else ""
    return (f"attn fwd TFLOP/s + % of {w.in_dtype} MFMA peak, {shape} d{w.d}"
            f"{' causal' if w.causal else ''}{drop}")


def batch_sizes(steps, batches=5):
    """Split `steps` launches into at most `batches` nearly equal batches."""
    nb = max(1, min(batches, steps))
    return [steps // nb + (1 if i < steps % nb else 0) for i in range(nb)]


def engine_clock_mhz(dev_index):
    """Peak engine clock the HIP runtime reports (hipDeviceAttributeClockRate,
    kHz), through the runtime library this process already loaded."""
    import ctypes
    try:
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            return None
        hip = ctypes.CDLL(path)
        val = ctypes.c_int(0)
        # hipDeviceAttributeClockRate is entry 5 of hipDeviceAttribute_t
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, int(dev_index)) != 0:
            return None
        return val.value / 1000.0
    except OSError:
        return None


def cold_launch_ms(step, dev, launches=20, flush_mib=512):
    """Median time of one launch right after reading a buffer larger than the
    L2 and the 256 MiB fabric cache (the launch's inputs then come from HBM,
    and the caches hold clean lines of that buffer, so no write-back competes
    with the launch): HIP events around the launch alone, on the current
    stream."""
    import torch
    stream = torch.cuda.current_stream(dev)
    buf = torch.ones(flush_mib << 18, dtype=torch.float32, device=dev)
    buf.max()                            # the first pass leaves its writes behind
    torch.cuda.synchronize()
    times = []
    for _ in range(launches):
        buf.max()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del buf
    times.sort()
    return times[len(times) // 2]


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info()
             if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def rotary_cpu_baseline(w, inp, rotated, nbytes, min_seconds=10.0):
    """Time the fp64 rotary oracle over the workload's Q and K (whole passes
    until about min_seconds); also check the GPU's rotation of them."""
    import numpy as np
    import oracle
    import workloads
    f64 = workloads.to_f64
    q, k = f64(inp["q"]), f64(inp["k"])
    passes = 0
    t0 = time.perf_counter()
    while True:
        refs = [oracle.rotate_dense(x, w.d, 10000.0, False) for x in (q, k)]
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    rel = 2.0 ** -7 if w.in_dtype == "bf16" else 2.0 ** -10
    excess = max(float(np.max(np.abs(g - r) - (rel * np.abs(r) + 1e-5)))
                 for g, r in zip(rotated, refs))
    err = max(float(np.max(np.abs(g - r))) for g, r in zip(rotated, refs))
    base = {"value": round(nbytes * passes / dt / 1e9, 4), "unit": "GB/s",
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"the whole {w.name} workload (Q and K), {passes} pass(es), "
                      f"fp64 numpy, {dt:.2f} s"}
    return base, {"max_abs_err": err, "pass": excess <= 0.0}


def cpu_baseline(w, inp, o_gpu, lse_gpu, flops, nbytes, min_seconds=10.0):
    """Time the fp64 oracle over the whole workload (repeated until about
    min_seconds have passed); also return parity of the GPU output.  The
    rate is in the workload's unit: TFLOP/s, or GB/s of algorithmic bytes
    for the HBM-bound decode."""
    import numpy as np
    import oracle
    import workloads
    f64 = workloads.to_f64
    args = (f64(inp["q"]), f64(inp["k"]), f64(inp["v"]))
    # whole passes over the workload until about min_seconds of CPU work
    passes = 0
    t0 = time.perf_counter()
    while True:
        if w.dropout:
            o_ref, l_ref = oracle.attention_dropout(*args, p=w.dropout, seed=DROPOUT_SEED,
                                                    scale=w.scale, causal=w.causal,
                                                    cu_seqlens_q=inp.get("cu_seqlens_q"),
                                                    cu_seqlens_k=inp.get("cu_seqlens_k"))
        else:
            o_ref, l_ref = oracle.attention(*args, scale=w.scale, causal=w.causal,
                                            cu_seqlens_q=inp.get("cu_seqlens_q"),
                                            cu_seqlens_k=inp.get("cu_seqlens_k"))
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    err_o = float(np.max(np.abs(o_gpu - o_ref)))
    live = np.isfinite(l_ref)
    err_l = float(np.max(np.abs(lse_gpu[live] - l_ref[live])))
    dead_ok = bool(np.all(lse_gpu[~live] == -math.inf))
    if w.decode:
        value, unit = round(nbytes * passes / dt / 1e9, 4), "GB/s"
    else:
        value, unit = round(flops * passes / dt / 1e12, 6), "TFLOP/s"
    base = {"value": value, "unit": unit,
            "cores": blas_threads(), "kind": "oracle",
            "sample": f"the whole {w.name} workload, {passes} pass(es), fp64 "
                      f"numpy (S and P materialised per head in 1024-row "
                      f"chunks), {dt:.2f} s"}
    # with dropout the bar on O scales with the keep scale 1 / (1 - p)
    tol_o = 1e-2 / (1.0 - w.dropout)
    parity = {"max_abs_err_o": err_o, "max_abs_err_lse": err_l,
              "dead_rows_exact": dead_ok, "tol_o": tol_o,
              "pass": err_o <= tol_o and err_l <= 1e-3 and dead_ok}
    return base, parity


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(dirpath, suffix):
    for root, _, files in os.walk(dirpath):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {dirpath}")


def _per_dispatch(path, kernel_sub):
    """Counter values per dispatch of the kernel: {counter: [values]}.
    rocprofv3 can print a counter's row twice for one dispatch (same
    correlation id, same value); such exact repeats are counted once."""
    per, seen = {}, set()
    for r in _csv_rows(path):
        if kernel_sub not in r["Kernel_Name"]:
            continue
        row = tuple(r.values())
        if row in seen:
            continue
        seen.add(row)
        key = (r["Dispatch_Id"], r["Counter_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (_, name), val in per.items():
        out.setdefault(name, []).append(val)
    return out


def read_bytes(d, agg=None):
    """HBM-side read bytes from the L2's fabric read requests by size
    (median over the dispatches, or agg)."""
    import statistics
    m = lambda k: (agg or statistics.median)(d[k])
    return (32 * m("TCC_EA0_RDREQ_32B_sum") + 64 * m("TCC_EA0_RDREQ_64B_sum")
            + 128 * m("TCC_EA0_RDREQ_128B_sum"))


def write_bytes(d, agg=None):
    """Write bytes: 64-byte requests and 32-byte ones (the rest)."""
    import statistics
    m = lambda k: (agg or statistics.median)(d[k])
    w_all, w64 = m("TCC_EA0_WRREQ_sum"), m("TCC_EA0_WRREQ_64B_sum")
    return 64 * w64 + 32 * (w_all - w64)


READ_PMC = ("TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum TCC_EA0_RDREQ_128B_sum "
            "TCC_EA0_RDREQ_sum")
WRITE_PMC = "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum"
MFMA_PMC = ("SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F16 "
            "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES")


def summarize_copy(dirpath):
    """Markdown summary of the copy calibration: what the byte formulas
    read for a plain device copy of known size."""
    import statistics
    rec = json.loads(open(os.path.join(dirpath, "copy.json")).read().strip()
                     .splitlines()[-1]) if os.path.exists(
        os.path.join(dirpath, "copy.json")) else {"copy_calibration_bytes": 256 << 20}
    n = rec["copy_calibration_bytes"]
    rd = _per_dispatch(_find(os.path.join(dirpath, "read"), "counter_collection.csv"),
                       "copyBuffer")
    wr = _per_dispatch(_find(os.path.join(dirpath, "write"), "counter_collection.csv"),
                       "copyBuffer")
    rb, wb = read_bytes(rd), write_bytes(wr)
    cmd = "python3 bench.py --copy-calibration 256 --steps 3"
    lines = [
        "# Copy calibration of the HBM byte counters (256 MiB device-to-device copy)", "",
        "Commands (repository root, MI355X, `TMPDIR=/tmp`):", "",
        f"    rocprofv3 --pmc {READ_PMC} --output-format csv -d DIR/read -o r -- {cmd}",
        f"    rocprofv3 --pmc {WRITE_PMC} --output-format csv -d DIR/write -o w -- {cmd}",
        "    python bench.py --summarize-copy DIR", "",
        "| quantity | per copy dispatch |", "|---|---|",
        f"| dispatches of the copy kernel | {len(rd['TCC_EA0_RDREQ_sum'])} |",
        f"| read requests 32 B / 64 B / 128 B | "
        f"{statistics.median(rd['TCC_EA0_RDREQ_32B_sum']):.0f} / "
        f"{statistics.median(rd['TCC_EA0_RDREQ_64B_sum']):.0f} / "
        f"{statistics.median(rd['TCC_EA0_RDREQ_128B_sum']):.0f} |",
        f"| read bytes (32·n32 + 64·n64 + 128·n128) | {rb / 2**20:.3f} MiB = {rb / n:.5f} x "
        f"the copy's {n / 2**20:.0f} MiB |",
        f"| write bytes (64·n64 + 32·(n − n64)) | {wb / 2**20:.3f} MiB = {wb / n:.5f} x |", "",
        "Both formulas read the copy's size with no scale factor, so the kernels' "
        "summaries use them unscaled.",
    ]
    print("\n".join(lines))


def summarize_bench(dirpath):
    """Markdown table of the bench lines under DIR/<workload>/bench.json."""
    import workloads
    rows = []
    for name in workloads.WORKLOADS:
        path = os.path.join(dirpath, name, "bench.json")
        if not os.path.exists(path):
            continue
        rec = json.loads([x for x in open(path).read().splitlines() if x.startswith("{")][-1])
        roof, base, par = rec["roofline"], rec.get("cpu_baseline") or {}, rec.get("parity") or {}
        err = (f"{par.get('max_abs_err_o', par.get('max_abs_err', float('nan'))):.3e}"
               if par else "-")
        errl = f"{par['max_abs_err_lse']:.3e}" if "max_abs_err_lse" in par else "-"
        rows.append(
            f"| {name} | {rec['ms_per_step'] * 1e3:.2f} | {rec['value']} {rec['unit']} | "
            f"{100 * roof['frac']:.2f} % of {roof['peak']} ({roof['bound']}) | {err} | {errl} | "
            f"{'pass' if par.get('pass') else 'FAIL' if par else '-'} | "
            f"{base.get('value', '-')} {base.get('unit', '')} ({base.get('cores', '-')} cores) |")
    lines = [
        "# Bench lines of every workload (one session, one box)", "",
        "Command per workload (repository root, MI355X):", "",
        "    python bench.py --workload <name>          # 200 timed steps, 20 warm-up",
        "    python bench.py --summarize-bench DIR      # this table", "",
        "Time per step: HIP events around graph-replayed launches on the launch stream (median "
        "of 5 batches reported in each line's ms_per_step_median_batch).  Parity: max-abs error "
        "of the run's GPU output against the fp64 oracle.  CPU: the oracle on the box's host "
        "cores over whole passes of the workload (about 10 s).", "",
        "| workload | us / step | value | roofline | max abs err O | max abs err LSE | parity "
        "| oracle on CPU |",
        "|---|---|---|---|---|---|---|---|",
        *rows,
    ]
    print("\n".join(lines))


def summarize_counters(dirpath, name, write_record):
    """Markdown summary of the rocprofv3 runs of one workload (see the
    commands it prints) and, optionally, the committed counter record."""
    import statistics
    import workloads
    w = workloads.WORKLOADS[name]
    inp = workloads.make(name, seed=0)
    flops = 0.0 if w.rotary else 4.0 * w.d * w.hq * visible_pairs(w, inp.get("lengths"))
    nbytes = algorithmic_bytes(w, inp)
    kern = ("attn_decode_kernel" if w.decode else "rotary_kernel" if w.rotary
            else "attn_fwd_mfma_kernel")
    wl = f"--workload {name} "
    run = f"-- python3 bench.py {wl}--steps 5 --warmup 2 --no-cpu-baseline"
    cmds = {
        "trace": f"rocprofv3 --kernel-trace --stats --output-format csv -d DIR/trace -o t "
                 f"-- python3 bench.py {wl}--steps 50 --warmup 5 --no-cpu-baseline",
        "read": f"rocprofv3 --pmc {READ_PMC} --output-format csv -d DIR/read -o r {run}",
        "write": f"rocprofv3 --pmc {WRITE_PMC} --output-format csv -d DIR/write -o w {run}",
        "mfma": f"rocprofv3 --pmc {MFMA_PMC} --output-format csv -d DIR/mfma -o m {run}",
    }
    tr = [r for r in _csv_rows(_find(os.path.join(dirpath, "trace"), "kernel_trace.csv"))
          if kern in r["Kernel_Name"]]
    dur = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr]
    t_avg = statistics.mean(dur) * 1e-9  # per launch (one per step)
    rd = _per_dispatch(_find(os.path.join(dirpath, "read"), "counter_collection.csv"), kern)
    wr = _per_dispatch(_find(os.path.join(dirpath, "write"), "counter_collection.csv"), kern)
    mf = _per_dispatch(_find(os.path.join(dirpath, "mfma"), "counter_collection.csv"), kern)
    agg = statistics.median              # counters: medians per dispatch
    m = lambda d, k: agg(d[k])
    n32, n64, n128 = (m(rd, f"TCC_EA0_RDREQ_{x}B_sum") for x in (32, 64, 128))
    nall = m(rd, "TCC_EA0_RDREQ_sum")
    read_b = read_bytes(rd, agg)
    w_all, w64 = m(wr, "TCC_EA0_WRREQ_sum"), m(wr, "TCC_EA0_WRREQ_64B_sum")
    write_b = write_bytes(wr, agg)
    busy = m(mf, "SQ_VALU_MFMA_BUSY_CYCLES")
    # GRBM_GUI_ACTIVE adds up the 8 XCDs' active cycles; it also counts
    # the profiler's window around a short dispatch, so it is context only
    gui = m(mf, "GRBM_GUI_ACTIVE") / 8
    mops = m(mf, "SQ_INSTS_VALU_MFMA_MOPS_F16") + m(mf, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy_peak = busy / (SIMDS * PEAK_CLOCK_HZ * t_avg)
    busy_gui = busy / (SIMDS * gui)
    exec_flops = mops * 512
    h = kernel_hash()
    q, k, v = inp["q"], inp["k"], inp["v"]
    in_b = (q.numel() + k.numel() + v.numel()) * 2
    if w.rotary:                         # Q and K in, Q and K out
        in_b = (q.numel() + k.numel()) * 2
    lines = [
        f"# {kern} — {name} — kernel trace, HBM bytes and MFMA counters", "",
        f"Workload: {metric_label(w)}; {flops / 1e9:.3f} GFLOP algorithmic per launch, "
        f"{nbytes} algorithmic bytes " + ("(Q and K read and written once)." if w.rotary else "(Q+K+V read once, O+LSE written once)."), "",
        "Commands (repository root, MI355X, `TMPDIR=/tmp`, library built by "
        "`python exact_attention_61_amd/build.py`; each counter pass its own run):", "",
        *[f"    {c}" for c in cmds.values()],
        f"    python bench.py --summarize-counters DIR --workload {name}", "",
        "Counter figures are medians over the kernel's dispatches in each run.", "",
        "| quantity | per launch |", "|---|---|",
        f"| kernel duration (trace, {len(dur)} dispatches) "
        f"| mean {t_avg * 1e6:.2f} us, median dispatch "
        f"{statistics.median(dur) / 1e3:.2f} us, min {min(dur) / 1e3:.2f} us |",
        f"| algorithmic TFLOP/s at the mean duration | {flops / t_avg / 1e12:.1f} "
        f"({100 * flops / t_avg / 1e12 / PEAK_TFLOPS[w.in_dtype]:.2f} % of {PEAK_TFLOPS[w.in_dtype]}) |",
        f"| algorithmic GB/s at the mean duration | {nbytes / t_avg / 1e9:.0f} "
        f"({100 * nbytes / t_avg / 1e9 / PEAK_HBM_GBS:.1f} % of {PEAK_HBM_GBS:.0f}) |",
        f"| read requests 32 B / 64 B / 128 B (all) | {n32:.0f} / {n64:.0f} / {n128:.0f} ({nall:.0f}) |",
        f"| HBM read bytes (32·n32 + 64·n64 + 128·n128) | {read_b / 2**20:.2f} MiB = "
        f"{read_b / in_b:.3f} x {'Q+K' if w.rotary else 'Q+K+V'} ({in_b / 2**20:.2f} MiB) |",
        f"| write requests (64 B of them) | {w_all:.0f} ({w64:.0f}) |",
        (f"| HBM write bytes | {write_b / 2**20:.2f} MiB = {write_b / in_b:.3f} x Q+K "
         f"({in_b / 2**20:.2f} MiB) |" if w.rotary else
         f"| HBM write bytes | {write_b / 2**20:.2f} MiB = {write_b / (nbytes - in_b):.3f} x O+LSE "
         f"({(nbytes - in_b) / 2**20:.2f} MiB) |"),
        f"| MFMA busy: busy cycles / ({SIMDS} SIMDs x 2.4 GHz x mean duration) | "
        f"{100 * busy_peak:.1f} % |",
        f"| MFMA busy against GRBM_GUI_ACTIVE / 8 (context: includes the profiler's "
        f"window) | {100 * busy_gui:.1f} % |",
        f"| executed MFMA flops (MOPS x 512) | {exec_flops / 1e9:.3f} GFLOP"
        + (f" = {exec_flops / flops:.3f} x algorithmic |" if flops else " |"), "",
        f"Kernel source sha256[:16] = {h}.",
    ]
    print("\n".join(lines))
    if write_record:
        try:
            with open(TRAFFIC_FILE) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            rec = {}
        if rec.get("kernel_sha256_16") != h:
            rec = {"kernel_sha256_16": h, "workloads": {}}
        rec["workloads"][name] = {
            "hbm_bytes_per_launch": int(round(read_b + write_b)),
            "hbm_read_bytes_per_launch": int(round(read_b)),
            "hbm_write_bytes_per_launch": int(round(write_b)),
            "mfma_busy": round(busy_peak, 4),
            "kernel_us_mean": round(t_avg * 1e6, 3),
            "executed_mfma_flops": exec_flops,
            "source": f"profiles/{kern}_{name}_counters.md"}
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB "
                         "(reference point for the HBM byte counters)")
    ap.add_argument("--summarize-counters", default=None, metavar="DIR",
                    help="print the Markdown summary of the rocprofv3 runs "
                         "under DIR (no GPU work)")
    ap.add_argument("--summarize-bench", default=None, metavar="DIR",
                    help="print the Markdown table of the bench lines under DIR (no GPU work)")
    ap.add_argument("--summarize-copy", default=None, metavar="DIR",
                    help="print the Markdown summary of the copy calibration's "
                         "counter runs under DIR (no GPU work)")
    ap.add_argument("--write-record", action="store_true",
                    help="with --summarize-counters: update the counter "
                         "record under profiles/")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): "
              "attention over independent (batch, head) pairs would shard "
              "with no exchange, and no multi-GPU figure is produced.",
              file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        sys.exit(2)
    if args.summarize_copy:
        summarize_copy(args.summarize_copy)
        return
    if args.summarize_bench:
        summarize_bench(args.summarize_bench)
        return
    if args.summarize_counters:
        import workloads
        summarize_counters(args.summarize_counters,
                           args.workload or workloads.HEADLINE,
                           args.write_record)
        return

    import torch
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n,
                          "launches": max(1, args.steps)}), flush=True)
        return
    import workloads
    import exact_attention_61_amd as mi

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    inp = workloads.make(name, seed=0)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    kw = dict(causal=w.causal, scale=w.scale)
    out_dtype = workloads.DTYPES[w.out_dtype]
    o = None if w.rotary else torch.empty(q.shape, dtype=out_dtype, device=dev)
    if w.rotary:
        lse = None
    elif w.varlen:
        kw.update(cu_seqlens_q=inp["cu_seqlens_q"].to(dev),
                  cu_seqlens_k=inp["cu_seqlens_k"].to(dev),
                  max_seqlen_q=inp["max_seqlen_q"],
                  max_seqlen_k=inp["max_seqlen_k"])
        lse = torch.empty((w.hq, q.shape[0]), dtype=torch.float32, device=dev)
    else:
        lse = torch.empty((w.batch, w.hq, w.lq), dtype=torch.float32,
                          device=dev)

    workspace = None
    if w.decode:
        nws = mi.mi_attn_decode_workspace_size(w.batch, w.hq, w.hkv, w.lq, w.lk, w.d)
        if nws:
            workspace = torch.zeros(nws, dtype=torch.uint8, device=dev)

        def step():
            mi.mi_attn_decode(q, k, v, o, lse, workspace=workspace, **kw)
    elif w.rotary:
        # one rotation of fresh copies for the parity check, then the timed
        # steps rotate q and k in place again and again
        qr, kr = q.clone(), k.clone()
        mi.mi_attn_rotary_qk(qr, kr, w.d)
        torch.cuda.synchronize()
        rotated = [x.to("cpu", torch.float64).numpy() for x in (qr, kr)]
        del qr, kr

        def step():
            mi.mi_attn_rotary_qk(q, k, w.d)
    elif w.dropout:
        def step():
            mi.mi_attn_fwd_dropout(q, k, v, o, lse, dropout_p=w.dropout, seed=DROPOUT_SEED,
                                   **kw)
    else:
        def step():
            mi.mi_attn_fwd(q, k, v, o, lse, **kw)

    lengths = inp.get("lengths")
    flops = 0.0 if w.rotary else 4.0 * w.d * w.hq * visible_pairs(w, lengths)
    nbytes = algorithmic_bytes(w, inp)

    # warm-up (eager), with torch's peak-allocation counter reset first:
    # everything allocated now is the inputs, outputs and cu_seqlens
    torch.cuda.synchronize()
    resident = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev)

    # the K timed steps: batches of back-to-back launches, one graph each
    sizes = batch_sizes(args.steps)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = {}
    for n in sorted(set(sizes)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                step()
        graphs[n] = g
    for g in graphs.values():
        g.replay()                       # warm replay
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(sizes) + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i, n in enumerate(sizes):
        graphs[n].replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_total = ev[0].elapsed_time(ev[-1])
    ms = ms_total / args.steps
    per_batch = sorted(ev[i].elapsed_time(ev[i + 1]) / n
                       for i, n in enumerate(sizes))
    ms_median = per_batch[len(per_batch) // 2]

    # plain eager calls, for context
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    # cold launches (inputs evicted from the caches first), for context
    ms_cold = cold_launch_ms(step, dev)

    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    peak_tf = PEAK_TFLOPS[w.in_dtype]
    props = torch.cuda.get_device_properties(dev)
    counters = load_counter_record(name)

    base, parity = (None, None)
    if w.rotary:
        if not args.no_cpu_baseline:
            base, parity = rotary_cpu_baseline(w, inp, rotated, nbytes)
    else:
        o_gpu = o.to("cpu", torch.float64).numpy()
        lse_gpu = lse.to("cpu", torch.float64).numpy()
        if not args.no_cpu_baseline:
            base, parity = cpu_baseline(w, inp, o_gpu, lse_gpu, flops, nbytes)

    hbm_bound = w.decode or w.rotary
    if hbm_bound:
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": None if counters is None else counters.get("hbm_bytes_per_launch"),
                    "mfma_busy": None if counters is None else counters.get("mfma_busy"),
                    "algorithmic_bytes": nbytes,
                    "kernel": "rotary_kernel" if w.rotary else "attn_decode_kernel"}
    else:
        roofline = {"bound": "mfma", "achieved": round(tflops, 3),
                    "peak": peak_tf, "unit": "TFLOP/s",
                    "frac": round(tflops / peak_tf, 4),
                    "traffic": None if counters is None else counters.get("hbm_bytes_per_launch"),
                    "mfma_busy": None if counters is None else counters.get("mfma_busy"),
                    "algorithmic_bytes": nbytes,
                    "kernel": "attn_fwd_mfma_kernel"}
    rec = {
        "metric": metric_label(w),
        "value": round(gbs, 1) if hbm_bound else round(tflops, 3),
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic (seeded N(0,1))",
        "config": {"workload": name, "batch": w.batch, "hq": w.hq,
                   "hkv": w.hkv, "lq": w.lq, "lk": w.lk, "head_dim": w.d,
                   "causal": w.causal, "varlen": w.varlen,
                   "in_dtype": w.in_dtype, "out_dtype": w.out_dtype,
                   "lengths": lengths},
        "pct_of_peak": round(100.0 * (gbs / PEAK_HBM_GBS if hbm_bound else tflops / peak_tf), 2),
        "algorithmic_flops": flops,
        "tflops": round(tflops, 3),
        # the common convention: 4*B*H*Lq*Lk*d, halved for causal
        "flops_common_convention": 0.0 if w.rotary else (2.0 if w.causal else 4.0) *
        w.batch * w.hq * w.lq * w.lk * w.d,
        "ms_per_step_median_batch": round(ms_median, 6),
        "batches": sizes,
        "ms_per_step_eager": round(ms_eager, 6),
        "cold": {"ms_per_launch_median": round(ms_cold, 6), "launches": 20,
                 "flush_bytes": 512 << 20,
                 "value": round(nbytes / (ms_cold * 1e-3) / 1e9, 1) if hbm_bound else
                 round(flops / (ms_cold * 1e-3) / 1e12, 3),
                 "note": "one launch after reading 512 MiB (more than L2 + fabric cache); "
                         "context only, not the headline value"},
        "roofline": roofline,
        "memory": {"peak_allocated_bytes": int(peak),
                   "inputs_outputs_bytes": int(resident),
                   "workspace_bytes": 0 if workspace is None else workspace.numel(),
                   "ratio": round(peak / resident, 4) if resident else None},
        "cpu_baseline": base,
        "parity": parity,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", None),
                   "peak_engine_clock_mhz": engine_clock_mhz(dev.index or 0)},
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
