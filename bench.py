#!/usr/bin/env python3
"""Throughput of the block-paged hot path on one MI355X.

One step is one pass of every stage of the path over one batch of the decode
workload (64 sequences, lengths uniform in 1..2048, page_size 16, 32 heads x
128 fp16, 12,000-page pool, uint32 block table of unique pages):

  1. hp_validate_async  storage invariants of the descriptor, enqueued on the
                        moves' stream; its verdict stays on the device;
  2. hp_gather          pool -> logical [T, 32, 128] fp16 tensor (streaming hint:
                        the table names each page once);
  3. hp_scatter         that tensor back into its slots (the write direction);
  4. hp_gather_dequant  the same table over an int8 copy of the pool with one
                        fp32 scale per slot -> bf16 [T, 32, 128].

The moves are gated (HP_FLAG_GATED): each reads its step's verdict on the
device and would write nothing for a rejected descriptor, so no host round
trip sits between steps.

Inputs are resident in HBM before timing starts. `value` is the step's
algorithmic bytes (each live row read once and written once per move, one
scale per row, the validator's metadata reads) over the wall-clock step time
(K steps bracketed by device synchronisation), in GB/s (1 GB = 1e9 B).

Per-kernel launch durations come from HIP events on the launch stream around
back-to-back launches of each kernel (the GPU stays busy, so the interval is
kernel time); `roofline` uses the gather kernel's, and adds the rocprofv3
averages of the committed kernel trace when it was taken on the current
kernel sources.

`configs` times every workload's moves on its own: tiny (gather + scatter),
decode (gather, scatter, dequant), prefix sharing (gather; unique and
logical bytes), append (scatter with tail zeroing) and the quantized large
pool (dequant, raw gather). Before each of `--flush-iters` iterations a
1 GiB buffer is read through to evict the caches; HIP events bracket the call;
median, p10 and p90 are reported. The CPU oracle is timed on the host on the
same work: one thread on a bounded prefix of the sequences, and every
sequence split into balanced ranges over one thread per core.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                  [--no-configs] [--extras]
  python bench.py --summarize-profiles TRACE_DIR FETCH_DIR WRITE_DIR
      (writes the rocprofv3 summaries under profiles/; the rocprofv3 commands
      below write their raw output under rocprof_out/)
"""
import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (and % of peak) for paged gather/scatter, tokens/s"
HBM_PEAK_GBS = 8000.0
CSRC = os.path.join(ROOT, "block_table_gather_amd", "csrc")
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("hp_kernels.hip", "hp_api.cpp", "hp_internal.h",
                                                  "hp_device.h")]
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "gather_copy_kernel_decode_traffic.json")
GATHER_KERNEL = "copy_kernel<unsigned int, (hp::Op)0, 16, true, true, -1, 2>"
KERNEL_LABELS = {
    "copy_kernel<unsigned int, (hp::Op)0, 16, true, true, -1, 2>":
        "gather (u32, 16 B vectors, fused, streaming loads, 2 loads per lane)",
    "copy_kernel<unsigned int, (hp::Op)1, 16, true, true, -1, 2>":
        "scatter (u32, 16 B vectors, fused, streamed source, 2 loads per lane)",
    "copy_kernel<unsigned int, (hp::Op)1, 16, true, false, -1, 8>":
        "scatter (u32, 16 B vectors, fused, 8 loads per lane)",
    "copy_kernel<unsigned int, (hp::Op)2, 8, true, false, -1, 8>":
        "dequant-gather (u32, 8 B int8 vectors, fused)",
    "validate_one_kernel<unsigned int>": "validator, one workgroup (u32)",
    "validate_kernel<unsigned int>": "validator (u32)",
    "validate_init_kernel": "validator init",
}
CALIBRATION_BYTES = 1 << 30
TRACE_STEPS, TRACE_WARMUP = 50, 5
PRE_STEPS = 100  # untimed steps before the warm-up ones (about 50 ms on MI355X)
TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d rocprof_out/prof_trace -o trace -- "
             f"python3 bench.py --steps {TRACE_STEPS} --warmup {TRACE_WARMUP} --no-cpu-baseline "
             "--no-reference-copies --no-configs")
PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d rocprof_out/prof_{d} -o {d} -- "
           "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-reference-copies "
           "--no-configs --copy-calibration")
ATTN_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d rocprof_out/prof_attn_trace -o trace "
                  "-- python3 bench.py --attention-only")
ATTN_PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d rocprof_out/prof_attn_{d} -o {d} -- "
                "python3 bench.py --attention-only --kernel-reps 3 --copy-calibration")
QW_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d rocprof_out/prof_qw_trace -o trace "
                "-- python3 bench.py --quant-write-only")
QW_PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d rocprof_out/prof_qw_{d} -o {d} -- "
              "python3 bench.py --quant-write-only --kernel-reps 3 --copy-calibration")


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def step_bytes(T, S, K, H, D, idx_bytes=4):
    """Algorithmic bytes of one step (see module docstring)."""
    row = H * D * 2                      # fp16 row
    gather = 2 * T * row                 # read each live row once, write it once
    scatter = 2 * T * row
    dequant = T * H * D + 4 * T + T * H * D * 2   # int8 rows + one scale per row + bf16 rows
    validate = idx_bytes * (K + (S + 1) + S)      # block table, seq_ptr, seq_lens
    return {"validate": validate, "gather": gather, "scatter": scatter, "dequant": dequant}


def traffic_for():
    """HBM bytes per gather launch from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# ---- CPU oracle legs ---------------------------------------------------------------

def cpu_info():
    """(cores this process may run on, CPU model name)."""
    cores = len(os.sched_getaffinity(0))
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_threads():
    """Threads of the all-core leg: every core of the affinity mask, within
    the OMP_NUM_THREADS share when the machine sets one."""
    cores, _ = cpu_info()
    lim = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(cores, int(lim))) if lim.isdigit() and int(lim) > 0 else cores


def seq_ranges(lens, n):
    """Split sequences into at most n contiguous ranges of about equal tokens."""
    import numpy as np
    lens = np.asarray(lens, dtype=np.int64)
    S = len(lens)
    if S == 0:
        return []
    cum = np.cumsum(lens)
    cuts = {0, S}
    for i in range(1, n):
        cuts.add(min(S, int(np.searchsorted(cum, cum[-1] * i / n, side="left")) + 1))
    cuts = sorted(cuts)
    return [(a, b) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]


def sub_desc(w, s0, s1):
    """Oracle arguments for sequences [s0, s1) alone: their slice of the table,
    seq_ptr rebased to 0, their counts (and starts)."""
    import numpy as np
    sp = w.seq_ptr.astype(np.int64)
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim,
              block_table=w.block_table[sp[s0]: sp[s1]],
              seq_ptr=(sp[s0: s1 + 1] - sp[s0]).astype(np.uint64),
              seq_lens=w.seq_lens[s0:s1])
    if w.seq_start is not None:
        kw["seq_start"] = w.seq_start[s0:s1]
    return kw


def cpu_legs(w, run, nbytes, seconds):
    """Times the oracle, as it stands, on the host: `run(s0, s1)` does the
    work of sequences [s0, s1) (plain oracle calls on that range alone);
    `nbytes(s0, s1)` gives its algorithmic bytes.

    single_thread: one thread on the longest prefix of sequences that fits
    about `seconds`; all_cores: every sequence, split into balanced ranges
    run concurrently by one thread per core (the oracle's C loops release
    the interpreter lock)."""
    import concurrent.futures
    import numpy as np
    lens = w.seq_lens.astype(np.int64)
    S = len(lens)

    def timed(s1):
        t0 = time.perf_counter()
        run(0, s1)
        return time.perf_counter() - t0

    n = 1
    dt = timed(n)
    while dt < seconds / 8 and n < S:
        n = min(S, n * 4)
        dt = timed(n)
    if dt < seconds / 2 and n < S:
        T = int(lens[:n].sum())
        target = T * seconds / 2 / max(dt, 1e-9)
        n = max(1, min(int(np.searchsorted(np.cumsum(lens), target)) + 1, S))
        dt = timed(n)
    T1 = int(lens[:n].sum())
    b1 = nbytes(0, n)
    threads = cpu_threads()
    ranges = seq_ranges(lens, threads)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(ranges)) as ex:
        t0 = time.perf_counter()
        list(ex.map(lambda r: run(*r), ranges))
        dt_all = time.perf_counter() - t0
    b_all = nbytes(0, S)
    T = int(lens.sum())
    cores, model = cpu_info()
    return {
        "single_thread": {"value": round(b1 / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                          "seconds": round(dt, 3), "tokens_per_s": round(T1 / dt, 1),
                          "sample": f"first {n} of {S} sequences ({T1} of {T} tokens)"},
        "all_cores": {"value": round(b_all / dt_all / 1e9, 4), "unit": "GB/s",
                      "cores": len(ranges), "seconds": round(dt_all, 3),
                      "tokens_per_s": round(T / dt_all, 1),
                      "sample": f"all {S} sequences in {len(ranges)} ranges, one thread each"},
        "affinity_cores": cores, "cpu_model": model}


# ---- rocprofv3 summaries --------------------------------------------------------

def _short(name):
    name = name.replace("hp::(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.rsplit("(", 1)[0]  # drop the parameter list


def summarize_profiles(trace_dir, fetch_dir, write_dir):
    """Writes the kernel-trace and counter summaries (markdown) and the gather
    kernel's calibrated traffic (json) under profiles/."""
    import csv
    import glob

    def one(d, pattern):
        files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
        if len(files) != 1:
            raise SystemExit(f"expected one {pattern} under {d}, found {files}")
        with open(files[0]) as f:
            return list(csv.DictReader(f))

    trace = one(trace_dir, "*kernel_trace.csv")
    launches = {}
    for r in trace:
        short = _short(r["Kernel_Name"])
        if short in KERNEL_LABELS:
            launches.setdefault(short, []).append(
                (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) -
                                             int(r["Start_Timestamp"])) / 1e3))
    # per move, in launch order: 21 back-to-back launches (the discarded
    # launch-timing pass), the untimed pre-pass steps, the warm-up and timed
    # steps, then the 21 kept back-to-back launches
    n_b2b, n_mid = 21, PRE_STEPS + TRACE_WARMUP + TRACE_STEPS
    lines = ["# Kernel durations: decode-batch bench step (rocprofv3 kernel trace)", "",
             "Command (from the repository root, on one MI355X):", "",
             f"    {TRACE_CMD}", "",
             "Each move runs 21 times back to back (a launch-timing pass, discarded), once "
             f"per step ({PRE_STEPS} untimed",
             f"steps, {TRACE_WARMUP} warm-up, {TRACE_STEPS} timed), then 21 times back to "
             "back for the event timing.",
             f"`step` averages the {TRACE_STEPS} timed steps' launches, `back-to-back` the "
             "last 21. Durations in microseconds.", "",
             "| kernel | what | calls | avg | min | max | step avg | back-to-back avg |",
             "|---|---|---|---|---|---|---|---|"]
    gather = None
    for short in sorted(launches, key=lambda k: KERNEL_LABELS[k]):
        ts = [d for _, d in sorted(launches[short])]
        avg = sum(ts) / len(ts)
        step = b2b = ""
        if not short.startswith("validate") and len(ts) == 2 * n_b2b + n_mid:
            st, bb = ts[n_b2b + n_mid - TRACE_STEPS:n_b2b + n_mid], ts[-n_b2b:]
            step, b2b = f"{sum(st) / len(st):.1f}", f"{sum(bb) / len(bb):.1f}"
            if short == GATHER_KERNEL:
                gather = (avg, sum(st) / len(st), sum(bb) / len(bb))
        lines.append(f"| `{short}` | {KERNEL_LABELS[short]} | {len(ts)} | {avg:.1f} | "
                     f"{min(ts):.1f} | {max(ts):.1f} | {step} | {b2b} |")
    lines += ["", "The validator (`hp_validate_async`) runs in line before each step's moves.",
              "", "Other kernels in the trace are PyTorch's input generation (random values,",
              "fills, index_put) and the runtime's copies; they are outside the timed step."]
    with open(os.path.join(PROFILES, "decode_step_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if gather is None:
        raise SystemExit("gather kernel not found in the kernel trace")
    gather_avg = gather[0]

    def per_kernel(rows, counter):
        agg = {}
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            agg.setdefault(r["Kernel_Name"], []).append((int(r["Grid_Size"]),
                                                         float(r["Counter_Value"])))
        for name, vals in agg.items():
            # one launch shape per kernel of the step; several would mean the
            # run mixed other work into the same kernel's average
            if "hp::" in name and len({g for g, _ in vals}) != 1:
                raise SystemExit(f"{name}: several grid sizes in one run; profile with "
                                 "--no-reference-copies")
        return agg

    fetch = per_kernel(one(fetch_dir, "*counter_collection.csv"), "FETCH_SIZE")
    write = per_kernel(one(write_dir, "*counter_collection.csv"), "WRITE_SIZE")

    def calib(agg):
        # the 1 GiB calibration copies are the runtime copy kernel's largest grids
        # (the profiled runs make no other large copy)
        rows = agg.get("__amd_rocclr_copyBuffer", [])
        g = max(x[0] for x in rows)
        vals = [x[1] for x in rows if x[0] == g]
        if len(vals) != 3:
            raise SystemExit(f"expected the 3 calibration copies, found {len(vals)}")
        return sum(vals) / len(vals), len(vals)

    f_kib, nf = calib(fetch)
    w_kib, nw = calib(write)
    f_factor = CALIBRATION_BYTES / (f_kib * 1024)
    w_factor = CALIBRATION_BYTES / (w_kib * 1024)
    out = ["# HBM traffic per launch: decode-batch kernels (rocprofv3 counters)", "",
           "Two counter passes, each in its own run (commands from the repository root):", "",
           f"    {PMC_CMD.format(c='FETCH_SIZE', d='fetch')}",
           f"    {PMC_CMD.format(c='WRITE_SIZE', d='write')}", "",
           "Calibration: `--copy-calibration` runs three plain 1 GiB device-to-device copies",
           "(the runtime's copy kernel) that read and write exactly 1,073,741,824 bytes.",
           f"They read FETCH_SIZE = {f_kib:.1f} KiB ({nf} dispatches) and WRITE_SIZE = "
           f"{w_kib:.1f} KiB ({nw}),",
           f"so bytes = FETCH_SIZE x 1024 x {f_factor:.4f} and WRITE_SIZE x 1024 x {w_factor:.4f}.", "",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read GB | HBM write GB | total GB |",
           "|---|---|---|---|---|---|"]
    traffic = None
    for name in sorted(fetch):
        short = _short(name)
        if short not in KERNEL_LABELS or name not in write:
            continue
        fk = sum(v for _, v in fetch[name]) / len(fetch[name])
        wk = sum(v for _, v in write[name]) / len(write[name])
        rb, wb = fk * 1024 * f_factor, wk * 1024 * w_factor
        out.append(f"| `{short}` | {fk:.1f} | {wk:.1f} | {rb / 1e9:.4f} | {wb / 1e9:.4f} | "
                   f"{(rb + wb) / 1e9:.4f} |")
        if short == GATHER_KERNEL:
            traffic = {"kernel": short, "fetch_kib": fk, "write_kib": wk,
                       "hbm_read_bytes": round(rb), "hbm_write_bytes": round(wb),
                       "hbm_bytes_per_launch": round(rb + wb)}
    out += ["", "Per launch, averaged over the run's launches of each kernel. The gather's",
            "algorithmic bytes per launch are 1,041,039,360 (63,540 rows of 8 KiB read once",
            "and written once)."]
    with open(os.path.join(PROFILES, "decode_step_hbm_traffic.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    if traffic is None:
        raise SystemExit("gather kernel not found in the counter runs")
    traffic.update({"kernel_source_sha256_16": kernel_source_hash(),
                    "fetch_factor": f_factor, "write_factor": w_factor,
                    "calibration_bytes": CALIBRATION_BYTES,
                    "rocprof_avg_launch_us": gather_avg,
                    "rocprof_avg_step_us": gather[1],
                    "rocprof_avg_back_to_back_us": gather[2],
                    "algorithmic_bytes_per_launch": 1041039360,
                    "trace_command": TRACE_CMD,
                    "commands": [PMC_CMD.format(c="FETCH_SIZE", d="fetch"),
                                 PMC_CMD.format(c="WRITE_SIZE", d="write")]})
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(traffic, f, indent=1)
    print(json.dumps(traffic))


def _csv_rows(d, pattern):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one {pattern} under {d}, found {files}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _calibration(rows, counter):
    """Mean counter value of the three 1 GiB calibration copies (the runtime
    copy kernel's largest grids in the run)."""
    vals = [(int(r["Grid_Size"]), float(r["Counter_Value"])) for r in rows
            if r["Counter_Name"] == counter and r["Kernel_Name"] == "__amd_rocclr_copyBuffer"]
    g = max(x[0] for x in vals)
    big = [v for gs, v in vals if gs == g]
    if len(big) != 3:
        raise SystemExit(f"expected the 3 calibration copies, found {len(big)}")
    return sum(big) / 3


# Counter passes of the per-workload run (one rocprofv3 --pmc run each; every
# pass stays within the per-block limits: at most 4 TCC, 4 TCP, 8 SQ and 2
# GRBM counters).
COUNTER_PASSES = {
    "reqsize": "TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_32B_sum TCC_EA0_RDREQ_64B_sum "
               "TCC_EA0_RDREQ_128B_sum TCP_UTCL1_TRANSLATION_MISS_sum "
               "TCP_UTCL1_TRANSLATION_HIT_sum TCP_UTCL1_REQUEST_sum "
               "TCP_UTCL1_STALL_MULTI_MISS_sum GRBM_GUI_ACTIVE",
    "writes": "TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_64B_sum TCC_HIT_sum TCC_MISS_sum "
              "TCP_TCC_READ_REQ_sum TCP_TCC_READ_REQ_LATENCY_sum TCP_PENDING_STALL_CYCLES_sum",
    "latency": "TCC_EA0_RDREQ_LEVEL_sum TCC_EA0_RDREQ_DRAM_sum TCC_EA0_WRREQ_LEVEL_sum "
               "TCC_EA0_WRREQ_DRAM_sum SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_INST_ANY",
}
COUNTER_CMD = ("rocprofv3 --pmc {c} -f csv -d rocprof_out/prof_cnt_{d} -o {d} -- "
               "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --flush-iters 3 "
               "--copy-calibration")


def summarize_counters(*dirs):
    """Per-dispatch averages of the COUNTER_PASSES counters for every kernel
    (and grid size) of the per-workload run, one directory per pass in the
    order of COUNTER_PASSES, into profiles/workload_kernel_counters.md. Read
    bytes from request sizes (32/64/128 B) are set beside FETCH_SIZE's
    formula, which takes a request that is not 32 B as 64 B."""
    names = list(COUNTER_PASSES)
    if len(dirs) != len(names):
        raise SystemExit(f"expected {len(names)} directories ({', '.join(names)})")
    agg = {}
    for d in dirs:
        for r in _csv_rows(d, "*counter_collection.csv"):
            short = _short(r["Kernel_Name"])
            if not (short.startswith(("copy_kernel", "validate", "copy_pages", "__amd_rocclr"))):
                continue
            key = (short, int(r["Grid_Size"]))
            agg.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    lines = ["# Counters per dispatch: every workload's moves (rocprofv3 --pmc)", "",
             "One run per pass (commands from the repository root, on one MI355X):", ""]
    for d in names:
        lines.append(f"    {COUNTER_CMD.format(c=COUNTER_PASSES[d], d=d)}")
    lines += ["", "Each dispatch is one move of one workload after a 1 GiB read flush (or the",
              "decode step's launches, or a plain 1 GiB runtime copy: `__amd_rocclr_copyBuffer`",
              "at the largest grid). Values are per-dispatch means over the run's dispatches",
              "of that kernel and grid. Read bytes by request size = 32 x RDREQ_32B + 64 x",
              "RDREQ_64B + 128 x RDREQ_128B; FETCH_SIZE's formula (no TCC_BUBBLE here)",
              "counts every request that is not 32 B as 64 B. Write bytes = 32 x (WRREQ -",
              "WRREQ_64B) + 64 x WRREQ_64B. Mean read latency = RDREQ_LEVEL / RDREQ (cycles),",
              "UTCL1 miss rate = TRANSLATION_MISS / REQUEST.", "",
              "| kernel (grid) | n | read MB (req sizes) | FETCH_SIZE-formula MB | 128 B share | "
              "write MB | L2 hit | UTCL1 requests | UTCL1 misses | miss rate | EA read lat. cyc "
              "| TCP-TCC read lat. cyc | GUI active cyc |",
              "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    rows = []
    for (short, grid), c in sorted(agg.items()):
        m = {k: sum(v) / len(v) for k, v in c.items()}
        n = max(len(v) for v in c.values())
        g = lambda k: m.get(k, float("nan"))
        r32, r64, r128, rall = (g("TCC_EA0_RDREQ_32B_sum"), g("TCC_EA0_RDREQ_64B_sum"),
                                g("TCC_EA0_RDREQ_128B_sum"), g("TCC_EA0_RDREQ_sum"))
        read_b = 32 * r32 + 64 * r64 + 128 * r128
        fetch_b = 32 * r32 + 64 * (rall - r32)
        wr, wr64 = g("TCC_EA0_WRREQ_sum"), g("TCC_EA0_WRREQ_64B_sum")
        write_b = 32 * (wr - wr64) + 64 * wr64
        hit, miss = g("TCC_HIT_sum"), g("TCC_MISS_sum")
        ureq, umiss = g("TCP_UTCL1_REQUEST_sum"), g("TCP_UTCL1_TRANSLATION_MISS_sum")
        lat = g("TCC_EA0_RDREQ_LEVEL_sum") / rall if rall else float("nan")
        tlat = g("TCP_TCC_READ_REQ_LATENCY_sum") / g("TCP_TCC_READ_REQ_sum")
        rows.append((short, grid, n, read_b, fetch_b, r128 / rall if rall else 0, write_b,
                     hit / (hit + miss) if hit + miss else float("nan"), ureq, umiss,
                     umiss / ureq if ureq else float("nan"), lat, tlat, g("GRBM_GUI_ACTIVE")))
    for (short, grid, n, rb, fb, s128, wb, hr, ureq, umiss, mr, lat, tlat, act) in rows:
        lines.append(f"| `{short}` ({grid}) | {n} | {rb / 1e6:.1f} | {fb / 1e6:.1f} | {s128:.3f} | "
                     f"{wb / 1e6:.1f} | {hr:.3f} | {ureq:.0f} | {umiss:.0f} | {mr:.4f} | "
                     f"{lat:.0f} | {tlat:.0f} | {act:.0f} |")
    with open(os.path.join(PROFILES, "workload_kernel_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_attention(trace_dir, fetch_dir, write_dir):
    """Kernel durations and calibrated HBM traffic of the attention kernels
    (bench.py --attention-only runs) into profiles/."""
    import numpy as np
    import workloads
    dec, pre = workloads.decode(), workloads.prefix()
    n_unique = len(np.unique(pre.block_table)) * pre.page_size

    def algo(w, group, q8=False, unique=False):
        """(logical, unique or None) algorithmic bytes of one call."""
        Hq = w.num_heads * group
        io = w.num_seqs * Hq * w.head_dim * 6  # queries read (2 bytes), fp32 output written
        row = w.num_heads * w.head_dim * (1 if q8 else 2) + (4 if q8 else 0)  # K or V slot
        logical = 2 * w.total_tokens * row + io
        return logical, (2 * n_unique * row + io if unique else None)

    # The --attention-only run calls its workloads in this order, each with
    # one main kernel (vector or matrix-core) of its own name and grid: the
    # main-kernel groups of the trace, in order of first launch, are these.
    order = [("decode, f16, G = 1", algo(dec, 1)),
             ("prefix, bf16, G = 4", algo(pre, 4, unique=True)),
             ("prefix, bf16, G = 8", algo(pre, 8, unique=True)),
             ("decode, f16, G = 4", algo(dec, 4)),
             ("decode, int8, G = 1", algo(dec, 1, q8=True)),
             ("decode, int8, G = 4", algo(dec, 4, q8=True)),
             ("prefix, int8, G = 4", algo(pre, 4, q8=True, unique=True))]

    trace = _csv_rows(trace_dir, "*kernel_trace.csv")
    groups, first = {}, {}
    for r in trace:
        if "attention" not in r["Kernel_Name"]:
            continue
        key = (_short(r["Kernel_Name"]),
               int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
        t0 = int(r["Start_Timestamp"])
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - t0) / 1e3)
        first[key] = min(first.get(key, t0), t0)
    main = sorted((k for k in groups if k[0].startswith(("attention_kernel<",
                                                            "attention_mfma_kernel<"))),
                  key=lambda k: first[k])
    if len(main) != len(order):
        raise SystemExit(f"expected {len(order)} main attention kernels, found {len(main)}")
    workload_of = dict(zip(main, order))

    def match(key):
        return workload_of.get(key)

    lines = ["# Kernel durations: decode attention through the block table (rocprofv3)", "",
             "Command (from the repository root, on one MI355X):", "", f"    {ATTN_TRACE_CMD}", "",
             "Seven workloads, each called 21 times (the prefix ones 21 more times reusing a",
             "plan made once, HP_FLAG_PLANNED: no comparison or plan kernel in those calls):",
             "the decode batch (64 sequences, 32 kv",
             "heads x 128, streaming loads) over f16 pools with one query head per kv head",
             "(vector kernel and combine) and with four (matrix-core kernel and combine); the",
             "prefix-sharing batch (256 sequences sharing 64 leading pages, 8 kv heads x 128)",
             "over bf16 pools with 4 and with 8 query heads per kv head (cached loads: the",
             "shared-prefix pass); and over int8 pools with one fp32 scale per slot",
             "(hp_paged_attention_q8, bf16 queries) the decode batch with 1 and 4 query heads",
             "per kv head and the prefix batch with 4. A prefix call runs four kernels: the",
             "leading-page comparison (one wave per sequence), the one-workgroup plan, the",
             "matrix-core kernel (shared work items first in its grid, then the units over the",
             "pages after the shared part) and the combine; the comparison and plan rows hold",
             "the prefix workloads' calls (same grid). Durations in microseconds. Logical",
             "bytes count every sequence's K/V rows (shared pages once per sequence; int8",
             "rows with their slot scale); unique bytes count each distinct page once (the",
             "least any call must read), both with the queries read and the fp32 output",
             "written.", "",
             "| kernel | calls | avg us | min us | max us | logical GB | unique GB | "
             "unique GB/s at avg |",
             "|---|---|---|---|---|---|---|---|"]
    for (name, grid), ts in sorted(groups.items(), key=lambda kv: first[kv[0]]):
        lg = ug = ugs = ""
        m = match((name, grid))
        if m is not None:
            what, (logical, unique) = m
            lg = f"{logical / 1e9:.4f} ({what})"
            if unique is not None:
                ug = f"{unique / 1e9:.4f}"
                ugs = f"{unique / (np.mean(ts) * 1e3):.0f}"
            else:
                ug = lg.split()[0]
                ugs = f"{logical / (np.mean(ts) * 1e3):.0f}"
        lines.append(f"| `{name}` (grid {grid}) | {len(ts)} | {np.mean(ts):.1f} | {min(ts):.1f} | "
                     f"{max(ts):.1f} | {lg} | {ug} | {ugs} |")
    with open(os.path.join(PROFILES, "attention_decode_prefix_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    fetch = _csv_rows(fetch_dir, "*counter_collection.csv")
    write = _csv_rows(write_dir, "*counter_collection.csv")
    ff = CALIBRATION_BYTES / (_calibration(fetch, "FETCH_SIZE") * 1024)
    wf = CALIBRATION_BYTES / (_calibration(write, "WRITE_SIZE") * 1024)

    def per_launch(rows, counter):
        agg = {}
        for r in rows:
            if r["Counter_Name"] == counter and "attention" in r["Kernel_Name"]:
                key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
                agg.setdefault(key, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fk, wk = per_launch(fetch, "FETCH_SIZE"), per_launch(write, "WRITE_SIZE")
    out = ["# HBM traffic per launch: attention kernels (rocprofv3 counters)", "",
           "Two counter passes, each in its own run (commands from the repository root):", "",
           f"    {ATTN_PMC_CMD.format(c='FETCH_SIZE', d='fetch')}",
           f"    {ATTN_PMC_CMD.format(c='WRITE_SIZE', d='write')}", "",
           "Calibrated with three plain 1 GiB device copies in the same runs: bytes =",
           f"FETCH_SIZE x 1024 x {ff:.4f} and WRITE_SIZE x 1024 x {wf:.4f}. The counters see",
           "the L2's traffic to the fabric, Infinity Cache hits included. Algorithmic bytes:",
           "decode, every live K and V row read once; prefix, every distinct page read once",
           "(unique bytes); both with the queries read and the fp32 output written. The",
           "attention kernels' writes include the per-unit partial results the combine",
           "kernel reads.", "",
           "| kernel | read GB | write GB | algorithmic GB |", "|---|---|---|---|"]
    for key in sorted(fk):
        if key not in wk:
            continue
        name = key[0]
        rb, wb = fk[key] * 1024 * ff, wk[key] * 1024 * wf
        gb = ""
        m = match(key)
        if m is not None:
            what, (logical, unique) = m
            gb = f"{(unique if unique is not None else logical) / 1e9:.4f} ({what})"
        out.append(f"| `{name}` (grid {key[1]}) | {rb / 1e9:.4f} | {wb / 1e9:.4f} | {gb} |")
    with open(os.path.join(PROFILES, "attention_decode_prefix_hbm_traffic.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(lines + [""] + out))


def quant_write_extras(hp, torch, np, dev, stream, reps, rounds=6):
    """Quantize-on-scatter on the decode batch: its fp16 rows (63,540 tokens,
    32 heads x 128) written into an int8 pool (symmetric, a scale per slot)
    and a uint8 pool (a scale and a zero point per slot). Algorithmic bytes:
    every row read (2 bytes a value) and its codes written (1 byte a value),
    plus 4 bytes of scale (and 1 of zero point) per token. The two forms are
    timed in alternating order over `rounds` rounds of `reps` back-to-back
    calls each (neither always runs second); the median round is reported."""
    import workloads
    w = workloads.decode()
    T, H, D = w.total_tokens, w.num_heads, w.head_dim

    def idx(a):
        return torch.from_numpy(np.asarray(a, dtype=np.uint32).view(np.int32).copy()).to(dev)

    bt, sp, sl = idx(w.block_table), idx(w.seq_ptr), idx(w.seq_lens)
    g = torch.Generator(device=dev).manual_seed(10)
    src = torch.randn((T, H, D), generator=g, device=dev).to(torch.float16)
    pool = torch.empty((w.num_pages, w.page_size, H, D), dtype=torch.int8, device=dev)
    sc = torch.zeros(w.num_pages * w.page_size, device=dev)
    zp = torch.zeros(w.num_pages * w.page_size, dtype=torch.uint8, device=dev)
    ws = torch.empty(max(hp.workspace_bytes(hp.Descriptor(pool, bt, sp, sl), T), 256),
                     dtype=torch.uint8, device=dev)
    forms = {}
    for name, pool_t, z in (("int8_symmetric", pool, None),
                            ("uint8_zero_points", pool.view(torch.uint8), zp)):
        qd = hp.Descriptor(pool_t, bt, sp, sl, scales=sc)
        forms[name] = (qd, z, T * H * D * 3 + 4 * T + (T if z is not None else 0))
    times = {name: [] for name in forms}
    for r in range(rounds):
        order = list(forms) if r % 2 == 0 else list(forms)[::-1]
        for name in order:
            qd, z, _ = forms[name]

            def call():
                hp.scatter_quant(qd, src, zero_points=z, workspace=ws, stream=stream)

            call()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                call()
            b.record(stream)
            b.synchronize()
            times[name].append(a.elapsed_time(b) / reps)
    res = {}
    for name, (_, _, nbytes) in forms.items():
        ms = float(np.median(times[name]))
        res[name] = {"algorithmic_bytes": nbytes, "launch_us": round(ms * 1e3, 1),
                     "gb_per_s": round(nbytes / (ms / 1e3) / 1e9, 1),
                     "rounds_us": [round(t * 1e3, 1) for t in times[name]]}
    del pool, src
    return res


def summarize_quant_write(trace_dir, fetch_dir, write_dir):
    """Kernel durations and calibrated HBM traffic of the quantize-on-scatter
    kernels (bench.py --quant-write-only runs) into profiles/."""
    import numpy as np
    import workloads
    w = workloads.decode()
    T, n = w.total_tokens, w.num_heads * w.head_dim
    algo = {0: 3 * T * n + 4 * T, 1: 3 * T * n + 5 * T}  # by the kernel's asymmetric bit

    def asym_of(name):
        # QM template argument = source * 2 + asymmetric; the f16 source is 0
        return int(name.rstrip(">").rsplit(",", 1)[1]) & 1

    trace = _csv_rows(trace_dir, "*kernel_trace.csv")
    groups = {}
    for r in trace:
        name = _short(r["Kernel_Name"])
        if "(hp::Op)3" not in name:
            continue
        groups.setdefault(name, []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel durations: quantize-on-scatter, decode batch (rocprofv3 kernel trace)", "",
             "Command (from the repository root, on one MI355X):", "", f"    {QW_TRACE_CMD}", "",
             "The decode batch's fp16 rows (63,540 tokens, 32 heads x 128) quantized into an",
             "int8 pool (symmetric: a scale per slot) and a uint8 pool (a scale and a zero point",
             "per slot), each call made 21 times. Durations in microseconds.", "",
             "| kernel | calls | avg us | min us | max us | algorithmic GB | GB/s at avg |",
             "|---|---|---|---|---|---|---|"]
    for name, ts in sorted(groups.items()):
        nbytes = algo[asym_of(name)]
        lines.append(f"| `{name}` | {len(ts)} | {np.mean(ts):.1f} | {min(ts):.1f} | "
                     f"{max(ts):.1f} | {nbytes / 1e9:.4f} | {nbytes / (np.mean(ts) * 1e3):.0f} |")
    with open(os.path.join(PROFILES, "quant_write_decode_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    fetch = _csv_rows(fetch_dir, "*counter_collection.csv")
    write = _csv_rows(write_dir, "*counter_collection.csv")
    ff = CALIBRATION_BYTES / (_calibration(fetch, "FETCH_SIZE") * 1024)
    wf = CALIBRATION_BYTES / (_calibration(write, "WRITE_SIZE") * 1024)

    def per_launch(rows, counter):
        agg = {}
        for r in rows:
            name = _short(r["Kernel_Name"])
            if r["Counter_Name"] == counter and "(hp::Op)3" in name:
                agg.setdefault(name, []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}

    fk, wk = per_launch(fetch, "FETCH_SIZE"), per_launch(write, "WRITE_SIZE")
    out = ["# HBM traffic per launch: quantize-on-scatter, decode batch (rocprofv3 counters)", "",
           "Two counter passes, each in its own run (commands from the repository root):", "",
           f"    {QW_PMC_CMD.format(c='FETCH_SIZE', d='fetch')}",
           f"    {QW_PMC_CMD.format(c='WRITE_SIZE', d='write')}", "",
           "Calibrated with three plain 1 GiB device copies in the same runs: bytes =",
           f"FETCH_SIZE x 1024 x {ff:.4f} and WRITE_SIZE x 1024 x {wf:.4f}.",
           "Algorithmic bytes: every fp16 row read once, its int8 codes written once, and",
           "4 bytes of scale (plus 1 of zero point) written per token.", "",
           "| kernel | read GB | write GB | total GB | algorithmic GB |", "|---|---|---|---|---|"]
    for name in sorted(fk):
        if name not in wk:
            continue
        rb, wb = fk[name] * 1024 * ff, wk[name] * 1024 * wf
        out.append(f"| `{name}` | {rb / 1e9:.4f} | {wb / 1e9:.4f} | {(rb + wb) / 1e9:.4f} | "
                   f"{algo[asym_of(name)] / 1e9:.4f} |")
    with open(os.path.join(PROFILES, "quant_write_decode_hbm_traffic.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(lines + [""] + out))


# ---- batched moves (optional) ----------------------------------------------------

def attention_extras(hp, torch, np, dev, stream, reps, gqa8=False):
    """Decode attention reading K and V through the block table: the decode
    batch (64 sequences, 32 kv heads x 128 fp16, one query head per kv head,
    streaming loads) and the prefix-sharing batch (256 sequences, 8 kv heads x
    128 bf16, 32 query heads, cached loads since 64 prefix pages are read by
    every sequence); with gqa8, the prefix batch with 64 query heads and the
    decode batch with 128 (four per kv head, matrix cores) too, and three of
    the workloads over int8 pools with per-slot scales (hp_paged_attention_q8,
    bf16 queries).
    Algorithmic bytes: every live K and V row read once (the prefix pages once
    per sequence that uses them, as logical bytes), with int8 pools each
    row's scale once, the queries read and the fp32 output written."""
    import workloads
    res = {}
    cases = [("decode_mha_f16", workloads.decode(), 1, True, False),
             ("prefix_gqa4_bf16", workloads.prefix(), 4, False, False)]
    if gqa8:
        cases.append(("prefix_gqa8_bf16", workloads.prefix(), 8, False, False))
        cases.append(("decode_gqa4_f16", workloads.decode(), 4, True, False))
        cases.append(("decode_mha_int8", workloads.decode(), 1, True, True))
        cases.append(("decode_gqa4_int8", workloads.decode(), 4, True, True))
        cases.append(("prefix_gqa4_int8", workloads.prefix(), 4, False, True))
    for name, w, group, streaming, q8 in cases:
        if q8:
            w = dataclasses.replace(w, dtype="i8", values="int8", with_scales=True)
        vw = dataclasses.replace(w, seed=w.seed * 7 + 3)
        k_pool, v_pool = w.make_pool(dev), vw.make_pool(dev)
        k_sc = w.make_scales(dev) if q8 else None
        v_sc = vw.make_scales(dev) if q8 else None

        def idx(a):
            return torch.from_numpy(np.asarray(a, dtype=np.uint32).view(np.int32).copy()).to(dev)

        desc = hp.Descriptor(k_pool, idx(w.block_table), idx(w.seq_ptr), idx(w.seq_lens),
                             scales=k_sc)
        T, S, H, D = w.total_tokens, w.num_seqs, w.num_heads, w.head_dim
        Hq = H * group
        g = torch.Generator(device=dev).manual_seed(9)
        q = torch.randn((S, Hq, D), generator=g, device=dev).to(
            torch.bfloat16 if q8 else k_pool.dtype)
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
        ws = torch.empty(hp.attention_workspace_bytes(desc, T, Hq), dtype=torch.uint8, device=dev)
        L = hp.lib()
        pd = desc.with_tokens(T)
        tail = (q.data_ptr(), Hq, ctypes.c_float(1.0 / D ** 0.5), out.data_ptr(),
                hp.DTYPE["f32"], ws.data_ptr(), ws.numel(),
                hp.HP_FLAG_STREAM if streaming else 0, stream.cuda_stream)
        if q8:
            args = (pd, v_pool.data_ptr(), v_sc.data_ptr()) + tail
            fn, fname = L.hp_paged_attention_q8, "hp_paged_attention_q8"
        else:
            args = (pd, v_pool.data_ptr()) + tail
            fn, fname = L.hp_paged_attention, "hp_paged_attention"

        def call():
            if fn(*args) != 0:
                raise SystemExit(f"{fname} failed")

        call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            call()
        b.record(stream)
        b.synchronize()
        ms = a.elapsed_time(b) / reps
        eb = 1 if q8 else 2
        row = H * D * eb + (4 if q8 else 0)   # one slot's K (or V) bytes, with its scale
        nbytes = 2 * T * row + S * Hq * D * 2 + S * Hq * D * 4
        unique = (len(np.unique(w.block_table)) * w.page_size * row * 2 if not streaming
                  else None)
        res[name] = {"sequences": S, "tokens": T, "kv_heads": H, "q_heads": Hq, "head_dim": D,
                     "kv_dtype": "int8 + fp32 scale per slot" if q8 else w.dtype,
                     "algorithmic_bytes": nbytes, "launch_us": round(ms * 1e3, 1),
                     "gb_per_s": round(nbytes / (ms / 1e3) / 1e9, 1),
                     "tokens_per_s": round(T / (ms / 1e3), 1)}
        if unique is not None:
            # the bytes a call must move at least when every distinct page is
            # read once: the rate against the 8 TB/s roofline
            ub = unique + S * Hq * D * 2 + S * Hq * D * 4
            res[name]["unique_kv_bytes"] = unique
            res[name]["unique_gb_per_s"] = round(ub / (ms / 1e3) / 1e9, 1)
            res[name]["unique_frac_of_8tbs"] = round(ub / (ms / 1e3) / 8e12, 3)
            # the same call reusing a plan made once (hp_attention_plan, then
            # HP_FLAG_PLANNED): what each layer after the first costs
            if L.hp_attention_plan(pd, Hq, ws.data_ptr(), ws.numel(), 0, stream.cuda_stream):
                raise SystemExit("hp_attention_plan failed")
            args = args[:-2] + (args[-2] | hp.HP_FLAG_PLANNED, args[-1])
            call()
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                call()
            b.record(stream)
            b.synchronize()
            pms = a.elapsed_time(b) / reps
            res[name]["planned_launch_us"] = round(pms * 1e3, 1)
            res[name]["planned_unique_frac_of_8tbs"] = round(ub / (pms / 1e3) / 8e12, 3)
        del k_pool, v_pool, q, out, ws, k_sc, v_sc
        torch.cuda.empty_cache()
    return res


def batched_append(hp, torch, np, dev, stream, reps):
    """One decode step's KV append for a 32-layer model: each of the decode
    batch's 64 sequences writes one new token (8 KV heads x 128 bf16) at its
    current length, into each of 64 pools (32 layers x {K, V}) that share one
    block table. 64 single hp_scatter calls against one hp_scatter_batch."""
    import workloads
    dec = workloads.decode()
    prior = dec.seq_lens.astype(np.int64)
    pages = (prior + 1 + 15) // 16
    rng = np.random.default_rng(5)
    n_pages = int(pages.sum()) + 64
    bt = rng.permutation(n_pages)[: int(pages.sum())].astype(np.uint32)
    sp = np.concatenate([[0], np.cumsum(pages)]).astype(np.uint32)

    def idx(a):
        return torch.from_numpy(np.asarray(a, dtype=np.uint32).view(np.int32).copy()).to(dev)

    S, H, D, layers = 64, 8, 128, 32
    tbt, tsp, tsl, tss = idx(bt), idx(sp), idx(np.ones(S)), idx(prior)
    pools = [torch.empty((n_pages, 16, H, D), dtype=torch.bfloat16, device=dev)
             for _ in range(2 * layers)]
    srcs = [torch.randn((S, H, D), device=dev).to(torch.bfloat16) for _ in pools]
    descs = [hp.Descriptor(p, tbt, tsp, tsl) for p in pools]
    if hp.validate(descs[0], S, tss) != ("HP_OK", 0):
        raise SystemExit("batched append descriptor failed validation")
    L = hp.lib()
    sh = stream.cuda_stream
    pds = [d.with_tokens(S) for d in descs]
    parr = (ctypes.c_void_p * len(pools))(*[p.data_ptr() for p in pools])
    sarr = (ctypes.c_void_p * len(srcs))(*[x.data_ptr() for x in srcs])
    src_p = [x.data_ptr() for x in srcs]
    ss_p = tss.data_ptr()
    flags = hp.HP_FLAG_ZERO_TAIL

    def singles():
        for pd, sp_ in zip(pds, src_p):
            if L.hp_scatter(pd, sp_, ss_p, None, 0, flags, sh) != 0:
                raise SystemExit("hp_scatter failed")

    def batched():
        if L.hp_scatter_batch(pds[0], len(pools), parr, sarr, ss_p, None, 0, flags, sh) != 0:
            raise SystemExit("hp_scatter_batch failed")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / reps

    t_single, t_batch = timed(singles), timed(batched)
    end = prior + 1
    tail_rows = int(((-end) % 16).sum())
    moved = len(pools) * (2 * S * H * D * 2 + tail_rows * H * D * 2)
    return {"workload": "decode-step KV append: 64 sequences x 1 token, 8 KV heads x 128 "
                        "bf16, 32 layers x {K, V} = 64 pools sharing one block table, "
                        "tails zeroed",
            "pools": len(pools), "algorithmic_bytes": moved,
            "single_calls_us": round(t_single * 1e3, 1),
            "batched_call_us": round(t_batch * 1e3, 1),
            "speedup": round(t_single / t_batch, 2),
            "batched_gb_per_s": round(moved / (t_batch / 1e3) / 1e9, 1)}


# ---- the benchmark -------------------------------------------------------------

def calibration_copies(torch, dev):
    """Three plain 1 GiB device copies: the counter runs' calibration."""
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    del a, b


def rocprof_gather():
    """The gather kernel's rocprof averages from the committed summary, when it
    was taken on the current kernel sources: over every launch of the
    profiled run, over its step launches, and over its back-to-back
    launches (the ones the event timing uses)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    algo = t.get("algorithmic_bytes_per_launch", 1041039360)
    out = {}
    for key, name in (("rocprof_avg_launch_us", "all"), ("rocprof_avg_step_us", "step"),
                      ("rocprof_avg_back_to_back_us", "back_to_back")):
        us = t.get(key)
        if us:
            gbs = algo / (us * 1e-6) / 1e9
            out[f"rocprof_{name}_avg_ms"] = round(us / 1e3, 4)
            out[f"rocprof_{name}_frac"] = round(gbs / HBM_PEAK_GBS, 4)
    if out:
        out["rocprof_from"] = os.path.relpath(TRAFFIC_FILE, ROOT)
    return out


def side_paths(hp, torch, np, dev, stream, args, w, wq, desc, qdesc, pool):
    """The side paths on the decode batch's pools: copy-on-write page copy,
    dequant under each quantization scheme, quantize-on-scatter, decode
    attention, and the batched KV append."""
    T, H, D = w.total_tokens, w.num_heads, w.head_dim

    def idx(a):
        return idx_on(torch, np, np.asarray(a).astype(np.uint32), dev)

    def back_to_back(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        a.record(stream)
        for _ in range(args.kernel_reps):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / args.kernel_reps

    # copy-on-write page copy: 1,024 referenced pages of the decode pool
    # (128 KiB each) into pages no sequence references
    free_pages = np.setdiff1d(np.arange(w.num_pages), w.block_table.astype(np.int64))
    rng = np.random.default_rng(6)
    n_copy = 1024
    src_p = idx(rng.choice(w.block_table.astype(np.int64), n_copy, replace=False))
    dst_p = idx(rng.choice(free_pages, n_copy, replace=False))
    t_copy = back_to_back(lambda: hp.copy_pages(desc, src_p, dst_p, stream=stream))
    copy_bytes = 2 * n_copy * 16 * H * D * 2
    # dequant-gather of the int8 pool under each quantization scheme, with
    # zero points (the general kernel); per-slot is the step's
    qout = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    zrng = np.random.default_rng(8)
    schemes = {}
    for name, scheme, axis, n_par, per_tok in (
            ("per_tensor_zp", "per_tensor", 0, 1, 0),
            ("per_channel_head_zp", "per_channel", 1, H, 0),
            ("per_channel_head_dim_zp", "per_channel", 2, D, 0),
            ("per_block_affine_zp", "per_block_affine", 0, wq.num_pages * 16, 5)):
        sc = torch.from_numpy(zrng.uniform(1e-3, 1e-1, n_par).astype(np.float32)).to(dev)
        zp = torch.from_numpy(zrng.integers(-128, 128, n_par).astype(np.int8)).to(dev)
        t_q = back_to_back(lambda: hp.gather_dequant_q(qdesc, qout, scheme, sc, axis=axis,
                                                       zero_points=zp, stream=stream))
        qb = T * H * D * 3 + per_tok * T
        schemes[name] = {"algorithmic_bytes": qb, "launch_us": round(t_q * 1e3, 1),
                         "gb_per_s": round(qb / (t_q / 1e3) / 1e9, 1)}
    del qout
    return {
        "quantize_on_scatter": quant_write_extras(hp, torch, np, dev, stream,
                                                  args.kernel_reps),
        "attention": attention_extras(hp, torch, np, dev, stream, args.kernel_reps, gqa8=True),
        "dequant_schemes": schemes,
        "batched_append": batched_append(hp, torch, np, dev, stream, args.kernel_reps),
        "copy_pages": {"workload": "1,024 pages of the decode pool (16 x 32 x 128 fp16 = "
                                   "128 KiB each) copied to unreferenced pages",
                       "algorithmic_bytes": copy_bytes, "launch_us": round(t_copy * 1e3, 1),
                       "gb_per_s": round(copy_bytes / (t_copy / 1e3) / 1e9, 1)}}


FLUSH_BYTES = 1 << 30  # read between flushed iterations: evicts L2 and the MALL


def idx_on(torch, np, a, dev):
    """An index array (uint32 / uint64) as a device tensor of the same width."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32).copy()).to(dev)
    return torch.from_numpy(a.astype(np.uint64).view(np.int64).copy()).to(dev)


class OnGpu:
    """A workload's descriptor tensors (pool, table, offsets, counts, starts,
    optional scales) on the GPU, and the binding's descriptor over them."""

    def __init__(self, hp, torch, np, w, dev, pool=None, scales=False):
        self.pool = w.make_pool(dev) if pool is None else pool
        self.bt = idx_on(torch, np, w.block_table.astype(w.index_dtype), dev)
        self.sp = idx_on(torch, np, w.seq_ptr.astype(w.index_dtype), dev)
        self.sl = idx_on(torch, np, w.seq_lens.astype(w.index_dtype), dev)
        self.ss = (idx_on(torch, np, w.seq_start.astype(w.index_dtype), dev)
                   if w.seq_start is not None else None)
        self.scales = w.make_scales(dev) if scales else None
        self.desc = hp.Descriptor(self.pool, self.bt, self.sp, self.sl, scales=self.scales)


def flushed_times(torch, np, stream, call, iters, flush):
    """Durations (us) of `call` over `iters` iterations; before each, the
    1 GiB buffer `flush` is read through (a sum), then HIP events on the
    call's stream bracket the call alone. A read leaves the L2s and the
    Infinity Cache holding clean flush lines: the previous call's dirty
    lines are written back during the flush, not during the timed call (a
    write flush would leave up to 256 MB of dirty lines for the call to
    write back)."""
    call()
    torch.cuda.synchronize()
    words = flush.view(torch.int64)
    pairs = []
    for _ in range(iters):
        words.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) * 1e3 for a, b in pairs])


def move_summary(np, nbytes, tokens, us, **extra_bytes):
    """Median / p10 / p90 of flushed durations, with GB/s and tokens/s at the
    median. extra_bytes: other byte counts of the same move (reported as GB/s
    at the median under their own names)."""
    med = float(np.median(us))
    p10, p90 = (float(x) for x in np.percentile(us, [10, 90]))
    gbs = nbytes / (med * 1e-6) / 1e9
    r = {"algorithmic_bytes": int(nbytes), "iterations": len(us), "median_us": round(med, 2),
         "p10_us": round(p10, 2), "p90_us": round(p90, 2), "gb_per_s": round(gbs, 1),
         "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
         "tokens_per_s": round(tokens / (med * 1e-6), 1)}
    for name, b in extra_bytes.items():
        r[name] = {"bytes": int(b), "gb_per_s": round(b / (med * 1e-6) / 1e9, 1)}
    return r


def token_slots(w, s0=0, s1=None):
    """Flat pool slot (phys * P + t mod P) of every token of sequences [s0, s1)."""
    import numpy as np
    s1 = w.num_seqs if s1 is None else s1
    lens = w.seq_lens[s0:s1].astype(np.int64)
    if lens.sum() == 0:
        return np.zeros(0, np.int64)
    seq = np.repeat(np.arange(s0, s1), lens)
    first = np.repeat(np.concatenate([[0], np.cumsum(lens)[:-1]]), lens)
    t = np.arange(int(lens.sum())) - first
    start = (w.seq_start[s0:s1].astype(np.int64) if w.seq_start is not None
             else np.zeros(s1 - s0, np.int64))
    t = t + np.repeat(start, lens)
    phys = w.block_table[w.seq_ptr.astype(np.int64)[seq] + t // w.page_size].astype(np.int64)
    return phys * w.page_size + t % w.page_size


def tail_rows(w, s0=0, s1=None):
    """Slots a tail-zeroing scatter clears: past each written sequence's last
    new token, to the end of that page."""
    import numpy as np
    s1 = w.num_seqs if s1 is None else s1
    lens = w.seq_lens[s0:s1].astype(np.int64)
    start = (w.seq_start[s0:s1].astype(np.int64) if w.seq_start is not None
             else np.zeros(s1 - s0, np.int64))
    r = (start + lens) % w.page_size
    return int(np.where((lens > 0) & (r != 0), w.page_size - r, 0).sum())


def measure_configs(hp, torch, np, dev, iters, cpu_seconds, with_cpu):
    """Each workload and the moves it names, timed with a 1 GiB flush between
    iterations (median, p10, p90), and the oracle timed on the host on the
    same work (single thread on a bounded prefix; all cores on everything)."""
    import oracle
    import workloads
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    L = hp.lib()
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    res = {}
    keep = []

    def workspace(desc, T):
        """The workspace the binding would pass: hp_workspace_bytes (the plan
        arrays of moves over many sequences, the validator's words)."""
        ws = torch.empty(max(hp.workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
        keep.append(ws)
        return ws.data_ptr(), ws.numel()

    def ok(code, what):
        if code != 0:
            raise SystemExit(f"{what}: {hp.status_str(code)}")

    def host(t):
        eb = t.element_size()
        return (t.contiguous().view(workloads.bits_dtype(eb)).cpu().numpy()
                .view(workloads.np_bits_dtype(eb)))

    def free():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    # -- tiny: gather to [114, 4, 8], scatter back into a blank pool
    w = workloads.tiny()
    g = OnGpu(hp, torch, np, w, dev)
    T, R = w.total_tokens, w.row_bytes
    out = torch.empty((T, w.num_heads, w.head_dim), dtype=g.pool.dtype, device=dev)
    g2 = OnGpu(hp, torch, np, w, dev, pool=torch.zeros_like(g.pool))
    pd, pb, o_p = g.desc.with_tokens(T), g2.desc.with_tokens(T), out.data_ptr()
    wsp, wsn = workspace(g.desc, T)
    e = {"workload": "tiny: 3 sequences of 40, 24, 50 tokens, page_size 16, 20-page pool, "
                     "4 heads x 8 fp16; gather to [114, 4, 8] and scatter it back",
         "tokens": T, "sequences": w.num_seqs,
         "gather": move_summary(np, 2 * T * R, T, flushed_times(
             torch, np, stream, lambda: ok(L.hp_gather(pd, o_p, wsp, wsn, 0, sh), "gather"),
             iters, flush)),
         "scatter": move_summary(np, 2 * T * R, T, flushed_times(
             torch, np, stream, lambda: ok(L.hp_scatter(pb, o_p, None, wsp, wsn, 0, sh),
                                           "scatter"), iters, flush))}
    if with_cpu:
        ph = host(g.pool)

        def run(s0, s1):
            kw = sub_desc(w, s0, s1)
            o = oracle.gather(ph, **kw)
            oracle.scatter(np.zeros_like(ph), o, **kw)
        e["cpu_oracle"] = cpu_legs(w, run, lambda s0, s1: 4 * int(
            w.seq_lens[s0:s1].astype(np.int64).sum()) * R, cpu_seconds)
    res["tiny"] = e
    del g, g2, out
    free()

    # -- decode: gather (streaming hint), scatter, int8 -> bf16 dequant
    w = workloads.decode()
    g = OnGpu(hp, torch, np, w, dev)
    T, R, HD = w.total_tokens, w.row_bytes, w.num_heads * w.head_dim
    wq = dataclasses.replace(w, name="decode-int8", dtype="i8", values="int8", with_scales=True)
    gq = OnGpu(hp, torch, np, wq, dev, scales=True)
    out = torch.empty((T, w.num_heads, w.head_dim), dtype=torch.float16, device=dev)
    qout = torch.empty((T, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    pd, pq, o_p, q_p = g.desc.with_tokens(T), gq.desc.with_tokens(T), out.data_ptr(), qout.data_ptr()
    wsp, wsn = workspace(g.desc, T)
    bf16 = hp.DTYPE["bf16"]
    res["decode"] = {
        "workload": "decode batch: 64 sequences, lengths uniform 1..2048, page_size 16, 32 "
                    "heads x 128 fp16, 12,000-page pool, uint32 table of unique pages; dequant "
                    "over an int8 copy with one fp32 scale per slot",
        "tokens": T, "sequences": w.num_seqs,
        "gather": move_summary(np, 2 * T * R, T, flushed_times(
            torch, np, stream,
            lambda: ok(L.hp_gather(pd, o_p, wsp, wsn, hp.HP_FLAG_STREAM, sh), "gather"),
            iters, flush)),
        "scatter": move_summary(np, 2 * T * R, T, flushed_times(
            torch, np, stream, lambda: ok(L.hp_scatter(pd, o_p, None, wsp, wsn, 0, sh),
                                          "scatter"), iters, flush)),
        "dequant": move_summary(np, 3 * T * HD + 4 * T, T, flushed_times(
            torch, np, stream, lambda: ok(L.hp_gather_dequant(pq, q_p, bf16, wsp, wsn, 0, sh),
                                          "dequant"), iters, flush))}
    del g, gq, out, qout
    free()

    # -- prefix: gather of 256 sequences that alias 64 leading pages
    w = workloads.prefix()
    g = OnGpu(hp, torch, np, w, dev)
    T, R = w.total_tokens, w.row_bytes
    out = torch.empty((T, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    pd, o_p = g.desc.with_tokens(T), out.data_ptr()
    wsp, wsn = workspace(g.desc, T)
    uniq = len(np.unique(token_slots(w)))
    us = flushed_times(torch, np, stream,
                       lambda: ok(L.hp_gather(pd, o_p, wsp, wsn, 0, sh), "gather"), iters, flush)
    e = {"workload": "prefix sharing: 256 sequences, a 1,024-token prefix on 64 shared pages "
                     "plus private suffixes of 16..512 tokens, page_size 16, 8 heads x 128 "
                     "bf16, 40,000-page pool; gather in logical order",
         "tokens": T, "sequences": w.num_seqs, "unique_rows_read": uniq,
         "gather": move_summary(np, (uniq + T) * R, T, us, logical=2 * T * R)}
    e["gather"]["bytes_counted"] = ("unique: each distinct pool row read once plus every "
                                    "output row written; logical: every row read per use")
    if with_cpu:
        ph = host(g.pool)
        e["cpu_oracle"] = cpu_legs(
            w, lambda s0, s1: oracle.gather(ph, **sub_desc(w, s0, s1)),
            lambda s0, s1: (len(np.unique(token_slots(w, s0, s1))) +
                            int(w.seq_lens[s0:s1].astype(np.int64).sum())) * R, cpu_seconds)
        del ph
    res["prefix"] = e
    del g, out
    free()

    # -- append: 512 one-token appends + an 8,192-token prefill, tails zeroed
    w = workloads.append()
    g = OnGpu(hp, torch, np, w, dev)
    T, R = w.total_tokens, w.row_bytes
    src = w.make_src(dev)
    pd, s_p, ss_p = g.desc.with_tokens(T), src.data_ptr(), g.ss.data_ptr()
    wsp, wsn = workspace(g.desc, T)
    nt = tail_rows(w)
    us = flushed_times(torch, np, stream, lambda: ok(L.hp_scatter(
        pd, s_p, ss_p, wsp, wsn, hp.HP_FLAG_ZERO_TAIL, sh), "scatter"), iters, flush)
    e = {"workload": "append: 512 decode sequences writing 1 token each into their partial "
                     "trailing page plus one 8,192-token prefill into fresh pages, page_size "
                     "16, 8 heads x 128 bf16, 60,000-page pool, unused trailing slots zeroed",
         "tokens": T, "sequences": w.num_seqs, "tail_rows_zeroed": nt,
         "scatter": move_summary(np, 2 * T * R + nt * R, T, us)}
    if with_cpu:
        ph = host(g.pool)
        sh_src = host(src)
        tok = np.concatenate([[0], np.cumsum(w.seq_lens.astype(np.int64))])

        def run(s0, s1):
            oracle.scatter(ph, sh_src[tok[s0]: tok[s1]], zero_tail=True, in_place=True,
                           **sub_desc(w, s0, s1))
        e["cpu_oracle"] = cpu_legs(
            w, run, lambda s0, s1: (2 * int(w.seq_lens[s0:s1].astype(np.int64).sum())
                                    + tail_rows(w, s0, s1)) * R, cpu_seconds)
        del ph, sh_src
    res["append"] = e
    del g, src
    free()

    # -- quant: int8 pool of 200,000 pages, per-slot scales, uint64 table
    w = workloads.quant()
    g = OnGpu(hp, torch, np, w, dev, scales=True)
    T, HD = w.total_tokens, w.num_heads * w.head_dim
    qout = torch.empty((T, w.num_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    pd, q_p = g.desc.with_tokens(T), qout.data_ptr()
    wsp, wsn = workspace(g.desc, T)
    us = flushed_times(torch, np, stream, lambda: ok(L.hp_gather_dequant(
        pd, q_p, bf16, wsp, wsn, 0, sh), "dequant"), iters, flush)
    e = {"workload": "quantized large pool: int8, 200,000 pages x 16 x 8 x 128, one fp32 scale "
                     "per slot, uint64 table, 1,024 sequences with log-normal lengths capped "
                     "at 8,192; gather + dequant to bf16",
         "tokens": T, "sequences": w.num_seqs,
         "dequant": move_summary(np, 3 * T * HD + 4 * T, T, us)}
    del qout
    free()
    raw = torch.empty((T, w.num_heads, w.head_dim), dtype=torch.int8, device=dev)
    r_p = raw.data_ptr()
    e["raw_gather"] = move_summary(np, 2 * T * HD, T, flushed_times(
        torch, np, stream, lambda: ok(L.hp_gather(pd, r_p, wsp, wsn, hp.HP_FLAG_STREAM, sh),
                                      "gather"), iters, flush))
    del raw
    free()
    if with_cpu:
        ph = host(g.pool).view(np.int8)
        sc = g.scales.cpu().numpy()
        e["cpu_oracle"] = cpu_legs(
            w, lambda s0, s1: oracle.gather_dequant(ph, sc, **sub_desc(w, s0, s1)),
            lambda s0, s1: (3 * HD + 4) * int(w.seq_lens[s0:s1].astype(np.int64).sum()),
            cpu_seconds)
        del ph, sc
    res["quant"] = e
    del g, flush
    free()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="single-thread oracle budget per workload (a bounded prefix)")
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="back-to-back launches per kernel for the launch durations")
    ap.add_argument("--flush-iters", type=int, default=50,
                    help="flushed iterations per move in the per-workload table")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload table (profiling runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 1 GiB device copies (counter calibration runs)")
    ap.add_argument("--extras", action="store_true",
                    help="also measure the side paths (schemes, attention, batched append, "
                         "page copy, quantize-on-scatter)")
    ap.add_argument("--no-reference-copies", action="store_true",
                    help="skip the identity-table gather and runtime copy (profiling runs)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE", "FETCH", "WRITE"))
    ap.add_argument("--attention-only", action="store_true",
                    help="only the decode-attention measurements (profiling runs)")
    ap.add_argument("--summarize-attention", nargs=3, metavar=("TRACE", "FETCH", "WRITE"))
    ap.add_argument("--quant-write-only", action="store_true",
                    help="only the quantize-on-scatter measurements (profiling runs)")
    ap.add_argument("--summarize-quant-write", nargs=3, metavar=("TRACE", "FETCH", "WRITE"))
    ap.add_argument("--summarize-counters", nargs=len(COUNTER_PASSES),
                    metavar=tuple(k.upper() for k in COUNTER_PASSES))
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.summarize_profiles:
        summarize_profiles(*args.summarize_profiles)
        return
    if args.summarize_attention:
        summarize_attention(*args.summarize_attention)
        return
    if args.summarize_quant_write:
        summarize_quant_write(*args.summarize_quant_write)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} (WORLD_SIZE {world}) requested, but the "
              "benchmark measures one GPU only: the block-paged path has no multi-GPU code "
              "(it would shard by heads, with no exchange, or by sequences).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    import block_table_gather_amd as hp

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.attention_only:
        if args.copy_calibration:
            calibration_copies(torch, dev)
        stream = torch.cuda.current_stream(dev)
        print(json.dumps({"attention": attention_extras(hp, torch, np, dev, stream,
                                                        args.kernel_reps, gqa8=True)}),
              flush=True)
        return
    if args.quant_write_only:
        if args.copy_calibration:
            calibration_copies(torch, dev)
        stream = torch.cuda.current_stream(dev)
        print(json.dumps({"quantize_on_scatter": quant_write_extras(
            hp, torch, np, dev, stream, args.kernel_reps)}), flush=True)
        return
    w = workloads.decode()
    T, S, K = w.total_tokens, w.num_seqs, w.num_block_entries
    H, D = w.num_heads, w.head_dim

    def idx(a):
        return idx_on(torch, np, a.astype(np.uint32), dev)

    g = OnGpu(hp, torch, np, w, dev)
    pool, desc = g.pool, g.desc
    wq = dataclasses.replace(w, name="decode-int8", dtype="i8", values="int8",
                             with_scales=True)
    gq = OnGpu(hp, torch, np, wq, dev, scales=True)
    qpool, scales, qdesc = gq.pool, gq.scales, gq.desc
    out = torch.empty((T, H, D), dtype=torch.float16, device=dev)
    qout = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    main_s = torch.cuda.current_stream(dev)
    if hp.validate(desc, T) != ("HP_OK", 0):
        raise SystemExit("bench descriptor failed validation")

    # Arguments marshalled once; each call below is one C-ABI call.
    L = hp.lib()
    sh = main_s.cuda_stream
    pd, pq = desc.with_tokens(T), qdesc.with_tokens(T)
    o_p, q_p = out.data_ptr(), qout.data_ptr()
    bf16 = hp.DTYPE["bf16"]
    G = hp.HP_FLAG_GATED

    # Each step checks its descriptor with hp_validate_async on the moves'
    # stream and the moves are gated on the verdict: no host round trip sits
    # between steps, and a rejected descriptor would be moved by no kernel.
    # (Checking the next step's descriptor on a second stream, with events
    # ordering the moves after their check, measured slower: 531 against
    # 475 us of kernels at 20 steps; the check alone takes about 4 us.)
    ws = torch.empty(max(hp.workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
    wsp, wsn = ws.data_ptr(), ws.numel()

    def do_validate():
        if L.hp_validate_async(pd, None, wsp, wsn, sh) != 0:
            raise SystemExit("hp_validate_async failed")

    def do_gather():
        if L.hp_gather(pd, o_p, wsp, wsn, hp.HP_FLAG_STREAM | G, sh) != 0:
            raise SystemExit("hp_gather failed")

    def do_scatter():
        if L.hp_scatter(pd, o_p, None, wsp, wsn, G, sh) != 0:
            raise SystemExit("hp_scatter failed")

    def do_dequant():
        if L.hp_gather_dequant(pq, q_p, bf16, wsp, wsn, G, sh) != 0:
            raise SystemExit("hp_gather_dequant failed")

    moves = [("gather", do_gather), ("scatter", do_scatter), ("dequant", do_dequant)]

    def run_steps(n):
        for _ in range(n):
            do_validate()
            for _, fn in moves:
                fn()

    if args.copy_calibration:
        calibration_copies(torch, dev)

    # A fresh process's first steps run slower, and the step time keeps
    # falling for about 40 ms of load (a kernel trace of 55 steps after the
    # launch-timing pass: 500 us for the first timed step, ~478 for the next
    # twenty, ~472 from the 40th on). So one pass of the per-kernel launch
    # timings (discarded), the reference copies and about 50 ms of untimed
    # steps run before the W warm-up steps and the timed ones, and the kept
    # launch timings after them.
    def back_to_back(fn, s=main_s):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        a.record(s)
        for _ in range(args.kernel_reps):
            fn()
        b.record(s)
        b.synchronize()
        return a.elapsed_time(b) / args.kernel_reps

    # Launch durations: back-to-back launches of each step kernel (gated, as
    # in the step) between two events on its stream.
    def launch_times():
        t = {n: back_to_back(fn) for n, fn in moves}
        t["validate"] = back_to_back(do_validate)
        return t

    do_validate()  # the gated moves read this verdict (a fresh workspace holds none)
    launch_times()

    # Reference copies of the gather's bytes: the same gather kernel on an
    # identity table (one sequence over pages 0..K-1: a contiguous copy) and
    # the runtime's plain device-to-device copy.
    refs = None
    if not args.no_reference_copies:
        ident = hp.Descriptor(pool, idx(np.arange(K)), idx(np.array([0, K])),
                              idx(np.array([K * 16])))
        ident_out = torch.empty((K * 16, H, D), dtype=torch.float16, device=dev)
        pi, io_p = ident.with_tokens(K * 16), ident_out.data_ptr()
        ident_bytes = 2 * K * 16 * H * D * 2
        copy_src = pool.view(-1)[: K * 16 * H * D]
        copy_dst = ident_out.view(-1)
        t_ident = back_to_back(lambda: L.hp_gather(pi, io_p, None, 0, hp.HP_FLAG_STREAM, sh))
        t_copy = back_to_back(lambda: copy_dst.copy_(copy_src))
        refs = {"identity_table_gather": round(ident_bytes / (t_ident / 1e3) / 1e9, 1),
                "runtime_device_copy": round(ident_bytes / (t_copy / 1e3) / 1e9, 1),
                "unit": "GB/s", "bytes": ident_bytes}
        del ident_out

    run_steps(PRE_STEPS)  # about 50 ms of the step, untimed
    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    verdict = hp.validate_verdict(desc, T, ws)
    if verdict != ("HP_OK", 0):
        raise SystemExit(f"the step's verdict: {verdict}")
    launch_ms = launch_times()

    nbytes = step_bytes(T, S, K, H, D)
    total_bytes = sum(nbytes.values())
    value = total_bytes / (ms_per_step / 1e3) / 1e9
    ops = {}
    for n in ("validate", "gather", "scatter", "dequant"):
        ms = launch_ms[n]
        gbs = nbytes[n] / (ms / 1e3) / 1e9
        ops[n] = {"algorithmic_bytes": nbytes[n], "launch_ms": round(ms, 4)}
        if n != "validate":
            ops[n].update({"gb_per_s": round(gbs, 1),
                           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
    kernel_sum = sum(launch_ms.values())
    g_achieved = nbytes["gather"] / (launch_ms["gather"] / 1e3) / 1e9
    roof = {"bound": "hbm", "kernel": GATHER_KERNEL + " (gather)",
            "achieved": round(g_achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(g_achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(),
            "algorithmic_bytes_per_launch": nbytes["gather"],
            "avg_launch_ms": round(launch_ms["gather"], 4),
            "avg_launch_from": "HIP events around back-to-back launches on the launch stream"}
    prof = rocprof_gather()
    if prof:
        roof.update(prof)
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "untimed_pre_steps": PRE_STEPS,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode batch: 64 sequences, lengths uniform 1..2048, "
                               "page_size 16, 32 heads x 128 fp16, 12,000-page pool, uint32 "
                               "block table of unique pages (gather with the streaming "
                               "hint); step = enqueue-only validation + gather + scatter + "
                               "int8->bf16 dequant-gather of the same table, the moves gated "
                               "on the device by the verdict",
                   "total_tokens": T, "num_seqs": S, "block_table_entries": K,
                   "step_algorithmic_bytes": total_bytes},
        "tokens_per_s": round(T / (ms_per_step / 1e3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kernel_sum_ms": round(kernel_sum, 4),
        "step_over_kernel_sum": round(ms_per_step / kernel_sum, 4),
        "ops": ops,
        "reference_copies": refs,
        "roofline": roof,
    }
    if args.extras:
        result["extras"] = side_paths(hp, torch, np, dev, main_s, args, w, wq, desc, qdesc,
                                      pool)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        pool_h = pool.view(torch.int16).cpu().numpy().view(np.uint16)
        qpool_h = qpool.cpu().numpy()
        scales_h = scales.cpu().numpy()

        def run(s0, s1):
            kw = sub_desc(w, s0, s1)
            Ts = int(w.seq_lens[s0:s1].astype(np.int64).sum())
            oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages,
                            page_size=w.page_size, block_table=kw["block_table"],
                            seq_ptr=kw["seq_ptr"], seq_lens=kw["seq_lens"], total_tokens=Ts)
            o = oracle.gather(pool_h, **kw)
            oracle.scatter(pool_h, o, in_place=True, **kw)
            oracle.gather_dequant(qpool_h, scales_h, **kw)

        def step_b(s0, s1):
            kw = sub_desc(w, s0, s1)
            Ts = int(w.seq_lens[s0:s1].astype(np.int64).sum())
            return sum(step_bytes(Ts, s1 - s0, len(kw["block_table"]), H, D).values())
        legs = cpu_legs(w, run, step_b, args.cpu_seconds)
        allc = legs["all_cores"]
        cpu = {"value": allc["value"], "unit": "GB/s", "cores": allc["cores"], "kind": "oracle",
               "sample": "the decode step (validate + gather + scatter + dequant-gather) on all "
                         f"{S} sequences, split into {allc['cores']} balanced ranges run by one "
                         "host thread each; single_thread: one thread on a prefix",
               "seconds": allc["seconds"], "tokens_per_s": allc["tokens_per_s"],
               "single_thread": legs["single_thread"],
               "affinity_cores": legs["affinity_cores"], "cpu_model": legs["cpu_model"]}
        del pool_h, qpool_h, scales_h
    result["cpu_baseline"] = cpu
    del g, gq, out, qout, pool, qpool, desc, qdesc
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = measure_configs(hp, torch, np, dev, args.flush_iters,
                                            args.cpu_seconds, not args.no_cpu_baseline)
        if cpu is not None:
            result["configs"]["decode"]["cpu_oracle"] = {
                k: cpu[k] for k in ("single_thread", "affinity_cores", "cpu_model")}
            result["configs"]["decode"]["cpu_oracle"]["all_cores"] = {
                k: cpu[k] for k in ("value", "unit", "cores", "seconds", "tokens_per_s")}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
