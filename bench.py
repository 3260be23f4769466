#!/usr/bin/env python3
"""Throughput of the block-paged hot path on one MI355X.

One step is one pass of every stage of the path over one batch of the decode
workload (64 sequences, lengths uniform in 1..2048, page_size 16, 32 heads x
128 fp16, 12,000-page pool, uint32 block table of unique pages):

  1. hp_validate        storage invariants of the descriptor (synchronous, on a
                        second stream: the next step's descriptor is checked
                        while this step's moves run, and the next moves are
                        enqueued only after that check returned HP_OK);
  2. hp_gather          pool -> logical [T, 32, 128] fp16 tensor (streaming hint:
                        the table names each page once);
  3. hp_scatter         that tensor back into its slots (the write direction);
  4. hp_gather_dequant  the same table over an int8 copy of the pool with one
                        fp32 scale per slot -> bf16 [T, 32, 128].

Inputs are resident in HBM before timing starts. `value` is the step's
algorithmic bytes (each live row read once and written once per move, one
scale per row, the validator's metadata reads) over the wall-clock step time
(K steps bracketed by device synchronisation), in GB/s (1 GB = 1e9 B).

Per-kernel launch durations come from HIP events on the launch stream around
back-to-back launches of each kernel (the GPU stays busy, so the interval is
kernel time); `roofline` uses the gather kernel's. The per-stage times inside
the step (`ops[*].in_step_ms`) are event intervals on the moves' stream, and
the host's wall time of each hp_validate call, taken in a separate run of 20
steps after the timed ones (events between the moves would slow the timed
steps). The CPU oracle is timed on the host on a
bounded prefix of the same batch (single-threaded, as it stands).

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
  python bench.py --summarize-profiles TRACE_DIR FETCH_DIR WRITE_DIR
      (writes the rocprofv3 summaries under profiles/)
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
TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_trace -o trace -- "
             "python3 bench.py --steps 50 --warmup 5 --no-cpu-baseline --no-reference-copies")
PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d gpurun_out/prof_{d} -o {d} -- "
           "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --no-reference-copies "
           "--copy-calibration")
ATTN_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_attn_trace -o trace "
                  "-- python3 bench.py --attention-only")
ATTN_PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d gpurun_out/prof_attn_{d} -o {d} -- "
                "python3 bench.py --attention-only --kernel-reps 3 --copy-calibration")
QW_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof_qw_trace -o trace "
                "-- python3 bench.py --quant-write-only")
QW_PMC_CMD = ("rocprofv3 --pmc {c} -f csv -d gpurun_out/prof_qw_{d} -o {d} -- "
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


def cpu_baseline(w, pool_h, qpool_h, scales_h, seconds):
    """The oracle, single-threaded, on the longest prefix of sequences that fits
    the time budget; returns GB/s of the same algorithmic bytes."""
    import numpy as np
    import oracle
    lens = w.seq_lens.astype(np.int64)
    kw = dict(page_size=w.page_size, num_heads=w.num_heads, head_dim=w.head_dim)

    def run(n):
        sp = w.seq_ptr[: n + 1]
        bt = w.block_table[: int(sp[-1])]
        sl = w.seq_lens[:n]
        T = int(lens[:n].sum())
        t0 = time.perf_counter()
        oracle.validate(rank=3, paged_axis=0, num_pages=w.num_pages, page_size=w.page_size,
                        block_table=bt, seq_ptr=sp, seq_lens=sl, total_tokens=T)
        out = oracle.gather(pool_h, block_table=bt, seq_ptr=sp, seq_lens=sl, **kw)
        oracle.scatter(pool_h, out, block_table=bt, seq_ptr=sp, seq_lens=sl, in_place=True,
                       **kw)
        oracle.gather_dequant(qpool_h, scales_h, block_table=bt, seq_ptr=sp, seq_lens=sl, **kw)
        return time.perf_counter() - t0, T, n, len(bt)

    n = 1
    dt, T, n, K = run(n)
    while dt < seconds / 8 and n < w.num_seqs:
        n = min(w.num_seqs, n * 4)
        dt, T, n, K = run(n)
    if dt < seconds / 2 and n < w.num_seqs:
        target_T = T * seconds / dt
        n = max(1, min(int(np.searchsorted(np.cumsum(lens), target_T)) + 1, w.num_seqs))
        dt, T, n, K = run(n)
    b = sum(step_bytes(T, n, K, w.num_heads, w.head_dim).values())
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 2), "tokens_per_s": round(T / dt, 1),
            "sample": f"first {n} of {w.num_seqs} sequences ({T} of {w.total_tokens} tokens), "
                      "one step: validate + gather + scatter + dequant-gather, single thread"}


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

    stats = one(trace_dir, "*kernel_stats.csv")
    lines = ["# Kernel durations: decode-batch bench step (rocprofv3 kernel trace)", "",
             "Command (from the repository root, on one MI355X):", "",
             f"    {TRACE_CMD}", "",
             "All launches of the run (50 timed + 5 warm-up steps, plus the back-to-back",
             "kernel-timing launches of each move). Durations in microseconds.", "",
             "| kernel | what | calls | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    gather_avg = None
    for r in stats:
        short = _short(r["Name"])
        if short not in KERNEL_LABELS:
            continue
        avg = float(r["AverageNs"]) / 1e3
        if short == GATHER_KERNEL:
            gather_avg = avg
        lines.append(f"| `{short}` | {KERNEL_LABELS[short]} | {r['Calls']} | {avg:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines += ["", "The validator runs on a second stream beside the moves (the next step's",
              "check), so its durations include time it shares the GPU with them; alone it",
              "takes the minimum shown.",
              "", "Other kernels in the trace are PyTorch's input generation (random values,",
              "fills, index_put) and the runtime's copies; they are outside the timed step."]
    with open(os.path.join(PROFILES, "decode_step_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

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


def summarize_attention(trace_dir, fetch_dir, write_dir):
    """Kernel durations and calibrated HBM traffic of the attention kernels
    (bench.py --attention-only runs) into profiles/."""
    import numpy as np
    import workloads
    algo = {}
    for w, group in ((workloads.decode(), 1), (workloads.prefix(), 4)):
        Hq = w.num_heads * group
        algo[w.dtype] = (w.name, 2 * w.total_tokens * w.num_heads * w.head_dim * 2
                         + w.num_seqs * Hq * w.head_dim * 6)
    lines = ["# Kernel durations: decode attention through the block table (rocprofv3)", "",
             "Command (from the repository root, on one MI355X):", "", f"    {ATTN_TRACE_CMD}", "",
             "The decode batch (64 sequences, 32 kv heads x 128 f16, one query head per kv",
             "head, streaming loads) and the prefix-sharing batch (256 sequences, 8 kv heads",
             "x 128 bf16, 32 query heads), each called 21 times. Durations in microseconds;",
             "the combine kernel's rows are per workload (grid size).", "",
             "| kernel | calls | avg us | min us | max us | algorithmic GB | GB/s at avg |",
             "|---|---|---|---|---|---|---|"]
    trace = _csv_rows(trace_dir, "*kernel_trace.csv")
    groups = {}
    for r in trace:
        if "attention" not in r["Kernel_Name"]:
            continue
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]))
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    for (name, grid), ts in sorted(groups.items()):
        gb = gbs = ""
        if name.startswith(("attention_kernel<", "attention_mfma_kernel<")):
            wl, nbytes = algo["bf16" if "BF16" in name else "f16"]
            gb = f"{nbytes / 1e9:.4f}"
            gbs = f"{nbytes / (np.mean(ts) * 1e3):.0f}"
        lines.append(f"| `{name}` (grid {grid}) | {len(ts)} | {np.mean(ts):.1f} | {min(ts):.1f} | "
                     f"{max(ts):.1f} | {gb} | {gbs} |")
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
           "the L2's traffic to the fabric, Infinity Cache hits included: the prefix batch's",
           "64 shared pages are read by every sequence but mostly served by the caches.",
           "Algorithmic bytes: every live K and V row read once (shared prefix pages once per",
           "sequence), the queries read and the fp32 output written. The attention kernels'",
           "writes are the per-unit partial results the combine kernel reads.", "",
           "| kernel | read GB | write GB | algorithmic GB |", "|---|---|---|---|"]
    for key in sorted(fk):
        if key not in wk:
            continue
        name = key[0]
        rb, wb = fk[key] * 1024 * ff, wk[key] * 1024 * wf
        gb = ""
        if name.startswith(("attention_kernel<", "attention_mfma_kernel<")):
            gb = f"{algo['bf16' if 'BF16' in name else 'f16'][1] / 1e9:.4f}"
        out.append(f"| `{name}` (grid {key[1]}) | {rb / 1e9:.4f} | {wb / 1e9:.4f} | {gb} |")
    with open(os.path.join(PROFILES, "attention_decode_prefix_hbm_traffic.md"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(lines + [""] + out))


def quant_write_extras(hp, torch, np, dev, stream, reps):
    """Quantize-on-scatter on the decode batch: its fp16 rows (63,540 tokens,
    32 heads x 128) written into an int8 pool (symmetric, a scale per slot)
    and a uint8 pool (a scale and a zero point per slot). Algorithmic bytes:
    every row read (2 bytes a value) and its codes written (1 byte a value),
    plus 4 bytes of scale (and 1 of zero point) per token."""
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
    res = {}
    for name, pool_t, z in (("int8_symmetric", pool, None),
                            ("uint8_zero_points", pool.view(torch.uint8), zp)):
        qd = hp.Descriptor(pool_t, bt, sp, sl, scales=sc)

        def call():
            hp.scatter_quant(qd, src, zero_points=z, workspace=ws, stream=stream)

        call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            call()
        b.record(stream)
        b.synchronize()
        ms = a.elapsed_time(b) / reps
        nbytes = T * H * D * 3 + 4 * T + (T if z is not None else 0)
        res[name] = {"algorithmic_bytes": nbytes, "launch_us": round(ms * 1e3, 1),
                     "gb_per_s": round(nbytes / (ms / 1e3) / 1e9, 1)}
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
    every sequence); with gqa8, the prefix batch with 64 query heads too.
    Algorithmic bytes: every live K and V row read once (the prefix pages once
    per sequence that uses them, as logical bytes), the queries read and the
    fp32 output written."""
    import workloads
    res = {}
    cases = [("decode_mha_f16", workloads.decode(), 1, True),
             ("prefix_gqa4_bf16", workloads.prefix(), 4, False)]
    if gqa8:
        cases.append(("prefix_gqa8_bf16", workloads.prefix(), 8, False))
    for name, w, group, streaming in cases:
        k_pool = w.make_pool(dev)
        v_pool = dataclasses.replace(w, seed=w.seed * 7 + 3).make_pool(dev)

        def idx(a):
            return torch.from_numpy(np.asarray(a, dtype=np.uint32).view(np.int32).copy()).to(dev)

        desc = hp.Descriptor(k_pool, idx(w.block_table), idx(w.seq_ptr), idx(w.seq_lens))
        T, S, H, D = w.total_tokens, w.num_seqs, w.num_heads, w.head_dim
        Hq = H * group
        g = torch.Generator(device=dev).manual_seed(9)
        q = torch.randn((S, Hq, D), generator=g, device=dev).to(k_pool.dtype)
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
        ws = torch.empty(hp.attention_workspace_bytes(desc, T, Hq), dtype=torch.uint8, device=dev)
        L = hp.lib()
        pd = desc.with_tokens(T)
        args = (pd, v_pool.data_ptr(), q.data_ptr(), Hq, ctypes.c_float(1.0 / D ** 0.5),
                out.data_ptr(), hp.DTYPE["f32"], ws.data_ptr(), ws.numel(),
                hp.HP_FLAG_STREAM if streaming else 0, stream.cuda_stream)

        def call():
            if L.hp_paged_attention(*args) != 0:
                raise SystemExit("hp_paged_attention failed")

        call()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            call()
        b.record(stream)
        b.synchronize()
        ms = a.elapsed_time(b) / reps
        nbytes = 2 * T * H * D * 2 + S * Hq * D * 2 + S * Hq * D * 4
        unique = (len(np.unique(w.block_table)) * w.page_size * H * D * 2 * 2 if not streaming
                  else None)
        res[name] = {"sequences": S, "tokens": T, "kv_heads": H, "q_heads": Hq, "head_dim": D,
                     "algorithmic_bytes": nbytes, "launch_us": round(ms * 1e3, 1),
                     "gb_per_s": round(nbytes / (ms / 1e3) / 1e9, 1),
                     "tokens_per_s": round(T / (ms / 1e3), 1)}
        if unique is not None:
            res[name]["unique_kv_bytes"] = unique
        del k_pool, v_pool, q, out, ws
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="back-to-back launches per kernel for the launch durations")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run plain 1 GiB device copies (counter calibration runs)")
    ap.add_argument("--extras", action="store_true",
                    help="also measure the batched calls (decode-step KV append over 64 pools)")
    ap.add_argument("--no-reference-copies", action="store_true",
                    help="skip the identity-table gather and runtime copy (profiling runs)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE", "FETCH", "WRITE"))
    ap.add_argument("--attention-only", action="store_true",
                    help="only the decode-attention measurements (profiling runs)")
    ap.add_argument("--summarize-attention", nargs=3, metavar=("TRACE", "FETCH", "WRITE"))
    ap.add_argument("--quant-write-only", action="store_true",
                    help="only the quantize-on-scatter measurements (profiling runs)")
    ap.add_argument("--summarize-quant-write", nargs=3, metavar=("TRACE", "FETCH", "WRITE"))
    args = ap.parse_args()
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
        print(f"bench.py: --gpus {args.gpus} (WORLD_SIZE {world}) requested, but this build "
              "measures one GPU only: the block-paged path has no multi-GPU code (see the "
              "sharding notes in DESIGN.md).", file=sys.stderr)
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
                                                        args.kernel_reps)}), flush=True)
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
        return torch.from_numpy(a.astype(np.uint32).view(np.int32).copy()).to(dev)

    pool = w.make_pool(dev)
    bt, sp, sl = idx(w.block_table), idx(w.seq_ptr), idx(w.seq_lens)
    desc = hp.Descriptor(pool, bt, sp, sl)
    wq = dataclasses.replace(w, name="decode-int8", dtype="i8", values="int8",
                             with_scales=True)
    qpool = wq.make_pool(dev)
    scales = wq.make_scales(dev)
    qdesc = hp.Descriptor(qpool, bt, sp, sl, scales=scales)
    out = torch.empty((T, H, D), dtype=torch.float16, device=dev)
    qout = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(hp.workspace_bytes(desc, T), 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    if hp.validate(desc, T, workspace=ws) != ("HP_OK", 0):
        raise SystemExit("bench descriptor failed validation")

    # Arguments marshalled once; each call below is one C-ABI call.
    L = hp.lib()
    sh = stream.cuda_stream
    pd, pq = desc.with_tokens(T), qdesc.with_tokens(T)
    wsp, wsn = ws.data_ptr(), ws.numel()
    res_mem = torch.zeros(ctypes.sizeof(hp.HpValidateResult), dtype=torch.uint8,
                          pin_memory=True)  # pinned: the check writes its result here
    res = hp.HpValidateResult.from_address(res_mem.data_ptr())
    pres = ctypes.byref(res)
    o_p, q_p = out.data_ptr(), qout.data_ptr()
    bf16 = hp.DTYPE["bf16"]

    # The validator runs on a stream of its own with its own workspace, so
    # that checking the next step's descriptor overlaps this step's moves (as
    # a serving loop would); the moves still start only after their
    # descriptor's check has returned HP_OK.
    vstream = torch.cuda.Stream(dev)
    vws = torch.empty(256, dtype=torch.uint8, device=dev)
    vsh, vwsp, vwsn = vstream.cuda_stream, vws.data_ptr(), vws.numel()

    def do_validate():
        if L.hp_validate(pd, None, vwsp, vwsn, pres, vsh) != 0:
            raise SystemExit(f"hp_validate: {hp.status_str(res.code)}")

    def do_gather():
        if L.hp_gather(pd, o_p, wsp, wsn, hp.HP_FLAG_STREAM, sh) != 0:
            raise SystemExit("hp_gather failed")

    def do_scatter():
        if L.hp_scatter(pd, o_p, None, wsp, wsn, 0, sh) != 0:
            raise SystemExit("hp_scatter failed")

    def do_dequant():
        if L.hp_gather_dequant(pq, q_p, bf16, wsp, wsn, 0, sh) != 0:
            raise SystemExit("hp_gather_dequant failed")

    stages = [("validate", do_validate), ("gather", do_gather), ("scatter", do_scatter),
              ("dequant", do_dequant)]
    moves = stages[1:]
    events, vtimes = [], []

    def run_steps(n, record):
        """n steps: validate step 1's descriptor, then for each step enqueue its
        moves and, while they run, validate the next step's descriptor."""
        t = time.perf_counter()
        do_validate()
        if record:
            vtimes.append(time.perf_counter() - t)
        for k in range(n):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
            for i, (_, fn) in enumerate(moves):
                if record:
                    ev[i].record(stream)
                fn()
            if record:
                ev[3].record(stream)
                events.append(ev)
            if k + 1 < n:
                t = time.perf_counter()
                do_validate()
                if record:
                    vtimes.append(time.perf_counter() - t)

    if args.copy_calibration:
        calibration_copies(torch, dev)

    run_steps(args.warmup, False)
    torch.cuda.synchronize()
    # The timed steps carry no instrumentation: timing events recorded between
    # the moves cost about 18 us a step on this path (measured), so the
    # per-stage breakdown comes from a separate, untimed run of the same steps.
    t0 = time.perf_counter()
    run_steps(args.steps, False)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    run_steps(min(args.steps, 20), True)
    torch.cuda.synchronize()
    in_step_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events]))
                  for i, (n, _) in enumerate(moves)}
    in_step_ms["validate"] = float(np.mean(vtimes)) * 1e3  # host wall time of the call

    # Launch durations: back-to-back launches of each kernel between two events.
    launch_ms = {}
    for n, fn in stages[1:]:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        a.record(stream)
        for _ in range(args.kernel_reps):
            fn()
        b.record(stream)
        b.synchronize()
        launch_ms[n] = a.elapsed_time(b) / args.kernel_reps

    # Reference copies of the gather's bytes: the same gather kernel on an
    # identity table (one sequence over pages 0..K-1: a contiguous copy) and
    # the runtime's plain device-to-device copy.
    ident = hp.Descriptor(pool, idx(np.arange(K)), idx(np.array([0, K])), idx(np.array([K * 16])))
    ident_out = torch.empty((K * 16, H, D), dtype=torch.float16, device=dev)
    pi, io_p = ident.with_tokens(K * 16), ident_out.data_ptr()

    def ident_gather():
        if L.hp_gather(pi, io_p, wsp, wsn, hp.HP_FLAG_STREAM, sh) != 0:
            raise SystemExit("hp_gather (identity table) failed")

    def back_to_back(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fn()
        a.record(stream)
        for _ in range(args.kernel_reps):
            fn()
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / args.kernel_reps

    refs = None
    if not args.no_reference_copies:
        ident_bytes = 2 * K * 16 * H * D * 2
        copy_src = pool.view(-1)[: K * 16 * H * D]
        copy_dst = ident_out.view(-1)
        t_ident = back_to_back(ident_gather)
        t_copy = back_to_back(lambda: copy_dst.copy_(copy_src))
        refs = {"identity_table_gather": round(ident_bytes / (t_ident / 1e3) / 1e9, 1),
                "runtime_device_copy": round(ident_bytes / (t_copy / 1e3) / 1e9, 1),
                "unit": "GB/s", "bytes": ident_bytes}
    del ident_out

    nbytes = step_bytes(T, S, K, H, D)
    total_bytes = sum(nbytes.values())
    value = total_bytes / (ms_per_step / 1e3) / 1e9
    ops = {}
    for n, _ in stages:
        ms = launch_ms.get(n)
        ops[n] = {"in_step_ms": round(in_step_ms[n], 4), "algorithmic_bytes": nbytes[n]}
        if ms is not None:
            gbs = nbytes[n] / (ms / 1e3) / 1e9
            ops[n].update({"launch_ms": round(ms, 4), "gb_per_s": round(gbs, 1),
                           "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
    g_achieved = nbytes["gather"] / (launch_ms["gather"] / 1e3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode batch: 64 sequences, lengths uniform 1..2048, "
                               "page_size 16, 32 heads x 128 fp16, 12,000-page pool, uint32 "
                               "block table of unique pages (gather with the streaming "
                               "hint); step = validate + gather + scatter + "
                               "int8->bf16 dequant-gather of the same table (the next "
                               "step's validation runs on a second stream beside the "
                               "moves)",
                   "total_tokens": T, "num_seqs": S, "block_table_entries": K,
                   "step_algorithmic_bytes": total_bytes},
        "tokens_per_s": round(T / (ms_per_step / 1e3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "ops": ops,
        "reference_copies": refs,
        "roofline": {"bound": "hbm", "kernel": GATHER_KERNEL + " (gather)",
                     "achieved": round(g_achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(g_achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(),
                     "algorithmic_bytes_per_launch": nbytes["gather"],
                     "avg_launch_ms": round(launch_ms["gather"], 4)},
    }
    if args.extras:
        # copy-on-write page copy: 1,024 referenced pages of the decode pool
        # (128 KiB each) into pages no sequence references
        free = np.setdiff1d(np.arange(w.num_pages), w.block_table.astype(np.int64))
        rng = np.random.default_rng(6)
        n_copy = 1024
        src_p = idx(rng.choice(w.block_table.astype(np.int64), n_copy, replace=False))
        dst_p = idx(rng.choice(free, n_copy, replace=False))
        t_copy = back_to_back(lambda: hp.copy_pages(desc, src_p, dst_p, stream=stream))
        copy_bytes = 2 * n_copy * 16 * H * D * 2
        # dequant-gather of the step's int8 pool under each quantization
        # scheme, with zero points (the general kernel); per-slot is the step's
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
        result["extras"] = {
            "quantize_on_scatter": quant_write_extras(hp, torch, np, dev, stream,
                                                      args.kernel_reps),
            "attention": attention_extras(hp, torch, np, dev, stream, args.kernel_reps,
                                          gqa8=True),
            "dequant_schemes": schemes,
            "batched_append": batched_append(hp, torch, np, dev, stream, args.kernel_reps),
            "copy_pages": {"workload": "1,024 pages of the decode pool (16 x 32 x 128 fp16 = "
                                       "128 KiB each) copied to unreferenced pages",
                           "algorithmic_bytes": copy_bytes, "launch_us": round(t_copy * 1e3, 1),
                           "gb_per_s": round(copy_bytes / (t_copy / 1e3) / 1e9, 1)}}
    if not args.no_cpu_baseline:
        pool_h = pool.view(torch.int16).cpu().numpy().view(np.uint16)
        qpool_h = qpool.cpu().numpy()
        scales_h = scales.cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(w, pool_h, qpool_h, scales_h, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
