#!/usr/bin/env python3
"""Throughput of the block-paged hot path on one MI355X.

One step is one pass of every stage of the path over one batch of the decode
workload (64 sequences, lengths uniform in 1..2048, page_size 16, 32 heads x
128 fp16, 12,000-page pool, uint32 block table):

  1. hp_validate        storage invariants of the descriptor (synchronous);
  2. hp_gather          pool -> logical [T, 32, 128] fp16 tensor;
  3. hp_scatter         that tensor back into its slots (the write direction);
  4. hp_gather_dequant  the same table over an int8 copy of the pool with one
                        fp32 scale per slot -> bf16 [T, 32, 128].

Inputs are resident in HBM before timing starts. `value` is the step's
algorithmic bytes (each live row read once and written once per move, scales,
metadata read by the validator) over the measured step time, in GB/s
(1 GB = 1e9 B). Per-stage kernel times come from HIP events recorded on the
launch stream around each call. The CPU oracle is timed on the host on a
bounded prefix of the same batch (single-threaded, as it stands).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
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
KERNEL_SRC = os.path.join(ROOT, "block_table_gather_amd", "csrc", "hp_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gather_copy_kernel_decode_traffic.json")


def kernel_source_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def step_bytes(T, S, K, H, D, idx_bytes=4):
    """Algorithmic bytes of one step (see module docstring)."""
    row = H * D * 2                      # fp16 row
    gather = 2 * T * row                 # read each live row once, write it once
    scatter = 2 * T * row
    dequant = T * H * D + 4 * T + T * H * D * 2   # int8 rows + one scale per row + bf16 rows
    validate = idx_bytes * (K + (S + 1) + S)      # block table, seq_ptr, seq_lens
    return {"validate": validate, "gather": gather, "scatter": scatter, "dequant": dequant}


def traffic_for(launch_count_bytes):
    """HBM bytes per gather launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, pool_h, qpool_h, scales_h, seconds):
    """The oracle, single-threaded, on the longest prefix of sequences that fits
    the time budget; returns GB/s of the same algorithmic bytes."""
    import numpy as np
    import oracle
    lens = w.seq_lens.astype(np.int64)
    # estimate from the first sequence, then take a prefix of ~`seconds`
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration runs)")
    args = ap.parse_args()
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

    names = ("validate", "gather", "scatter", "dequant")
    events = []

    def step(record):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)] if record else None
        if record:
            ev[0].record(stream)
        code = hp.validate(desc, T, workspace=ws, stream=stream)
        if code[0] != "HP_OK":
            raise SystemExit(f"validation failed: {code}")
        if record:
            ev[1].record(stream)
        hp.gather(desc, out, streaming=True, workspace=ws, stream=stream)
        if record:
            ev[2].record(stream)
        hp.scatter(desc, out, workspace=ws, stream=stream)
        if record:
            ev[3].record(stream)
        hp.gather_dequant(qdesc, qout, workspace=ws, stream=stream)
        if record:
            ev[4].record(stream)
            events.append(ev)

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    per_op_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events]))
                 for i, n in enumerate(names)}
    nbytes = step_bytes(T, S, K, H, D)
    total_bytes = sum(nbytes.values())
    value = total_bytes / (ms_per_step / 1e3) / 1e9
    ops = {n: {"ms": round(per_op_ms[n], 4),
               "gb_per_s": round(nbytes[n] / (per_op_ms[n] / 1e3) / 1e9, 1),
               "frac_of_hbm_peak": round(nbytes[n] / (per_op_ms[n] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
               "algorithmic_bytes": nbytes[n]} for n in names}
    g_achieved = nbytes["gather"] / (per_op_ms["gather"] / 1e3) / 1e9
    traffic = traffic_for(nbytes["gather"])
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
                               "int8->bf16 dequant-gather of the same table",
                   "total_tokens": T, "num_seqs": S, "block_table_entries": K,
                   "step_algorithmic_bytes": total_bytes},
        "tokens_per_s": round(T / (ms_per_step / 1e3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "ops": ops,
        "roofline": {"bound": "hbm",
                     "kernel": "copy_kernel (gather, fused, 16-byte vectors, streaming loads)",
                     "achieved": round(g_achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(g_achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": nbytes["gather"],
                     "avg_launch_ms": round(per_op_ms["gather"], 4)},
    }
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
