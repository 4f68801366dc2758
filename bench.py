#!/usr/bin/env python3
"""Benchmark of one paged-attention decode step on one MI355X.

A step is the whole hot path over one batch: ``pa_kv_append`` of this step's new
tokens into their pool slots, then ``pa_decode`` (split-context partitions and their
log-sum-exp merge). The default workload is the Llama-7B-layer-shaped decode batch:
256 sequences, context lengths U{128..2048}, 32 heads x 128, 16-token blocks, fp16,
physical blocks shuffled, one new token per sequence.

Printed: one JSON line with the KV-read rate (algorithmic bytes: every cached token's
K and V row once per step) over the whole step, seq-steps/s, the decode kernel's
roofline fraction against the 8 TB/s HBM peak, and the oracle's rate on the host
cores (measured before the GPU is touched).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_294_amd", "csrc", "pa_decode.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kv_read_bytes(inp) -> int:
    """Algorithmic KV bytes of a decode step: each context token's K and V rows once."""
    lens = inp.seq_lens[inp.num_prefill:].astype(np.int64)
    return int(lens.sum()) * 2 * inp.num_kv_heads * inp.head_size * 2


def source_digest(path) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(name, digest):
    """HBM traffic per launch from a committed rocprofv3 counter summary, if it still
    describes the current kernel source (else None)."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    kv = {}
    for ln in open(path, encoding="utf-8"):
        if ":" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != digest:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host cores, before any GPU call
# ---------------------------------------------------------------------------------------

_CPU = {}


def _cpu_worker(chunk):
    import oracle  # the oracle runs only in this leg of the benchmark
    inp, pool = _CPU["inp"], _CPU["pool"]
    q, bt, lens = inp.decode_part()
    oracle.decode(q[chunk], pool, bt[chunk], lens[chunk], inp.scale)
    return len(chunk)


def cpu_baseline(inp, max_cores):
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # noqa: BLE001 - thread limits are best effort
        pass
    cores = max(1, min(max_cores, len(os.sched_getaffinity(0))))
    t0 = time.perf_counter()
    pool = oracle.kv_append(inp.pool, inp.key_new, inp.value_new, inp.slot_mapping)
    t_append = time.perf_counter() - t0
    _CPU["inp"], _CPU["pool"] = inp, pool
    seqs = np.arange(inp.num_decode)
    chunks = [c for c in np.array_split(seqs, cores * 4) if len(c)]
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores) as workers:
        done = sum(workers.map(_cpu_worker, chunks))
    t_decode = time.perf_counter() - t0
    _CPU.clear()
    assert done == inp.num_decode
    t = t_append + t_decode
    return {
        "value": kv_read_bytes(inp) / t / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"whole step of the same batch: oracle kv_append of {len(inp.slot_mapping)} tokens "
                   f"(copies the pool, 1 core, {t_append:.2f} s) + oracle decode of all "
                   f"{inp.num_decode} sequences in fp64 over {cores} worker processes "
                   f"({t_decode:.2f} s)"),
        "seq_steps_per_s": inp.num_decode / t,
        "seconds": t,
    }


# ---------------------------------------------------------------------------------------
# GPU
# ---------------------------------------------------------------------------------------

def stream_read_gbps(torch, pkv, nbytes=4 << 30, reps=10):
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(pkv.pa_stream_read_sink_len(nbytes), dtype=torch.float32, device="cuda")
    for _ in range(3):
        pkv.pa_stream_read(buf, sink)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        pkv.pa_stream_read(buf, sink)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    del buf, sink
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def run_counter_sequence(inp, partition_size):
    """Dispatches for counter passes, in a fixed order: a torch copy of 1 GiB (reads and
    writes exactly 1 GiB: the calibration of FETCH_SIZE / WRITE_SIZE), pa_stream_read of
    1 GiB (reads 1 GiB), then three decode steps (kv_append + pa_decode)."""
    import torch
    import paged_kv_cache_294_amd as pkv

    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(pkv.pa_stream_read_sink_len(nbytes), dtype=torch.float32, device="cuda")
    pool = torch.from_numpy(inp.pool).cuda()
    q = torch.from_numpy(inp.q).cuda()
    bt = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.seq_lens).cuda()
    key = torch.from_numpy(inp.key_new).cuda()
    value = torch.from_numpy(inp.value_new).cuda()
    slots = torch.from_numpy(inp.slot_mapping).cuda()
    out = torch.empty_like(q)
    mcl = int(inp.seq_lens.max())
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    pkv.pa_stream_read(src, sink)
    torch.cuda.synchronize()
    for _ in range(3):
        pkv.pa_kv_append(pool, key, value, slots)
        pkv.pa_decode(out, q, pool, bt, lens, mcl, inp.scale, partition_size)
        torch.cuda.synchronize()
    log(f"counter sequence done: copy {nbytes} B, stream_read {nbytes} B, 3 decode steps; "
        f"decode algorithmic KV bytes per launch {kv_read_bytes(inp)}")


def summarize_trace(path, command):
    import csv
    rows = list(csv.DictReader(open(path)))
    print(f"# rocprofv3 kernel statistics\n# command: {command}")
    print(f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}")
    for r in rows:
        print(f"{r['Name'][:72]:<72} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
              f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
              f"{float(r['Percentage']):>6.2f}")


def summarize_counters(fetch_csv, write_csv, command):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the --mode counters sequence, scaled by
    the reading of the 1 GiB copy (the second 1 GiB dispatch reads and writes 1 GiB)."""
    import csv
    fetch = list(csv.DictReader(open(fetch_csv)))
    write = list(csv.DictReader(open(write_csv)))
    gib = float(1 << 30)
    # the 1 GiB device-to-device copy is the first dispatch that writes >= 1 GiB after the fills
    copy_i = next(i for i, r in enumerate(write)
                  if "copy" in r["Kernel_Name"].lower() and float(r["Counter_Value"]) * 1024 >= gib * 0.99)
    f_scale = gib / (float(fetch[copy_i]["Counter_Value"]) * 1024)
    w_scale = gib / (float(write[copy_i]["Counter_Value"]) * 1024)
    print(f"# rocprofv3 FETCH_SIZE / WRITE_SIZE passes of `bench.py --mode counters`")
    print(f"# command: {command}")
    print(f"# calibration: 1 GiB copy reads FETCH_SIZE={fetch[copy_i]['Counter_Value']} KiB, "
          f"WRITE_SIZE={write[copy_i]['Counter_Value']} KiB")
    print(f"fetch_scale: {f_scale:.5f}")
    print(f"write_scale: {w_scale:.5f}")
    per = {}
    for f, w in zip(fetch, write):
        name = f"{f['Kernel_Name'][:60]} [grid {f['Grid_Size']}]"
        rb = float(f["Counter_Value"]) * 1024 * f_scale
        wb = float(w["Counter_Value"]) * 1024 * w_scale
        per.setdefault(name, []).append((rb, wb))
    print(f"{'kernel':<72} {'n':>3} {'read_bytes':>14} {'write_bytes':>14}")
    for name, v in per.items():
        rb = sum(x[0] for x in v) / len(v)
        wb = sum(x[1] for x in v) / len(v)
        print(f"{name[:72]:<72} {len(v):>3} {rb:>14.0f} {wb:>14.0f}")
    dec = [sum(x[0] + x[1] for x in v) / len(v) for n, v in per.items()
           if "decode_partition_kernel" in n or "decode_reduce_kernel" in n]
    print(f"hbm_bytes_per_launch: {sum(dec):.0f}")
    print(f"kernel_source_sha256_16: {source_digest(DECODE_SRC)}")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--partition-size", type=int, default=512)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-read", action="store_true")
    ap.add_argument("--cpu-cores", type=int, default=16)
    ap.add_argument("--mode", choices=("bench", "counters"), default="bench",
                    help="counters: a short fixed dispatch sequence for rocprofv3 --pmc passes "
                         "(1 GiB torch copy, 1 GiB pa_stream_read, then 3 decode steps)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="print a profile summary of a rocprofv3 --stats kernel_stats.csv and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc passes of "
                         "--mode counters (FETCH_SIZE, then WRITE_SIZE) and exit")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path would shard by sequence or KV head with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    log("generating the 256-sequence decode batch (seed 2)")
    t0 = time.perf_counter()
    inp = workloads.config2()
    log(f"generated in {time.perf_counter() - t0:.1f}s: {inp.num_blocks} blocks, "
        f"sum L = {int(inp.seq_lens.sum())}")
    kv_bytes = kv_read_bytes(inp)

    if args.mode == "counters":
        run_counter_sequence(inp, args.partition_size)
        return

    cpu = None
    if not args.no_cpu_baseline:
        log("CPU baseline: oracle on the host cores")
        cpu = cpu_baseline(inp, args.cpu_cores)
        log(f"CPU baseline done in {cpu['seconds']:.1f}s on {cpu['cores']} cores")

    import torch
    import paged_kv_cache_294_amd as pkv

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    pkv.load()

    stream_gbps = None
    if not args.no_stream_read:
        stream_gbps = stream_read_gbps(torch, pkv)
        log(f"stream_read: {stream_gbps:.0f} GB/s")

    log("copying the batch to the GPU")
    pool = torch.from_numpy(inp.pool).cuda()
    q = torch.from_numpy(inp.q).cuda()
    bt = torch.from_numpy(inp.block_tables).cuda()
    lens = torch.from_numpy(inp.seq_lens).cuda()
    key = torch.from_numpy(inp.key_new).cuda()
    value = torch.from_numpy(inp.value_new).cuda()
    slots = torch.from_numpy(inp.slot_mapping).cuda()
    out = torch.empty_like(q)
    mcl = int(inp.seq_lens.max())
    ws_bytes = pkv.pa_decode_workspace_bytes(inp.num_seqs, inp.num_q_heads, mcl,
                                             args.partition_size, inp.head_size)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        pkv.pa_kv_append(pool, key, value, slots)
        if ev is not None:
            ev[1].record()
        pkv.pa_decode(out, q, pool, bt, lens, mcl, inp.scale, args.partition_size, ws)
        if ev is not None:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done; timing {args.steps} steps")

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(evs[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = start.elapsed_time(end) / args.steps
    append_ms = [e[0].elapsed_time(e[1]) for e in evs]
    decode_ms = [e[1].elapsed_time(e[2]) for e in evs]
    dec_avg = float(np.mean(decode_ms))
    log(f"step {ms_step:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms), decode {dec_avg:.3f} ms, "
        f"append {np.mean(append_ms) * 1e3:.1f} us")

    achieved = kv_bytes / (dec_avg * 1e-3) / 1e9
    nparts = pkv.pa_num_partitions(mcl, args.partition_size)
    digest = source_digest(DECODE_SRC)
    traffic = read_traffic("pa_decode_c2_counters.txt", digest)
    used_blocks = int(sum(-(-int(L) // 16) for L in inp.seq_lens))
    result = {
        "metric": "paged-attn decode KV-read GB/s (% of HBM peak) + seq-steps/s, 1 GPU",
        "value": kv_bytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "decode step: kv_append of 256 tokens + paged decode of 256 sequences, "
                        "context U{128..2048}, 32 heads x 128, block 16, fp16, shuffled blocks",
            "num_seqs": inp.num_seqs, "num_heads": inp.num_q_heads, "head_size": inp.head_size,
            "block_size": inp.block_size, "partition_size": args.partition_size,
            "partitions": nparts, "sum_context_tokens": int(inp.seq_lens.sum()), "seed": 2,
        },
        "pct_of_hbm_peak": 100.0 * kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "seq_steps_per_s": inp.num_seqs / (ms_step * 1e-3),
        "decode_ms": dec_avg,
        "append_us": float(np.mean(append_ms)) * 1e3,
        "roofline": {
            "kernel": "pa_decode" + (" (partition + log-sum-exp reduce kernels)" if nparts > 1
                                     else " (partition kernel)"),
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
        },
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in
                                                  ("value", "unit", "cores", "kind", "sample")},
        "stream_read_gbps": stream_gbps,
        "frac_of_stream_read": None if not stream_gbps else achieved / stream_gbps,
        "context": {
            "slot_utilisation": float(inp.seq_lens.sum()) / (used_blocks * 16),
            "gpu_cache_usage": used_blocks / inp.num_blocks,
        },
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
