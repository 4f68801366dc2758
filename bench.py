#!/usr/bin/env python3
"""Benchmark of one paged-attention step on one MI355X.

A step is the whole hot path over one batch: ``pa_kv_append`` of this step's new tokens
into their pool slots, ``pa_prefill_chunk`` for prefill chunks (mixed workload only) and
``pa_decode`` (split-context partitions and their log-sum-exp merge). Workloads:

  tiny                 4 decode sequences (1, 15, 16, 33 tokens), 4 heads x 64: launch-bound
  decode256 (default)  256 decode sequences, context U{128..2048}, 32 heads x 128, + append
  long32k              8 sequences x 32768 tokens, 32 x 128 (split-context partitions)
  prefix-groups        64 prompt groups x 4 samples sharing 64 blocks, 32q / 8kv heads x 128
  prefix-private       prefix-groups with private copies of the shared blocks
                       (grouped-query decode from HBM)
  mixed                8 prefill chunks of 512 over priors U{0..3584} + 248 decodes
                       U{256..4096}, append of all 4344 new tokens
  long-prefill         the last 512-row chunk of a 32768-token prompt + 8 decodes
                       U{256..4096} (few row tiles over a long context: the prefill's
                       context split)

The timed steps replay the step captured once into a HIP graph (``--launch graph``, the
default, as a serving engine runs it) or launch it call by call (``--launch eager``).

Timing: by default each timed step is bracketed by its own HIP events and followed by an
untimed 1 GiB read that flushes the L2 caches and the Infinity Cache (``--flush on``), so
no step starts with the previous one's blocks cached; the mean, median and min of those
per-step times are reported, and back-to-back steps without the flush beside them.

Printed: one JSON line. ``value`` is the KV-read rate of the step (algorithmic bytes:
every decode context token's K and V row once) over the mean step time; ``roofline``
is the step's dominant call: the decode against the 8 TB/s HBM peak, or, when the
prefill takes longer (long-prefill), the prefill against the fp16 matrix-core peak;
``cpu_baseline`` is the oracle on
the host cores, run before the GPU is touched.
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

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 matrix peak, vendor figure
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_294_amd", "csrc", "pa_decode.hip")

WORKLOADS = {  # name: (generator in workloads.WORKLOADS, description)
    "tiny": ("tiny", "tiny decode: 4 sequences of 1, 15, 16, 33 tokens over a 16-block pool, "
              "4 heads x 64, block 16, fp16 (launch-bound)"),
    "decode256": ("decode256", "decode step: kv_append of 256 tokens + paged decode of 256 sequences, "
              "context U{128..2048}, 32 heads x 128, block 16, fp16, shuffled blocks"),
    "long32k": ("long32k", "long-context decode: 8 sequences x 32768 tokens, 32 heads x 128, block 16, "
              "fp16, split-context partitions"),
    "prefix-groups": ("prefix-groups", "prefix-shared GQA decode: 64 groups x 4 samples, 1024-token shared prompt "
              "(64 blocks) + 64..256 private tokens, 32 q / 8 kv heads x 128, fp16"),
    "prefix-private": ("prefix-groups", "the prefix-groups batch with private copies of "
                       "every shared prefix block (no sharing): 256 GQA sequences of 1088..1280 tokens, 32 q / 8 kv heads x 128, fp16"),
    "mixed": ("mixed", "mixed step: kv_append of 4344 tokens + 8 prefill chunks of 512 over priors "
              "U{0..3584} + 248 decodes U{256..4096}, 32 heads x 128, fp16"),
    "long-prefill": ("long-prefill", "long-prompt step: kv_append of 520 tokens + the last 512-row "
                     "chunk of a 32768-token prompt + 8 decodes U{256..4096}, 32 heads x 128, fp16"),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------------------

def kv_read_bytes(inp, elem_bytes=2) -> int:
    """Decode KV bytes: each decode context token's K and V rows once (logical)."""
    lens = inp.seq_lens[inp.num_prefill:].astype(np.int64)
    return int(lens.sum()) * 2 * inp.num_kv_heads * inp.head_size * elem_bytes


def kv_unique_bytes(inp, elem_bytes=2) -> int:
    """Decode KV bytes counting each physical block's filled slots once (shared prefixes)."""
    row = 2 * inp.num_kv_heads * inp.head_size * elem_bytes
    seen = {}
    for b in range(inp.num_prefill, inp.num_seqs):
        L = int(inp.seq_lens[b])
        for j in range(-(-L // 16)):
            blk = int(inp.block_tables[b, j])
            seen[blk] = max(seen.get(blk, 0), min(16, L - 16 * j))
    return sum(seen.values()) * row


def prefill_flops(inp) -> int:
    """Causal pairs only: 4 * D * Hq * sum_r (C * P_r + C (C + 1) / 2)."""
    tot = 0
    for r in range(inp.num_prefill):
        C = int(inp.q_lens[r])
        P = int(inp.seq_lens[r]) - C
        tot += C * P + C * (C + 1) // 2
    return 4 * inp.head_size * inp.num_q_heads * tot


def append_bytes(inp, elem_bytes=2) -> int:
    """fp16 rows read, pool rows written (fp16 or one byte per FP8 element)."""
    return len(inp.slot_mapping) * 2 * inp.num_kv_heads * inp.head_size * (2 + elem_bytes)


def shares_blocks(inp) -> bool:
    used = [inp.block_tables[b, : -(-int(inp.seq_lens[b]) // 16)] for b in range(inp.num_seqs)]
    allb = np.concatenate(used) if used else np.zeros(0)
    return len(np.unique(allb)) < len(allb)


def source_digest(path) -> str:
    """Digest of a kernel source together with the shared device header and the build
    script (its compiler flags change the code as much as the source does)."""
    h = hashlib.sha256()
    for f in (path, os.path.join(os.path.dirname(path), "pa_device.h"),
              os.path.join(ROOT, "paged_kv_cache_294_amd", "build.py")):
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


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


def _cpu_decode(chunk):
    import oracle  # the oracle runs only in this leg of the benchmark
    inp, pool = _CPU["inp"], _CPU["pool"]
    q, bt, lens = inp.decode_part()
    oracle.decode(q[chunk], pool, bt[chunk], lens[chunk], inp.scale)
    return len(chunk)


def _cpu_prefill(rows):
    import oracle
    inp, pool = _CPU["inp"], _CPU["pool"]
    q, bt, qsl, lens = inp.prefill_part()
    oracle.prefill_chunk(q, pool, bt, qsl, lens, inp.scale, rows=set(rows))
    return len(rows)


def cpu_baseline(inp, max_cores, decode_seqs=None, prefill_every=8):
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
    nd = inp.num_decode if decode_seqs is None else min(decode_seqs, inp.num_decode)
    chunks = [c for c in np.array_split(np.arange(nd), cores * 4) if len(c)]
    ctx = mp.get_context("fork")
    # repeat the decode pass until about 12 s of CPU work (at most 4 passes), mean time
    passes, t_sum = 0, 0.0
    with ctx.Pool(cores) as workers:
        while True:
            t0 = time.perf_counter()
            done = sum(workers.map(_cpu_decode, chunks))
            t_sum += time.perf_counter() - t0
            passes += 1
            if passes >= 4 or t_sum * cores >= 12.0:
                break
    t_decode = t_sum / passes * inp.num_decode / nd
    sample = [f"oracle kv_append of {len(inp.slot_mapping)} tokens (copies the pool, 1 core, "
              f"{t_append:.2f} s)",
              f"oracle fp64 decode of {nd} of {inp.num_decode} sequences over {cores} worker "
              f"processes, mean of {passes} passes ({t_sum * cores:.0f} s of CPU work), time "
              f"scaled to all ({t_decode:.2f} s)"]
    t_prefill = 0.0
    if inp.num_prefill:
        total_q = inp.num_prefill_tokens
        rows = np.arange(0, total_q, prefill_every)
        parts = [list(map(int, c)) for c in np.array_split(rows, cores * 4) if len(c)]
        t0 = time.perf_counter()
        with ctx.Pool(cores) as workers:
            workers.map(_cpu_prefill, parts)
        t_prefill = (time.perf_counter() - t0) * total_q / len(rows)
        sample.append(f"oracle prefill of every {prefill_every}th of {total_q} chunk rows, "
                      f"time scaled to all rows ({t_prefill:.2f} s)")
    _CPU.clear()
    assert done == nd
    t = t_append + t_decode + t_prefill
    return {
        "value": kv_read_bytes(inp) / t / 1e9,
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "; ".join(sample),
        "seq_steps_per_s": inp.num_seqs / t,
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


def make_flush(torch, nbytes=1 << 30):
    """An untimed cache flush between timed steps: one read of a 1 GiB buffer with ordinary
    (cached) loads, which evicts what the last step left in the XCDs' L2 and in the
    256 MB Infinity Cache. Reads only, so no dirty lines are written back during the next
    step."""
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")

    def flush():
        buf.sum()
    return flush


def stats_ms(xs):
    xs = np.asarray(xs, dtype=np.float64)
    return {"mean": float(xs.mean()), "median": float(np.median(xs)), "min": float(xs.min())}


def block_manager_leg(pkv, inp):
    """The host block manager (C++, pa_bm_*) doing the bookkeeping of this batch: admit
    every sequence with its cached tokens, then one step: reserve the slots of the step's
    new tokens and write the padded block tables the kernels read."""
    m = pkv.BlockManager(inp.num_blocks, inp.block_size)
    B = inp.num_seqs
    t0 = time.perf_counter()
    for b in range(B):
        m.allocate(b, int(inp.cached_lens[b]))
    t1 = time.perf_counter()
    ids = np.repeat(np.arange(B, dtype=np.int64), (inp.seq_lens - inp.cached_lens).astype(np.int64))
    slots, copies = m.append_slots(ids)
    tables, lens = m.block_tables(np.arange(B, dtype=np.int64), inp.block_tables.shape[1], pad=0)
    t2 = time.perf_counter()
    assert np.array_equal(lens, inp.seq_lens.astype(np.int32)) and len(copies) == 0
    out = {"sequences": B, "new_tokens": int(len(ids)), "admit_us": (t1 - t0) * 1e6,
           "step_us": (t2 - t1) * 1e6, "gpu_cache_usage": m.usage(),
           "slot_utilisation": m.slot_utilisation()}
    m.close()
    return out


def block_copy_leg(torch, pkv, num_kv_heads, head_size, reps=10, flush=None):
    """Rates of the block copies, on buffers of their own: copy-on-write copies inside a
    2 GiB pool, half its blocks onto the other half (disjoint pairs: every byte read once
    and written once, against HBM; 8x the 256 MB last-level cache), and swaps of 128
    blocks to pinned host memory and back (against a torch copy of the same bytes between
    the same memories, the host-link rate). With ``flush`` each repetition is timed on its
    own after the flush (median); the copy-on-write rate back to back is reported too."""
    elems = 16 * 2 * num_kv_heads * head_size
    block_bytes = 2 * elems
    nb = (2 << 30) // block_bytes
    npairs, nswap = nb // 2, min(128, nb // 4)
    pool = torch.zeros((nb, elems), dtype=torch.float16, device="cuda")
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(0))
    pairs = torch.stack([perm[:npairs], perm[npairs:]], 1).contiguous().cuda()
    host_area = torch.zeros((nswap, elems), dtype=torch.float16).pin_memory()
    out_pairs = torch.stack([perm[:nswap], torch.arange(nswap)], 1).contiguous().cuda()
    in_pairs = torch.stack([torch.arange(nswap), perm[npairs:npairs + nswap]], 1).contiguous().cuda()
    flat_dev = torch.zeros((nswap, elems), dtype=torch.float16, device="cuda")
    flat_pool = pool.view(nb, elems)

    def rate(fn, nbytes, flushed=True):
        fn()
        torch.cuda.synchronize()
        if flush is not None and flushed:
            ts = []
            for _ in range(reps):
                flush()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                fn()
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            ms = float(np.median(ts))
        else:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
        return {"us": ms * 1e3, "GBps": nbytes / (ms * 1e-3) / 1e9}

    def cow():
        pkv.pa_copy_blocks(pool.view(nb, 16, 2, num_kv_heads, head_size), pairs)

    res = {
        "block_bytes": block_bytes,
        "copy_on_write": rate(cow, 2 * npairs * block_bytes),
        "copy_on_write_no_flush": rate(cow, 2 * npairs * block_bytes, flushed=False),
        "torch_copy_d2d": rate(lambda: flat_pool[npairs:2 * npairs].copy_(flat_pool[:npairs]), 2 * npairs * block_bytes),
        "swap_out": rate(lambda: pkv.pa_move_blocks(host_area, pool, out_pairs), nswap * block_bytes),
        "swap_in": rate(lambda: pkv.pa_move_blocks(pool, host_area, in_pairs), nswap * block_bytes),
        "torch_copy_d2h": rate(lambda: host_area.copy_(flat_dev, non_blocking=True), nswap * block_bytes),
        "torch_copy_h2d": rate(lambda: flat_dev.copy_(host_area, non_blocking=True), nswap * block_bytes),
    }
    res["copy_on_write"]["frac_hbm_peak"] = res["copy_on_write"]["GBps"] / HBM_PEAK_GBPS
    return res


class Step:
    """Device copies of a batch and one step of the hot path over them."""

    def __init__(self, torch, pkv, inp, partition_size, kv_stream, kv_fp8=False,
                 shared_prefix=False, prefill_split=True):
        self.torch, self.pkv, self.inp = torch, pkv, inp

        def c(a):
            return torch.from_numpy(np.ascontiguousarray(a)).cuda()

        self.pool = c(inp.pool)
        self.kv_fp8 = kv_fp8
        if kv_fp8:  # E4M3 codes of the same values (scale 1; N(0, 1) data is in range)
            self.pool = self.pool.to(torch.float8_e4m3fn).view(torch.uint8)
            torch.cuda.synchronize()
        self.key, self.value, self.slots = c(inp.key_new), c(inp.value_new), c(inp.slot_mapping)
        qd, btd, lensd = inp.decode_part()
        self.dq, self.dbt, self.dlens = c(qd), c(btd), c(lensd)
        self.dout = torch.empty_like(self.dq)
        self.mcl = int(lensd.max()) if len(lensd) else 0
        self.ps = partition_size
        self.flags = pkv.PA_DECODE_KV_STREAM if kv_stream else 0
        ws = pkv.pa_decode_workspace_bytes(len(lensd), inp.num_q_heads, self.mcl, partition_size,
                                           inp.head_size)
        self.shared_prefix = shared_prefix
        if shared_prefix:  # the generator's groups: consecutive sequences sharing prefix blocks
            g = inp.groups[inp.num_prefill:]
            starts = np.flatnonzero(np.r_[True, g[1:] != g[:-1]])
            gs = np.r_[starts, len(g)].astype(np.int32)
            self.gs = c(gs)
            self.pl = c(np.full(len(starts), inp.prefix_blocks * inp.block_size, np.int32))
            self.max_group = int(np.diff(gs).max())
            self.max_prefix = inp.prefix_blocks * inp.block_size
            ws = pkv.pa_decode_shared_prefix_workspace_bytes(len(lensd), inp.num_q_heads, self.mcl,
                                                             self.max_prefix, partition_size,
                                                             inp.head_size)
        self.ws = torch.empty(max(ws, 256), dtype=torch.uint8, device="cuda")
        self.has_prefill = inp.num_prefill > 0
        if self.has_prefill:
            qp, btp, qsl, lensp = inp.prefill_part()
            self.pq, self.pbt, self.qsl, self.plens = c(qp), c(btp), c(qsl), c(lensp)
            self.pout = torch.empty_like(self.pq)
            self.max_q = int(np.diff(qsl).max())
            self.max_s = int(lensp.max())
            # split-context workspace (caller-owned, so the captured graph uses it too)
            self.pws_bytes = (pkv.pa_prefill_workspace_bytes(len(lensp), inp.num_q_heads, self.max_q,
                                                             self.max_s, inp.head_size)
                              if prefill_split else 0)
            self.pws = (torch.empty(self.pws_bytes, dtype=torch.uint8, device="cuda")
                        if self.pws_bytes > 0 else None)

    def run(self, ev=None, stream=None):
        pkv = self.pkv

        def rec(i):
            if ev is not None:
                ev[i].record()

        rec(0)
        if len(self.inp.slot_mapping):
            if self.kv_fp8:
                pkv.pa_kv_append_fp8(self.pool, self.key, self.value, self.slots, 1.0, 1.0, stream=stream)
            else:
                pkv.pa_kv_append(self.pool, self.key, self.value, self.slots, stream=stream)
        rec(1)
        if self.has_prefill and self.kv_fp8:
            pkv.pa_prefill_chunk_fp8(self.pout, self.pq, self.pool, self.pbt, self.qsl, self.plens,
                                     self.max_q, self.max_s, self.inp.scale, 1.0, 1.0,
                                     workspace=self.pws, split=self.pws is not None, stream=stream)
        elif self.has_prefill:
            pkv.pa_prefill_chunk(self.pout, self.pq, self.pool, self.pbt, self.qsl, self.plens,
                                 self.max_q, self.max_s, self.inp.scale, workspace=self.pws,
                                 split=self.pws is not None, stream=stream)
        rec(2)
        if self.shared_prefix and self.kv_fp8:
            pkv.pa_decode_shared_prefix_fp8(self.dout, self.dq, self.pool, self.dbt, self.dlens,
                                            self.mcl, self.gs, self.pl, self.max_group,
                                            self.max_prefix, self.inp.scale, 1.0, 1.0, self.ps,
                                            self.ws, stream=stream)
        elif self.shared_prefix:
            pkv.pa_decode_shared_prefix(self.dout, self.dq, self.pool, self.dbt, self.dlens, self.mcl,
                                        self.gs, self.pl, self.max_group, self.max_prefix,
                                        self.inp.scale, self.ps, self.ws, stream=stream)
        elif self.kv_fp8:
            pkv.pa_decode_fp8(self.dout, self.dq, self.pool, self.dbt, self.dlens, self.mcl,
                              self.inp.scale, 1.0, 1.0, self.ps, self.ws, self.flags, stream=stream)
        else:
            pkv.pa_decode(self.dout, self.dq, self.pool, self.dbt, self.dlens, self.mcl,
                          self.inp.scale, self.ps, self.ws, self.flags, stream=stream)
        rec(3)


def run_counter_sequence(inp, partition_size, kv_stream, kv_fp8=False, shared_prefix=False,
                         prefill_split=True):
    """Dispatches for counter passes, in a fixed order: a torch copy of 1 GiB (reads and
    writes exactly 1 GiB: the calibration of FETCH_SIZE / WRITE_SIZE), pa_stream_read of
    1 GiB (reads 1 GiB), then three steps of the workload, run as the bench runs them."""
    import torch
    import paged_kv_cache_294_amd as pkv

    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(pkv.pa_stream_read_sink_len(nbytes), dtype=torch.float32, device="cuda")
    step = Step(torch, pkv, inp, partition_size, kv_stream, kv_fp8, shared_prefix, prefill_split)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    pkv.pa_stream_read(src, sink)
    torch.cuda.synchronize()
    for _ in range(3):
        step.run()
        torch.cuda.synchronize()
    log(f"counter sequence done: copy {nbytes} B, stream_read {nbytes} B, 3 steps; "
        f"decode algorithmic KV bytes per launch {kv_read_bytes(inp, 1 if kv_fp8 else 2)}")


def summarize_trace(path, command):
    import csv
    rows = list(csv.DictReader(open(path)))
    print(f"# rocprofv3 kernel statistics\n# command: {command}")
    print(f"{'kernel':<72} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}")
    for r in rows:
        print(f"{r['Name'][:72]:<72} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
              f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
              f"{float(r['Percentage']):>6.2f}")


def summarize_pmc(paths, kernel, command):
    """Median per-dispatch value of each counter for the dispatches of `kernel`, and the
    matrix-core busy fraction: SQ_VALU_MFMA_BUSY_CYCLES over all SIMD cycles, where
    GRBM_GUI_ACTIVE sums the active cycles of the 8 XCDs (128 SIMDs each)."""
    import csv
    import statistics
    per = {}  # counter -> {(pass, dispatch): value summed over the pass's rows}
    for k, path in enumerate(paths):
        for r in csv.DictReader(open(path)):
            if kernel not in r["Kernel_Name"]:
                continue
            d = per.setdefault(r["Counter_Name"], {})
            key = (k, r["Dispatch_Id"])
            d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    print(f"# rocprofv3 --pmc counters of kernels matching '{kernel}' (median per dispatch)")
    print(f"# command: {command}")
    med = {}
    for name in sorted(per):
        vals = list(per[name].values())
        med[name] = statistics.median(vals)
        print(f"{name:32s} {med[name]:16.0f}   ({len(vals)} dispatches)")
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
        print(f"mfma_busy_fraction: {med['SQ_VALU_MFMA_BUSY_CYCLES'] / (med['GRBM_GUI_ACTIVE'] * 128):.3f}")
    if "SQ_INSTS_VALU" in med and "SQ_INSTS_MFMA" in med:
        print(f"valu_per_mfma: {med['SQ_INSTS_VALU'] / med['SQ_INSTS_MFMA']:.2f}")
    if "SQ_LDS_BANK_CONFLICT" in med and "SQ_LDS_IDX_ACTIVE" in med:
        print(f"lds_bank_conflict_fraction: {med['SQ_LDS_BANK_CONFLICT'] / med['SQ_LDS_IDX_ACTIVE']:.3f}")


def summarize_counters(fetch_csv, write_csv, command):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the --mode counters sequence, scaled by
    the reading of the 1 GiB copy."""
    import csv
    fetch = list(csv.DictReader(open(fetch_csv)))
    write = list(csv.DictReader(open(write_csv)))
    gib = float(1 << 30)
    copy_i = next(i for i, r in enumerate(write)
                  if "copy" in r["Kernel_Name"].lower() and float(r["Counter_Value"]) * 1024 >= gib * 0.99)
    f_scale = gib / (float(fetch[copy_i]["Counter_Value"]) * 1024)
    w_scale = gib / (float(write[copy_i]["Counter_Value"]) * 1024)
    print("# rocprofv3 FETCH_SIZE / WRITE_SIZE passes of `bench.py --mode counters`")
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
           if "decode_partition_kernel" in n or "decode_gqa_kernel" in n or "decode_reduce_kernel" in n]
    print(f"hbm_bytes_per_launch: {sum(dec):.0f}")
    print(f"kernel_source_sha256_16: {source_digest(DECODE_SRC)}")


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="decode256")
    ap.add_argument("--partition-size", type=int, default=0,
                    help="decode partition in tokens; 0 (default): the library's "
                         "pa_decode_default_partition_size for the workload (512 for "
                         "shared-prefix decode)")
    ap.add_argument("--kv-stream", choices=("auto", "on", "off"), default="auto",
                    help="non-temporal K/V loads in decode; auto: on unless blocks are shared")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="graph: time replays of the step captured once into a HIP graph "
                         "(StepGraph), the serving path; eager: time the launches themselves. "
                         "Per-kernel times always come from eager steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-stream-read", action="store_true")
    ap.add_argument("--no-block-copies", action="store_true")
    ap.add_argument("--decode", choices=("auto", "plain", "shared-prefix"), default="auto",
                    help="shared-prefix: pa_decode_shared_prefix over the workload's prompt "
                         "groups (reads each shared prefix once); auto: that when the workload "
                         "has prompt groups, else plain")
    ap.add_argument("--kv-dtype", choices=("fp16", "fp8"), default="fp16",
                    help="cache element: fp16, or FP8 E4M3 codes with per-tensor key and value "
                         "scales (append, decode and prefill all read and write the codes)")
    ap.add_argument("--prefill-split", choices=("on", "off"), default="on",
                    help="on: pa_prefill_chunk gets its split-context workspace (long contexts "
                         "cut into pieces merged by log-sum-exp); off: one workgroup per row tile")
    ap.add_argument("--flush", choices=("on", "off"), default="on",
                    help="on: an untimed 1 GiB cache-flushing read between timed steps, each "
                         "step timed on its own (mean, median, min reported; back-to-back "
                         "steps are timed too and reported as *_no_flush); off: back-to-back "
                         "steps only")
    ap.add_argument("--cpu-cores", type=int, default=16)
    ap.add_argument("--mode", choices=("bench", "counters"), default="bench",
                    help="counters: a short fixed dispatch sequence for rocprofv3 --pmc passes "
                         "(1 GiB torch copy, 1 GiB pa_stream_read, then 3 steps)")
    ap.add_argument("--summarize-trace", metavar="KERNEL_STATS_CSV",
                    help="print a profile summary of a rocprofv3 --stats kernel_stats.csv and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc passes of "
                         "--mode counters (FETCH_SIZE, then WRITE_SIZE) and exit")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="COUNTER_CSV",
                    help="print the median per-dispatch counters of --kernel from rocprofv3 "
                         "--pmc passes (one CSV per pass) and exit")
    ap.add_argument("--kernel", default="prefill_kernel",
                    help="kernel-name substring for --summarize-pmc")
    ap.add_argument("--command", default="", help="command line recorded in a summary")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.kernel, args.command)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the decode path would shard by sequence or KV head with no exchange).",
              file=sys.stderr)
        sys.exit(2)

    gen, desc = WORKLOADS[args.workload]
    log(f"generating workload {args.workload}")
    t0 = time.perf_counter()
    inp = workloads.WORKLOADS[gen]()
    seed = inp.seed
    if args.workload == "prefix-private":
        inp = workloads.unshare_prefix(inp)
    log(f"generated in {time.perf_counter() - t0:.1f}s: {inp.num_blocks} blocks, "
        f"{inp.num_seqs} sequences, sum L = {int(inp.seq_lens.sum())}")
    shared = shares_blocks(inp)
    kv_stream = {"on": True, "off": False, "auto": not shared}[args.kv_stream]
    kv_fp8 = args.kv_dtype == "fp8"
    elem_bytes = 1 if kv_fp8 else 2
    shared_prefix = {"plain": False, "shared-prefix": True,
                     "auto": bool(inp.prefix_blocks)}[args.decode]
    if shared_prefix and not inp.prefix_blocks:
        print("--decode shared-prefix needs prompt groups (workload prefix-groups)", file=sys.stderr)
        sys.exit(2)
    if args.partition_size <= 0 and shared_prefix:
        args.partition_size = 512  # fastest of 256 .. 2048 for 64 groups of 1024-token prompts
    elif args.partition_size <= 0 and args.workload == "long32k":
        args.partition_size = 512  # the long-context workload is specified with 512-token partitions
    elif args.partition_size <= 0:  # the library's choice for its kernels (a host-only call)
        import paged_kv_cache_294_amd as pkv
        args.partition_size = pkv.pa_decode_default_partition_size(
            inp.num_seqs - inp.num_prefill, inp.num_q_heads, inp.num_kv_heads,
            int(inp.seq_lens.max()))
    # algorithmic bytes: every decode context token's K and V once; with shared prefix
    # blocks, every physical block's filled slots once (the logical count is reported too)
    logical_bytes = kv_read_bytes(inp, elem_bytes)
    kv_bytes = kv_unique_bytes(inp, elem_bytes) if shared else logical_bytes

    if args.mode == "counters":
        run_counter_sequence(inp, args.partition_size, kv_stream, kv_fp8, shared_prefix,
                             args.prefill_split == "on")
        return

    cpu = None
    if kv_fp8 and not args.no_cpu_baseline:
        log("CPU baseline skipped for the FP8 cache (the oracle's fp16 run is the reference)")
    elif not args.no_cpu_baseline:
        log("CPU baseline: oracle on the host cores")
        cpu = cpu_baseline(inp, args.cpu_cores, decode_seqs=4 if args.workload == "long32k" else None)
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

    bm = None
    if not inp.prefix_blocks:  # prefix sharing comes from the generator's own tables
        bm = block_manager_leg(pkv, inp)
        log(f"host block manager: admit {bm['admit_us']:.0f} us, step {bm['step_us']:.0f} us "
            f"({bm['new_tokens']} slots + tables)")
    log("copying the batch to the GPU")
    step = Step(torch, pkv, inp, args.partition_size, kv_stream, kv_fp8, shared_prefix,
                args.prefill_split == "on")
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    log(f"warmup done; timing {args.steps} steps")

    flush = make_flush(torch) if args.flush == "on" else None

    def eager_loop(with_flush):
        """Per-step event times (ms) of append, prefill, decode and the whole step."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            step.run(evs[i])
            if with_flush:
                flush()
        torch.cuda.synchronize()
        return {"append": [e[0].elapsed_time(e[1]) for e in evs],
                "prefill": [e[1].elapsed_time(e[2]) for e in evs],
                "decode": [e[2].elapsed_time(e[3]) for e in evs],
                "step": [e[0].elapsed_time(e[3]) for e in evs]}

    w0 = time.perf_counter()
    eag = eager_loop(flush is not None)
    wall = time.perf_counter() - w0
    eag_nf = eager_loop(False) if flush is not None else eag
    append_ms = float(np.mean(eag["append"]))
    prefill_ms = float(np.mean(eag["prefill"]))
    decode_ms = float(np.mean(eag["decode"]))
    decode_stats = stats_ms(eag["decode"])
    decode_nf_ms = float(np.mean(eag_nf["decode"]))
    ms_step = float(np.mean(eag["step"]))
    step_stats = stats_ms(eag["step"])
    ms_step_nf = float(np.mean(eag_nf["step"]))
    log(f"step {ms_step:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms): append "
        f"{append_ms * 1e3:.1f} us, prefill {prefill_ms * 1e3:.1f} us, decode {decode_ms * 1e3:.1f} us"
        f" (median {decode_stats['median'] * 1e3:.1f}, min {decode_stats['min'] * 1e3:.1f};"
        f" back to back without flush {decode_nf_ms * 1e3:.1f} us)")

    eager_ms_step = ms_step
    if args.launch == "graph":
        side = torch.cuda.Stream()
        graph = pkv.StepGraph(side)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            with graph:
                step.run(stream=side)
        for _ in range(args.warmup):
            graph.launch()
        torch.cuda.synchronize()
        if flush is not None:  # each replay timed on its own, the flush between them untimed
            gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)]
            with torch.cuda.stream(side):
                for gs_, ge_ in gev:
                    gs_.record(side)
                    graph.launch()
                    ge_.record(side)
                    flush()
            torch.cuda.synchronize()
            step_stats = stats_ms([a.elapsed_time(b) for a, b in gev])
            ms_step = step_stats["mean"]
        gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gs.record(side)
        for _ in range(args.steps):
            graph.launch()
        ge.record(side)
        torch.cuda.synchronize()
        ms_step_nf = gs.elapsed_time(ge) / args.steps
        if flush is None:
            ms_step = ms_step_nf
            step_stats = {"mean": ms_step}
        graph.close()
        log(f"graph replay: step {ms_step:.3f} ms (back to back without flush {ms_step_nf:.3f} ms; "
            f"eager {eager_ms_step:.3f} ms)")

    copies = None
    if not args.no_block_copies:
        copies = block_copy_leg(torch, pkv, inp.num_kv_heads, inp.head_size, flush=flush)
        log("block copies: copy-on-write {:.0f} GB/s ({:.0f} back to back; torch's contiguous copy "
            "{:.0f}), swap out {:.1f} GB/s, swap in {:.1f} GB/s (torch copies {:.1f} / {:.1f} GB/s)".format(
                copies["copy_on_write"]["GBps"], copies["copy_on_write_no_flush"]["GBps"],
                copies["torch_copy_d2d"]["GBps"], copies["swap_out"]["GBps"], copies["swap_in"]["GBps"],
                copies["torch_copy_d2h"]["GBps"], copies["torch_copy_h2d"]["GBps"]))

    achieved = kv_bytes / (decode_ms * 1e-3) / 1e9
    nparts = pkv.pa_num_partitions(step.mcl, args.partition_size)
    traffic = read_traffic(f"pa_decode_{args.workload}{'_fp8' if kv_fp8 else ''}_counters.txt", source_digest(DECODE_SRC))
    used_blocks = int(sum(-(-int(L) // 16) for L in inp.seq_lens))
    kernels = {"decode": {"ms": decode_ms, "ms_median": decode_stats["median"],
                          "ms_min": decode_stats["min"], "kv_read_GBps": achieved,
                          "frac_hbm_peak": achieved / HBM_PEAK_GBPS, "partitions": nparts,
                          "kv_stream": kv_stream, "ms_no_flush": decode_nf_ms,
                          "kv_read_GBps_no_flush": kv_bytes / (decode_nf_ms * 1e-3) / 1e9}}
    if len(inp.slot_mapping):
        kernels["append"] = {"us": append_ms * 1e3, "tokens": len(inp.slot_mapping),
                             "GBps": append_bytes(inp, elem_bytes) / (append_ms * 1e-3) / 1e9}
    if inp.num_prefill:
        fl = prefill_flops(inp)
        tf = fl / (prefill_ms * 1e-3) / 1e12
        kernels["prefill"] = {"us": prefill_ms * 1e3, "gflop": fl / 1e9, "TFLOPs": tf,
                              "frac_mfma_peak": tf / MFMA_F16_PEAK_TFLOPS,
                              "split_workspace_bytes": step.pws_bytes}
    if shared:
        kernels["decode"]["logical_kv_bytes"] = logical_bytes
        kernels["decode"]["logical_kv_GBps"] = logical_bytes / (decode_ms * 1e-3) / 1e9
    result = {
        "metric": "paged-attn decode KV-read GB/s (% of HBM peak) + seq-steps/s, 1 GPU",
        "value": kv_bytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_median": step_stats.get("median"),
        "ms_per_step_min": step_stats.get("min"),
        "ms_per_step_no_flush": ms_step_nf,
        "cache_flush": ("an untimed 1 GiB read between timed steps; each step timed on its "
                        "own with HIP events" if flush is not None else None),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16, fp8 e4m3 cache" if kv_fp8 else "f16",
        "data": "synthetic",
        "config": {
            "workload": desc,
            "num_seqs": inp.num_seqs, "num_q_heads": inp.num_q_heads,
            "num_kv_heads": inp.num_kv_heads, "head_size": inp.head_size,
            "block_size": inp.block_size, "partition_size": args.partition_size,
            "sum_context_tokens": int(inp.seq_lens.sum()), "seed": seed,
            "launch": "hip graph replay" if args.launch == "graph" else "eager",
            "kv_dtype": args.kv_dtype,
            "decode": "shared-prefix" if shared_prefix else "plain",
        },
        "eager_ms_per_step": eager_ms_step,
        "pct_of_hbm_peak": 100.0 * kv_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "seq_steps_per_s": inp.num_seqs / (ms_step * 1e-3),
        "roofline": {
            "kernel": (("pa_decode_shared_prefix_fp8" if kv_fp8 else "pa_decode_shared_prefix") +
                       " (prefix, own-token and log-sum-exp reduce kernels)"
                       if shared_prefix else
                       ("pa_decode_fp8" if kv_fp8 else "pa_decode") + " (" +
                       ("partition + log-sum-exp reduce kernels" if nparts > 1
                        else "partition kernel") +
                       ("; a longest-first order pre-pass when the items exceed what the GPU "
                        "holds at once" if kv_stream and nparts <= 16 else "") + ")"),
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kv_bytes,
        },
        "kernels": kernels,
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in
                                                  ("value", "unit", "cores", "kind", "sample")},
        "block_manager": bm,
        "block_copies": copies,
        "stream_read_gbps": stream_gbps,
        "frac_of_stream_read": None if not stream_gbps else achieved / stream_gbps,
        "context": {
            "slot_utilisation": float(inp.seq_lens.sum()) / (used_blocks * 16),
            "gpu_cache_usage": used_blocks / inp.num_blocks,
        },
    }
    if inp.num_prefill and prefill_ms > decode_ms:
        # the prefill call dominates the step: its roofline is the matrix-core peak
        pf = kernels["prefill"]
        result["decode_roofline"] = result["roofline"]
        result["roofline"] = {
            "kernel": ("pa_prefill_chunk_fp8" if kv_fp8 else "pa_prefill_chunk") +
                      (" (prefill and context-split merge kernels)" if step.pws_bytes
                       else " (prefill kernel)"),
            "bound": "mfma",
            "achieved": pf["TFLOPs"],
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": pf["frac_mfma_peak"],
            "traffic": None,
            "algorithmic_flops_per_launch": prefill_flops(inp),
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
