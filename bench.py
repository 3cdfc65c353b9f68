"""Benchmark of one paged-attention decode step on one MI355X.

A step is the whole hot path over one batch: copy-on-write block copies (when
the workload has any), the append of every sequence's new K/V through the slot
mapping, decode attention, and the log-sum-exp merge of split sequences.  By
default the append runs inside the decode launch (pa_decode_append) when every
write of the step is a sequence's last position; ``--append separate`` times
pa_kv_append and pa_decode as two launches.  The
default workload is the Llama-3.1-8B-class batch (32 query / 8 KV heads,
head_dim 128, bf16, 16-token blocks, 64 sequences with context lengths uniform
in [128, 4096]).

Inputs are resident in HBM before timing starts.  The step cycles through
``--rotate`` independent copies of the KV pools, so each step reads a cache
that at least (rotate-1) other caches' worth of traffic has passed since it was
last touched - more than the 256 MB Infinity Cache and the L2s hold - the way a
model's layers each read their own cache once per step.

Two timed regions, each bracketed by HIP events on the launch stream with no
event inside: ``--steps`` whole steps (``value``, ``ms_per_step``), then
``--steps`` decode launches back to back (``decode_us`` and the roofline).
Each timed region follows at least ``--warmup`` untimed calls of what it
times, and at least WARM_SECONDS of them: the GPU's clocks ramp up over the
first milliseconds of work, which a handful of 60-90 us steps does not cover.

Prints one JSON line.  ``value`` is the KV bytes the step's decode must read
divided by the step time (GB/s).

``--part prefill`` times mixed-batch attention (pa_prefill) on three named
workloads against the bf16 MFMA peak; ``--part swap`` times block swaps between the device pools and pinned
host pools (pa_swap_blocks, both directions, 8B-class blocks) against the
PCIe link; ``--part scheduler`` times the host-side block manager's step on a
serving trace at the batch-64 scale, native against the oracle (no GPU
needed).  Each prints its own JSON line.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from paged_kv_cache_93_amd import lib  # noqa: E402
from paged_kv_cache_93_amd import workloads as W  # noqa: E402

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense
# PCIe 5.0 x16 host link, per direction: 32 GT/s x 16 lanes x 128/130 / 8 bits
PCIE_PEAK_GBPS = 32.0 * 16 * 128 / 130 / 8


def to_device(arr, dtype):
    """Device copy of stored values: bf16 bit patterns, f32, or uint8 E4M3 codes."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def paper_alibi_slopes(num_heads: int) -> torch.Tensor:
    """ALiBi's geometric slopes 2^(-8h/H), h = 1..H (Press, Smith and Lewis), on
    the device as float32."""
    h = np.arange(1, num_heads + 1, dtype=np.float64)
    return torch.tensor(2.0 ** (-8.0 * h / num_heads), dtype=torch.float32).cuda()


def algorithmic_bytes(w: W.Workload, window: int = 0) -> dict:
    """Bytes the decode step must move, per component (a sliding window reads
    only its last ``window`` positions and the table entries of their blocks)."""
    e = W.element_bytes(w.dtype)                    # cache element
    eq = W.element_bytes(W.query_dtype(w.dtype))    # q, new tokens and output

    def entries(n):
        first = (n - window) // w.block_size if 0 < window < n else 0
        return W.blocks_for(n, w.block_size) - first

    table_entries = sum(entries(int(n)) for n in w.context_lens)
    return dict(
        kv=w.kv_bytes(window),
        q=w.num_seqs * w.num_heads * w.head_dim * eq,
        out=w.num_seqs * w.num_heads * w.head_dim * eq,
        tables=4 * table_entries,
        lens=4 * w.num_seqs,
        append=2 * len(w.slot_mapping) * w.num_kv_heads * w.head_dim * (eq + e),
    )


def cpu_baseline(w: W.Workload, budget_s: float, window: int = 0, alibi: bool = False) -> dict:
    """The float64 oracle's decode on a bounded sample of the same workload
    (with the same attention variant)."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - reporting only
        threads = 1
    kp, vp = oracle.copy_blocks(w.k_pool, w.v_pool, w.copy_pairs)
    kp, vp = oracle.kv_append(kp, vp, w.k_new, w.v_new, w.slot_mapping,
                              fp8_scales=(w.k_scale, w.v_scale) if w.dtype == "fp8" else None)
    scale = 1.0 / math.sqrt(w.head_dim)
    slopes = None
    if alibi:
        slopes = paper_alibi_slopes(w.num_heads).cpu().numpy().astype(np.float64)
    # sequences one at a time, cycling over the batch until the time budget is spent
    done = 0
    kv = 0
    c0 = time.process_time()  # CPU time of every thread of this process
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        i = done % w.num_seqs
        sl = slice(i, i + 1)
        oracle.decode(w.q[sl], kp, vp, w.block_tables[sl], w.context_lens[sl], scale, w.dtype,
                      k_scale=w.k_scale, v_scale=w.v_scale, window=window, alibi_slopes=slopes)
        n = int(w.context_lens[i])
        n = min(n, window) if window > 0 else n
        kv += n * w.num_kv_heads * w.head_dim * 2 * W.element_bytes(w.dtype)
        done += 1
    dt = time.perf_counter() - t0
    cpu = time.process_time() - c0
    # cores actually kept busy: CPU time over wall time (the BLAS pool may be
    # larger, but small per-sequence products leave most of it idle)
    used = max(1, round(cpu / dt)) if dt > 0 else 1
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": int(used),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle decode (gather + two-pass softmax), one sequence at "
                      f"a time, cycling over the workload's {w.num_seqs} sequences: {done} "
                      f"sequence decodes ({done / w.num_seqs:.1f} passes, {kv / 1e6:.1f} MB of "
                      f"KV) in {dt:.1f} s, {cpu:.1f} s of CPU time ({cpu / dt:.2f} cores busy "
                      f"on average; BLAS pool of {threads} threads, host has {os.cpu_count()} "
                      f"CPUs)",
            "seqs_per_s": round(done / dt, 3)}


KERNEL_SOURCES = ("pa_decode_kernel.h", "pa_decode.hip", "pa_decode_bf16.hip", "pa_decode_f32.hip",
                  "pa_decode_fp8.hip")
PROFILES = os.path.join(ROOT, "profiles")
CAL_BLOCKS = 4096  # calibration copy: blocks [0, 2048) -> [2048, 4096) of a scratch pool pair


def kernel_digest() -> str:
    """Digest of the decode kernels' sources: traffic figures taken from
    counters apply only while it is unchanged."""
    import hashlib

    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_cache_93_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str, mode: str) -> str:
    return os.path.join(PROFILES, f"traffic_decode_{workload}_{mode}.md")


def read_traffic(workload: str, mode: str):
    """HBM bytes per decode launch from the counter summary, or None when
    there is none or the kernels changed since it was taken."""
    path = traffic_path(workload, mode)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_digest") != kernel_digest():
        return None
    return int(fields["hbm_bytes_per_launch"])


def _counter_rows(d: str):
    """(kernel key, counter, value) of every dispatch in a rocprofv3 --pmc run."""
    import csv
    import glob

    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            name = row["Kernel_Name"]
            key = next((k for k in ("decode_kernel", "merge_kernel", "reduce_kernel",
                                    "copy_kernel") if k in name), None)
            if key:
                yield key, row["Counter_Name"], float(row["Counter_Value"])


def pmc_summary(dirs, workload: str, block_bytes: int, mode: str, command: str) -> str:
    """Summarise the rocprofv3 --pmc runs of ``--pmc-pass`` into
    profiles/traffic_decode_<workload>_<mode>.md: FETCH_SIZE, then WRITE_SIZE,
    then (optional third run) TCC_HIT_sum, TCC_MISS_sum and
    TCC_EA0_RDREQ_DRAM_sum.

    The calibration copy moves a known number of bytes each way; the ratio of
    those bytes to the counter's reading for it scales the decode kernels'
    readings to bytes.  The L2 (TCC) hit rate is HIT / (HIT + MISS) over the
    kernel's requests; DRAM read requests are the L2's reads that went to
    HBM rather than another cache."""
    from collections import defaultdict

    vals = defaultdict(list)  # (kernel, counter) -> per-dispatch values
    for d in dirs:
        for key, counter, v in _counter_rows(d):
            vals[(key, counter)].append(v)
    mean = lambda v: sum(v) / len(v) if v else float("nan")
    cal_bytes = 2 * (CAL_BLOCKS // 2) * block_bytes
    f_cal, w_cal = mean(vals[("copy_kernel", "FETCH_SIZE")]), mean(vals[("copy_kernel", "WRITE_SIZE")])
    f_factor = cal_bytes / (f_cal * 1024)
    w_factor = cal_bytes / (w_cal * 1024)
    kernels = [k for k in ("decode_kernel", "merge_kernel", "reduce_kernel")
               if vals[(k, "FETCH_SIZE")]]
    has_tcc = any(vals[(k, "TCC_HIT_sum")] for k in kernels)
    rows, total = [], 0.0
    for k in kernels:
        fk, wk = vals[(k, "FETCH_SIZE")], vals[(k, "WRITE_SIZE")]
        fb = mean(fk) * 1024 * f_factor
        wb = mean(wk) * 1024 * w_factor
        total += fb + wb
        row = (f"| {k} | {len(fk)} | {mean(fk):.1f} | {fb / 1e6:.2f} | {mean(wk):.1f} | "
               f"{wb / 1e6:.2f} |")
        if has_tcc:
            hit, miss = mean(vals[(k, "TCC_HIT_sum")]), mean(vals[(k, "TCC_MISS_sum")])
            dram = mean(vals[(k, "TCC_EA0_RDREQ_DRAM_sum")])
            rate = hit / (hit + miss) if hit + miss > 0 else float("nan")
            row += f" {100 * rate:.1f} | {hit:.0f} | {miss:.0f} | {dram:.0f} |"
        rows.append(row)
    head = ("| kernel | dispatches | FETCH_SIZE KiB | read MB (scaled) | WRITE_SIZE KiB | "
            "written MB (scaled) |")
    rule = "|---|---|---|---|---|---|"
    if has_tcc:
        head += " TCC hit % | TCC_HIT | TCC_MISS | TCC_EA0_RDREQ_DRAM |"
        rule += "---|---|---|---|"
    dk = "decode_kernel"
    extra = []
    if has_tcc:
        hit, miss = mean(vals[(dk, "TCC_HIT_sum")]), mean(vals[(dk, "TCC_MISS_sum")])
        dram = mean(vals[(dk, "TCC_EA0_RDREQ_DRAM_sum")])
        fetched = mean(vals[(dk, "FETCH_SIZE")]) * 1024 * f_factor
        extra = [f"- tcc_hit_rate_decode: {hit / (hit + miss):.4f}",
                 f"- dram_read_requests_decode: {dram:.0f}",
                 f"- dram_read_bytes_decode_at_128B: {int(dram * 128)} "
                 f"({dram * 128 / fetched:.3f} of the scaled FETCH_SIZE)"]
    text = "\n".join([
        f"# HBM traffic of one decode launch: {workload}, mode {mode}",
        "",
        "rocprofv3 counter runs of the same program (`bench.py --pmc-pass`), one per counter set:",
        "",
        "```",
        command,
        "```",
        "",
        f"Calibration: the copy kernel moves {cal_bytes} bytes each way "
        f"({CAL_BLOCKS // 2} blocks, K and V pools); it read FETCH_SIZE {f_cal:.1f} KiB and "
        f"WRITE_SIZE {w_cal:.1f} KiB per dispatch, so FETCH_SIZE is scaled by {f_factor:.4f} and "
        f"WRITE_SIZE by {w_factor:.4f}.  Counter values are means over the dispatches.",
        "",
        head,
        rule,
        *rows,
        "",
        f"- hbm_bytes_per_launch: {int(round(total))}",
        f"- fetch_factor: {f_factor:.4f}",
        f"- write_factor: {w_factor:.4f}",
        *extra,
        f"- kernel_digest: `{kernel_digest()}`",
        "",
    ])
    os.makedirs(PROFILES, exist_ok=True)
    with open(traffic_path(workload, mode), "w") as f:
        f.write(text)
    return text


def ktrace_summary(trace_dir: str, workload: str, mode: str, steps: int, command: str,
                   note: str = "") -> str:
    """Summarise a rocprofv3 --kernel-trace run of bench.py into
    profiles/kernels_<workload>_<mode>.md: per kernel, every dispatch, and the
    last `steps` dispatches (the decode-only timed region, which runs last)."""
    import csv
    import glob
    from collections import defaultdict

    disp = defaultdict(list)
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            disp[row["Kernel_Name"]].append((int(row["Start_Timestamp"]),
                                             int(row["End_Timestamp"])))
    lines = []
    decode_total = 0.0
    for name in sorted(disp, key=lambda n: -len(disp[n])):
        ds = sorted(disp[name])
        us = [(e - b) / 1e3 for b, e in ds]
        last = us[-steps:] if len(us) >= steps else us
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        if any(k in name for k in ("decode_kernel", "merge_kernel", "reduce_kernel")):
            decode_total += sum(last) / len(last)
        lines.append(f"| `{short}` | {len(us)} | {sum(us) / len(us):.2f} | {len(last)} | "
                     f"{sum(last) / len(last):.2f} | {pct(last, 50):.2f} | {pct(last, 10):.2f} | "
                     f"{pct(last, 90):.2f} | {min(last):.2f} | {max(last):.2f} |")
    text = "\n".join([
        f"# Kernel durations: {workload}, decode mode {mode}",
        "",
        "```",
        command,
        "```",
        "",
        "Durations are end minus start of each dispatch in the kernel trace (us). `last` = the "
        f"last {steps} dispatches of a kernel: for the decode kernels, the bench's decode-only "
        "timed region (the roofline's launches), which runs last.",
        "",
        "| kernel | dispatches | mean (all) | last | mean | median | p10 | p90 | min | max |",
        "|---|---|---|---|---|---|---|---|---|---|",
        *lines,
        "",
        f"- decode_launch_us (decode-path kernels, mean of the last {steps}): {decode_total:.2f}",
        *( [note] if note else []),
        "",
    ])
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"kernels_{workload}_{mode}.md"), "w") as f:
        f.write(text)
    return text


def workload_shape(k: int, block_size=None, dtype=None, head_dim=None):
    """(name, bytes of one block of one pool) of workload k, as make_config names it."""
    c = W.CONFIGS[k]
    bs = int(block_size or c["block_size"])
    dt = dtype or c["dtype"]
    d = int(head_dim or c["head_dim"])
    name = (c["name"] + ("" if dt == c["dtype"] else f"_{dt}") +
            ("" if bs == c["block_size"] else f"_bs{bs}") +
            ("" if d == c["head_dim"] else f"_d{d}"))
    return name, c["num_kv_heads"] * bs * d * W.element_bytes(dt)


def bench_swap(args) -> dict:
    """pa_swap_blocks at the 8B-class block shape (8 KV heads x 16 x 128 bf16:
    32 KiB per pool per block), ``--swap-blocks`` random blocks per launch."""
    hkv, bs, d, dt = 8, 16, 128, torch.bfloat16
    n = args.swap_blocks
    n_dev, n_host = 4 * n, 2 * n
    dk = torch.randn((n_dev, hkv, bs, d), device="cuda").to(dt)
    dv = torch.randn_like(dk)
    hk = torch.empty((n_host, hkv, bs, d), dtype=dt, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    rng = np.random.default_rng(9393)
    out_pairs = torch.from_numpy(np.stack([rng.permutation(n_dev)[:n],
                                           rng.permutation(n_host)[:n]], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([rng.permutation(n_host)[:n],
                                          rng.permutation(n_dev)[:n]], 1)).cuda()
    nbytes = 2 * n * hkv * bs * d * dk.element_size()

    def timed(fn, k):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(k):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k

    swap_out = lambda: lib.pa_swap_blocks(dk, dv, hk, hv, out_pairs, lib.PA_SWAP_OUT)
    swap_in = lambda: lib.pa_swap_blocks(dk, dv, hk, hv, in_pairs, lib.PA_SWAP_IN)
    # the same bytes as one contiguous copy each way (torch, DMA): the link's practical rate
    flat_d, flat_h = dk[:2 * n].reshape(-1), hk.reshape(-1)
    bulk_out = lambda: flat_h.copy_(flat_d, non_blocking=True)
    bulk_in = lambda: flat_d.copy_(flat_h, non_blocking=True)
    res = {}
    for name, fn in (("swap_out", swap_out), ("swap_in", swap_in), ("bulk_out", bulk_out),
                     ("bulk_in", bulk_in)):
        warm_up(lambda i: fn(), args.warmup)
        ms = timed(fn, args.steps)
        res[name] = dict(us=round(ms * 1e3, 1), gbps=round(nbytes / (ms * 1e-3) / 1e9, 2))
    return {
        "metric": "KV block swap GB/s between HBM and pinned host memory (pa_swap_blocks)",
        "value": min(res["swap_out"]["gbps"], res["swap_in"]["gbps"]),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": True, "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"swap {n} random 8B-class blocks (K and V) per launch",
                   "bytes_per_launch": nbytes, "device_blocks": n_dev, "host_blocks": n_host},
        "directions": res,
        "roofline": {"bound": "pcie", "peak": round(PCIE_PEAK_GBPS, 2), "unit": "GB/s",
                     "frac_out": round(res["swap_out"]["gbps"] / PCIE_PEAK_GBPS, 3),
                     "frac_in": round(res["swap_in"]["gbps"] / PCIE_PEAK_GBPS, 3)},
    }


# Untimed work before each timed region: at least --warmup calls and at least
# this long (GPU clocks ramp up over the first milliseconds of activity).
WARM_SECONDS = 0.2


def warm_up(fn, calls: int, rotate: int = 1) -> int:
    """Call fn(i % rotate) at least `calls` times and for at least WARM_SECONDS;
    returns the number of calls."""
    t0 = time.perf_counter()
    i = 0
    while i < calls or time.perf_counter() - t0 < WARM_SECONDS:
        fn(i % rotate)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()  # keep the host from running far ahead of the GPU
    torch.cuda.synchronize()
    return i


def bench_prefill(args) -> dict:
    """pa_prefill on the named mixed-batch workloads (8B-class heads, bf16 or
    8-bit cache): algorithmic flops per launch / average launch time."""
    import torch

    names = [args.prefill_workload] if args.prefill_workload else PREFILL_WORKLOADS
    dtype = args.dtype or "bf16"
    rows = {}
    for name in names:
        w = W.prefill_config(name, dtype=dtype, block_size=args.block_size or 16)
        k, v = to_device(w.k_pool, w.dtype), to_device(w.v_pool, w.dtype)
        q = to_device(w.q, "bf16")
        tables = torch.from_numpy(w.block_tables).cuda()
        qs = torch.from_numpy(w.query_start).cuda()
        lens = torch.from_numpy(w.context_lens).cuda()
        out = torch.empty((w.num_tokens, w.num_heads, w.head_dim), dtype=torch.bfloat16,
                          device="cuda")
        ws = lib.prefill_workspace(w.num_seqs, w.num_tokens, w.num_heads, w.num_kv_heads)
        scale = 1.0 / math.sqrt(w.head_dim)

        slopes = paper_alibi_slopes(w.num_heads) if args.alibi else None

        def call():
            lib.pa_prefill(k, v, q, tables, qs, lens, scale, out, workspace=ws,
                           k_scale=w.k_scale, v_scale=w.v_scale, window=args.window,
                           alibi_slopes=slopes)

        warm_up(lambda i: call(), args.warmup)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            call()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) / args.steps * 1e3
        flops = w.flops(args.window)
        tflops = flops / (us * 1e-6) / 1e12
        rows[name] = dict(us=round(us, 1), gflop=round(flops / 1e9, 2),
                          tflops=round(tflops, 1), frac=round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                          seqs=w.num_seqs, tokens=w.num_tokens)
        print(f"# prefill {name}: {us:.1f} us, {tflops:.1f} TFLOP/s", file=sys.stderr, flush=True)
    head = rows[names[0]]
    return {
        "metric": "paged prefill attention TFLOP/s (pa_prefill, mixed batches)",
        "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": PREFILL_DESCRIPTIONS[names[0]],
                   "block_size": args.block_size or 16, "sliding_window": args.window,
                   "alibi": bool(args.alibi)},
        "workloads": rows,
        "roofline": {"bound": "mfma",
                     "kernel": "prefill_dma_kernel" if dtype == "bf16" else "prefill_dma8_kernel",
                     "achieved": head["tflops"],
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": head["frac"],
                     "traffic": None},
    }


PREFILL_WORKLOADS = ["cached_preamble", "long_prompts", "mixed_step"]
PREFILL_DESCRIPTIONS = {
    "cached_preamble": "cached_preamble: 16 x (304 new tokens over a 1,200-token context), "
                       "32 query / 8 KV heads, head_dim 128",
    "long_prompts": "long_prompts: 4 x 4,096-token prompts from scratch, 32 query / 8 KV heads, "
                    "head_dim 128",
    "mixed_step": "mixed_step: 60 decode rows + a 2,048-token slice + a 1,024-token prompt, "
                  "32 query / 8 KV heads, head_dim 128",
}

# SQ counter passes of the prefill attention kernel (each within one pass's
# hardware limits: at most 8 SQ counters and 2 GRBM counters)
SQ_PASSES = {
    "mix": ["SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VALU", "SQ_INSTS_SALU",
            "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES",
            "SQ_BUSY_CU_CYCLES", "GRBM_GUI_ACTIVE"],
    "lds": ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT",
            "SQ_LDS_DATA_FIFO_FULL", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
            "SQ_INSTS_LDS_LOAD_BANDWIDTH", "SQ_INSTS_VALU_TRANS_F32", "GRBM_GUI_ACTIVE"],
}


def sq_summary(root: str, dtype: str, command: str) -> str:
    """Summarise rocprofv3 --pmc runs of ``--part prefill --prefill-workload W``
    (directories root/<workload>/<pass>, one per SQ_PASSES entry) into
    profiles/sq_prefill_<dtype>.md: per dispatch of the attention kernel, the
    instruction mix and how busy the matrix cores, the VALU and the LDS were.

    Utilisations follow rocprofv3's own derived metrics: MFMA busy cycles over
    GPU-busy cycles times the 1,024 SIMDs; LDS active cycles over GPU-busy
    cycles times the 256 CUs; VALU active cycles (summed over waves) over
    GPU-busy cycles times the CUs; bank-conflict cycles over the LDS's
    conflict-free active cycles."""
    import csv
    import glob
    from collections import defaultdict

    cus, simds = 256, 1024
    lines = []
    for wl in PREFILL_WORKLOADS:
        vals = defaultdict(list)
        for pname in SQ_PASSES:
            d = os.path.join(root, wl, pname)
            for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
                for row in csv.DictReader(open(f)):
                    name = row["Kernel_Name"]
                    if any(k in name for k in ("prefill_dma_kernel", "prefill_dma8_kernel",
                                               "prefill_kernel")):
                        vals[(pname, row["Counter_Name"])].append(float(row["Counter_Value"]))
        if not vals:
            continue
        mean = lambda k: (sum(vals[k]) / len(vals[k])) if vals[k] else float("nan")
        # GRBM_GUI_ACTIVE comes summed over the 8 XCDs: per XCD, the kernel's cycles
        g1 = mean(("mix", "GRBM_GUI_ACTIVE")) / 8
        g2 = mean(("lds", "GRBM_GUI_ACTIVE")) / 8
        mfma = mean(("mix", "SQ_INSTS_MFMA"))
        lds_i = mean(("mix", "SQ_INSTS_LDS"))
        valu = mean(("mix", "SQ_INSTS_VALU"))
        salu = mean(("mix", "SQ_INSTS_SALU"))
        mfma_util = 100 * mean(("mix", "SQ_VALU_MFMA_BUSY_CYCLES")) / (g1 * simds)
        valu_busy = 100 * mean(("mix", "SQ_ACTIVE_INST_VALU")) / (g1 * cus)
        occ = 400 * mean(("mix", "SQ_WAVE_CYCLES")) / g1 / cus / 32
        idx = mean(("lds", "SQ_LDS_IDX_ACTIVE"))
        bank = mean(("lds", "SQ_LDS_BANK_CONFLICT"))
        lds_util = 100 * idx / (g2 * cus)
        bank_ratio = bank / (idx - bank) if idx > bank else float("nan")
        lds_bytes = 64 * mean(("lds", "SQ_INSTS_LDS_LOAD_BANDWIDTH"))
        trans = mean(("lds", "SQ_INSTS_VALU_TRANS_F32"))
        lines.append(
            f"| {wl} | {len(vals[('mix', 'SQ_INSTS_MFMA')])} | {g1:.0f} | {mfma:.0f} | "
            f"{lds_i:.0f} | {lds_i / mfma:.2f} | {valu / mfma:.2f} | {salu / mfma:.2f} | "
            f"{trans / mfma:.2f} | {lds_bytes / 1e6:.1f} | {lds_bytes / mfma:.0f} | "
            f"{mfma_util:.1f} | {lds_util:.1f} | {100 * bank_ratio:.1f} | {valu_busy:.1f} | "
            f"{occ:.1f} |")
        lines.append(
            f"| ↳ raw | | {g2:.0f} (lds pass) | | | | | | | | | "
            f"addr-conflict {mean(('lds', 'SQ_LDS_ADDR_CONFLICT')):.0f}, "
            f"data-FIFO-full {mean(('lds', 'SQ_LDS_DATA_FIFO_FULL')):.0f} | "
            f"active-inst-LDS {mean(('lds', 'SQ_ACTIVE_INST_LDS')):.0f} | "
            f"wait-inst-LDS {mean(('lds', 'SQ_WAIT_INST_LDS')):.0f} | | |")
    text = "\n".join([
        f"# SQ counters of the prefill attention kernel ({dtype} cache)",
        "",
        "rocprofv3 counter passes of `bench.py --part prefill` (one workload per run, one pass "
        "per counter set):",
        "",
        "```",
        command,
        "```",
        "",
        "Per dispatch of the attention kernel, means over the dispatches.  Columns: GPU-busy "
        "cycles (GRBM_GUI_ACTIVE, which the counter run reports summed over the 8 XCDs, / 8); MFMA, LDS, VALU, SALU and 32-bit transcendental VALU "
        "instructions (VALU/SALU/trans per MFMA); bytes the LDS returned to the waves "
        "(SQ_INSTS_LDS_LOAD_BANDWIDTH x 64), in MB and per MFMA; MFMA util % "
        "(SQ_VALU_MFMA_BUSY_CYCLES / (busy cycles x 1,024 SIMDs)); LDS util % "
        "(SQ_LDS_IDX_ACTIVE / (busy cycles x 256 CUs)); bank conflicts % (conflict cycles / "
        "conflict-free LDS active cycles); VALU busy % (SQ_ACTIVE_INST_VALU / (busy cycles x "
        "256 CUs)); occupancy % of 32 wave slots per CU (SQ_WAVE_CYCLES).",
        "",
        "| workload | dispatches | busy cycles | MFMA | LDS inst | LDS/MFMA | VALU/MFMA | "
        "SALU/MFMA | trans/MFMA | LDS read MB | LDS B/MFMA | MFMA util % | LDS util % | "
        "bank confl % | VALU busy % | occupancy % |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|",
        *lines,
        "",
    ])
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"sq_prefill_{dtype}.md"), "w") as f:
        f.write(text)
    return text


def prefill_ktrace_summary(root: str, dtype: str, steps: int, command: str) -> str:
    """Summarise rocprofv3 --kernel-trace runs of ``--part prefill
    --prefill-workload W`` (directories root/<workload>) into
    profiles/kernels_prefill_<dtype>_three_workloads.md: per workload, the
    attention kernel's last `steps` dispatches (the timed calls, which run
    last) against the algorithmic flops, and the tile-map kernel."""
    import csv
    import glob

    rows, prep = [], []
    for wl in PREFILL_WORKLOADS:
        attn, tiles = [], []
        for f in glob.glob(os.path.join(root, wl, "**", "*kernel_trace.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                name = row["Kernel_Name"]
                d = (int(row["Start_Timestamp"]), int(row["End_Timestamp"]))
                if "prefill_tiles_kernel" in name:
                    tiles.append(d)
                elif any(k in name for k in ("prefill_dma_kernel", "prefill_dma8_kernel",
                                             "prefill_kernel")):
                    attn.append((d, name.replace("void ", "").split("(")[0]))
        if not attn:
            continue
        attn.sort()
        us = [(e - b) / 1e3 for (b, e), _ in attn][-steps:]
        kname = attn[-1][1]
        gflop = W.prefill_config(wl, dtype=dtype).flops() / 1e9
        mean = sum(us) / len(us)
        tf = gflop / (mean * 1e-6) / 1e3
        rows.append(f"| `{kname}` | {wl} | {len(us)} | {mean:.1f} | {pct(us, 50):.1f} | "
                    f"{pct(us, 10):.1f} | {pct(us, 90):.1f} | {min(us):.1f} | {max(us):.1f} | "
                    f"{gflop:.2f} | {tf:.0f} | {tf / MFMA_BF16_PEAK_TFLOPS:.3f} |")
        prep += [(e - b) / 1e3 for b, e in tiles]
    text = "\n".join([
        f"# Kernel durations: pa_prefill on three mixed-batch workloads ({dtype} cache)",
        "",
        "rocprofv3 kernel traces, one run per workload:",
        "",
        "```",
        command,
        "```",
        "",
        "32 query / 8 KV heads, head_dim 128, 16-token blocks, bf16 output.  Every call is "
        "`prefill_tiles_kernel` (the tile map, one workgroup) then the attention kernel; the "
        f"table covers the attention kernel's last {steps} dispatches (the timed calls).  "
        "Durations are end minus start of each dispatch (us); TFLOP/s = algorithmic flops "
        "(4 x head_dim x query heads per (query token, visible key)) / mean duration, against "
        f"the {MFMA_BF16_PEAK_TFLOPS:,.0f} TFLOP/s dense bf16 MFMA peak.",
        "",
        "Workloads: " + "; ".join(PREFILL_DESCRIPTIONS[w] for w in PREFILL_WORKLOADS) + ".",
        "",
        "| kernel | workload | calls | mean us | median | p10 | p90 | min | max | GFLOP | "
        "TFLOP/s | of peak |",
        "|---|---|---|---|---|---|---|---|---|---|---|---|",
        *rows,
        "",
        f"- prefill_tiles_kernel: {len(prep)} dispatches, mean "
        f"{(sum(prep) / len(prep)) if prep else float('nan'):.2f} us",
        "",
    ])
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"kernels_prefill_{dtype}_three_workloads.md"), "w") as f:
        f.write(text)
    return text


def event_times(fn, n: int) -> list:
    """Per-call durations (us) of n calls, each bracketed by its own pair of
    HIP events on the current stream (for medians and percentiles; the mean
    of back-to-back calls is timed without events in between)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(evs):
        a.record()
        fn(i)
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in evs]


def pct(xs, q: float) -> float:
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def bench_stream(args) -> dict:
    """The streaming-read probe (pa_probe_stream_read): one read of a buffer
    of --stream-mib MiB, the achievable HBM read rate the decode figures are
    compared with.  Grids of 1, 2 and 4 workgroups of 512 lanes per CU; the
    best is the ceiling.  With --xcd-masks, the same read by subsets of the
    eight XCDs (does one XCD's share of bandwidth grow when others idle?)."""
    nbytes = args.stream_mib * (1 << 20)
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.random_(0, 255)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rows, best = {}, None
    masks = [0xFF] + [int(m, 0) for m in args.xcd_masks.split(",") if m] if args.xcd_masks else [0xFF]
    for per_cu in (1, 2, 4):
        groups = cus * per_cu
        sink = torch.empty(groups * 16, dtype=torch.uint8, device="cuda")
        for mask in masks:
            call = lambda i, m=mask, g=groups, k=sink: lib.probe_stream_read(src, g, k, m)
            warm_up(call, args.warmup)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for i in range(args.steps):
                call(i)
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) / args.steps * 1e3
            per = event_times(call, min(args.steps, 100))
            key = f"{per_cu}_per_cu" + ("" if mask == 0xFF else f"_xcd_{mask:#04x}")
            rows[key] = dict(us=round(us, 2), gbps=round(nbytes / (us * 1e-6) / 1e9, 1),
                             median_us=round(pct(per, 50), 2), p10_us=round(pct(per, 10), 2),
                             p90_us=round(pct(per, 90), 2), workgroups=groups,
                             xcds=bin(mask).count("1"))
            print(f"# stream {key}: {us:.1f} us, {rows[key]['gbps']:.0f} GB/s", file=sys.stderr,
                  flush=True)
            if mask == 0xFF and (best is None or rows[key]["gbps"] > rows[best]["gbps"]):
                best = key
    return {
        "metric": "streaming HBM read GB/s (pa_probe_stream_read), the ceiling decode is "
                  "compared with",
        "value": rows[best]["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "vs_baseline": None, "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": f"one read of {args.stream_mib} MiB, 16-byte non-temporal "
                               f"loads, 64 KiB slices per workgroup step", "best_grid": best},
        "grids": rows,
        "roofline": {"bound": "hbm", "kernel": "stream_read_kernel",
                     "achieved": rows[best]["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(rows[best]["gbps"] / HBM_PEAK_GBPS, 4), "traffic": None},
    }


def stream_ktrace_summary(trace_dir: str, mib: int, command: str) -> str:
    """Summarise a rocprofv3 --kernel-trace run of ``--part stream`` into
    profiles/kernels_stream_read_<mib>mib.md: per grid, every dispatch of the
    probe kernel and the read rate it implies (bytes read / duration)."""
    import csv
    import glob
    from collections import defaultdict

    nbytes = mib * (1 << 20)
    grids = defaultdict(list)
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if "stream_read" not in row["Kernel_Name"]:
                continue
            wgs = int(row["Grid_Size_X"]) // int(row["Workgroup_Size_X"])
            grids[wgs].append((int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    lines = []
    for wgs in sorted(grids):
        us = grids[wgs]
        gb = lambda t: nbytes / (t * 1e-6) / 1e9
        lines.append(f"| {wgs} | {len(us)} | {sum(us) / len(us):.1f} | {pct(us, 50):.1f} | "
                     f"{pct(us, 10):.1f} | {pct(us, 90):.1f} | {gb(sum(us) / len(us)):,.0f} | "
                     f"{gb(pct(us, 50)):,.0f} | {gb(min(us)):,.0f} |")
    text = "\n".join([
        f"# Kernel durations: streaming-read probe, one read of {mib} MiB",
        "",
        "```",
        command,
        "```",
        "",
        "`pa_probe_stream_read`: 512-lane workgroups read 64 KiB slices with 16-byte "
        "non-temporal loads (8 per lane in flight) and fold them into a sink; grids of 1, 2 "
        "and 4 workgroups per CU.  Durations are end minus start of each dispatch (us); GB/s "
        "= bytes read / duration.  The best grid's rate is the read ceiling the decode "
        "figures are compared with.",
        "",
        "| workgroups | dispatches | mean us | median | p10 | p90 | GB/s (mean) | GB/s (median) "
        "| GB/s (fastest) |",
        "|---|---|---|---|---|---|---|---|---|",
        *lines,
        "",
    ])
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"kernels_stream_read_{mib}mib.md"), "w") as f:
        f.write(text)
    return text


class ServingTrace:
    """Seeded serving workload for the block manager at the batch-64 scale.

    ``live`` requests at a time; prompts of U{128..4096} tokens, 30 % of them
    opening with one shared 1,008-token system prompt; each request generates
    U{64..512} tokens and finishes, and a new one arrives in its place.
    """

    def __init__(self, seed: int, live: int = 64):
        self.rng = np.random.default_rng(seed)
        self.live = live
        self.system = self.rng.integers(0, 32000, 1008).tolist()
        self.next_rid = 0
        self.target = {}   # rid -> total length at which it finishes
        self.length = {}   # rid -> tokens so far

    def _new(self, managers):
        rid = self.next_rid
        self.next_rid += 1
        n = int(self.rng.integers(128, 4097))
        toks = self.rng.integers(0, 32000, n).tolist()
        if self.rng.random() < 0.3:
            toks = (self.system + toks)[:n]
        for m in managers:
            m.add_request(rid, toks)
        self.length[rid] = n
        self.target[rid] = n + int(self.rng.integers(64, 513))

    def admit(self, managers):
        while len(self.target) < self.live:
            self._new(managers)

    def post(self, managers, plan):
        """After a step: each scheduled request whose KV now covers all its
        tokens samples one more token, or finishes at its target length."""
        done, rids = [], []
        for rid, ctx in zip(list(plan.seq_ids), list(plan.context_lens)):
            rid = int(rid)
            if int(ctx) != self.length[rid]:
                continue          # a prompt slice: nothing to sample yet
            (done if self.length[rid] >= self.target[rid] else rids).append(rid)
        toks = self.rng.integers(0, 32000, len(rids)).tolist()
        for m in managers:
            if hasattr(m, "append_batch"):
                m.append_batch(rids, toks)
            else:
                for r, t in zip(rids, toks):
                    m.append_token(r, t)
            for rid in done:
                m.finish(rid)
        for rid in rids:
            self.length[rid] += 1
        for rid in done:
            del self.target[rid], self.length[rid]

    def step(self, managers, budget: int):
        self.admit(managers)
        plans = [m.schedule(budget) for m in managers]
        self.post(managers, plans[0])
        return plans


def bench_scheduler(args) -> dict:
    """Host time of the block manager's schedule() per serving step (pool and
    batch of the 8B-class batch-64 workload), the native library against the
    oracle.  ``step_us`` adds the driver's own work (drawing tokens, appending
    them, finishing requests)."""
    sys.path.insert(0, ROOT)
    from oracle.block_manager import BlockManager as OracleBM

    cfg = dict(num_gpu_blocks=10598, num_cpu_blocks=4096, block_size=16, prefix_caching=True,
               preempt_mode="swap", watermark_blocks=64)
    budget = 8192
    m = lib.BlockManager(**cfg)
    trace = ServingTrace(9302)
    t_warm = time.perf_counter()
    for _ in range(args.warmup):
        trace.step([m], budget)
    warm_s = time.perf_counter() - t_warm
    sched_s, total_s, seqs, toks = 0.0, 0.0, 0, 0
    for _ in range(args.steps):
        t0 = time.perf_counter()
        trace.admit([m])
        t1 = time.perf_counter()
        plan = m.schedule(budget)
        t2 = time.perf_counter()
        trace.post([m], plan)
        t3 = time.perf_counter()
        seqs += len(plan.seq_ids)
        toks += len(plan.slot_mapping)
        sched_s += t2 - t1
        total_s += t3 - t0
    st = m.stats()
    # the oracle on the same serving trace, for a bounded number of steps
    o = OracleBM(**cfg)
    otrace = ServingTrace(9302)
    for _ in range(args.warmup):
        otrace.step([o], budget)
    o_steps, o_s, o_sched = 0, 0.0, 0.0
    while o_s < args.cpu_budget and o_steps < args.steps:
        t0 = time.perf_counter()
        otrace.admit([o])
        t1 = time.perf_counter()
        oplan = o.schedule(budget)
        t2 = time.perf_counter()
        otrace.post([o], oplan)
        o_s += time.perf_counter() - t0
        o_sched += t2 - t1
        o_steps += 1
    return {
        "metric": "block manager schedule() host time per serving step (plan copied out)",
        "value": round(sched_s / args.steps * 1e6, 1), "unit": "us",
        "n_gpus": 0, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
        "vs_baseline": None, "dtype": "int64", "data": "synthetic",
        "config": {"workload": "64 live requests, prompts U{128..4096} (30% with a shared "
                               "1,008-token system prompt), U{64..512} generated tokens each, "
                               "pool 10,598 blocks of 16, 4,096 CPU blocks, swap preemption, "
                               "token budget 8,192", **cfg},
        "step_us": round(total_s / args.steps * 1e6, 1),
        "seqs_per_step": round(seqs / args.steps, 1),
        "tokens_per_step": round(toks / args.steps, 1),
        "warmup_s": round(warm_s, 3),
        "stats": st,
        "cpu_baseline": {"value": round(o_sched / max(o_steps, 1) * 1e6, 1), "unit": "us",
                         "cores": 1, "kind": "oracle",
                         "sample": f"schedule() over {o_steps} steps of the same serving "
                                   f"trace after the same {args.warmup} warm-up steps"},
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--head-dim", type=int, default=None, choices=[64, 128],
                    help="decode: the named workload with this head_dim (same seed)")
    ap.add_argument("--dtype", default=None, choices=["f32", "bf16", "fp8"],
                    help="cache element type (default: the workload's; fp8 = E4M3 codes)")
    ap.add_argument("--mode", default="balanced",
                    help="balanced | single | <partition size in tokens> (split-KV + merge)")
    ap.add_argument("--rotate", type=int, default=3, help="independent copies of the KV pools")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for cpu_baseline (0 = skip)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run the calibration copy, then --steps decode launches, and exit "
                         "(the program to run under rocprofv3 --pmc)")
    ap.add_argument("--pmc-summary", nargs="+", metavar="DIR",
                    help="write the traffic summary from --pmc-pass counter runs: FETCH_SIZE "
                         "dir, WRITE_SIZE dir, [TCC hit/miss/DRAM dir]")
    ap.add_argument("--ktrace-summary", metavar="DIR",
                    help="write the kernel-duration summary of a --kernel-trace run of bench")
    ap.add_argument("--pmc-command", default="", help="command line recorded in the summary")
    ap.add_argument("--prefill-workload", default=None, choices=PREFILL_WORKLOADS,
                    help="prefill: time only this workload")
    ap.add_argument("--stream-ktrace-summary", metavar="DIR",
                    help="stream: write the kernel-trace summary of a --part stream run")
    ap.add_argument("--prefill-ktrace-summary", metavar="DIR",
                    help="prefill: write the kernel-trace summary of the runs under DIR "
                         "(DIR/<workload>)")
    ap.add_argument("--sq-summary", metavar="DIR",
                    help="prefill: write the SQ counter summary of the runs under DIR "
                         "(DIR/<workload>/<pass>)")
    ap.add_argument("--ceiling", type=int, default=1,
                    help="decode: also time the streaming-read probe (the read ceiling)")
    ap.add_argument("--stream-mib", type=int, default=2048,
                    help="stream: MiB read per probe call")
    ap.add_argument("--xcd-masks", default="",
                    help="stream: comma-separated XCD bit masks to time besides all eight")
    ap.add_argument("--part", default="decode",
                    choices=["decode", "swap", "scheduler", "prefill", "stream"],
                    help="decode: the decode step (default); swap: block swaps to pinned host "
                         "memory; scheduler: the host block manager (no GPU needed)")
    ap.add_argument("--swap-blocks", type=int, default=1024, help="blocks per swap launch")
    ap.add_argument("--append", default="fused", choices=["fused", "separate"],
                    help="step: append fused into the decode launch (pa_decode_append; not "
                         "with split-KV partitions or extra writes) or pa_kv_append then "
                         "pa_decode")
    ap.add_argument("--window", type=int, default=0,
                    help="decode and prefill: sliding window in tokens (0: none)")
    ap.add_argument("--alibi", action="store_true",
                    help="decode and prefill: ALiBi with the paper's slopes")
    args = ap.parse_args()

    if args.part == "scheduler":
        print(json.dumps(bench_scheduler(args)), flush=True)
        return 0

    if args.pmc_summary:
        name, block_bytes = workload_shape(args.workload, args.block_size, args.dtype, args.head_dim)
        print(pmc_summary(args.pmc_summary, name, block_bytes, args.mode, args.pmc_command))
        return 0
    if args.sq_summary:
        print(sq_summary(args.sq_summary, args.dtype or "bf16", args.pmc_command))
        return 0
    if args.stream_ktrace_summary:
        print(stream_ktrace_summary(args.stream_ktrace_summary, args.stream_mib,
                                    args.pmc_command))
        return 0
    if args.prefill_ktrace_summary:
        print(prefill_ktrace_summary(args.prefill_ktrace_summary, args.dtype or "bf16",
                                     args.steps, args.pmc_command))
        return 0
    if args.ktrace_summary:
        name, _ = workload_shape(args.workload, args.block_size, args.dtype, args.head_dim)
        print(ktrace_summary(args.ktrace_summary, name, args.mode, args.steps, args.pmc_command))
        return 0

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
                                   "--gpus must be 1"}), flush=True)
        return 2
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 2
    lib.load()
    if args.part == "swap":
        print(json.dumps(bench_swap(args)), flush=True)
        return 0
    if args.part == "prefill":
        print(json.dumps(bench_prefill(args)), flush=True)
        return 0
    if args.part == "stream":
        print(json.dumps(bench_stream(args)), flush=True)
        return 0

    w = W.make_config(args.workload, dtype=args.dtype, block_size=args.block_size,
                      head_dim=args.head_dim)
    qdt = W.query_dtype(w.dtype)
    sc = dict(k_scale=w.k_scale, v_scale=w.v_scale)
    mode = args.mode if args.mode in ("balanced", "single") else int(args.mode)
    scale = 1.0 / math.sqrt(w.head_dim)
    variant = bool(args.window or args.alibi)
    if variant and isinstance(mode, int):
        print(json.dumps({"error": "split-KV partitions take no attention variant"}), flush=True)
        return 2
    nbytes = algorithmic_bytes(w, args.window)
    print(f"# workload {w.name}: {w.num_seqs} seqs, KV {nbytes['kv'] / 1e6:.1f} MB, "
          f"pool {w.num_blocks} blocks, mode {mode}", file=sys.stderr, flush=True)

    shared = dict(q=to_device(w.q, qdt),
                  tables=torch.from_numpy(w.block_tables).cuda(),
                  lens=torch.from_numpy(w.context_lens).cuda(),
                  slots=torch.from_numpy(w.slot_mapping).cuda(),
                  pairs=torch.from_numpy(w.copy_pairs).cuda(),
                  k_new=to_device(w.k_new, qdt), v_new=to_device(w.v_new, qdt))
    var = dict(window=args.window)
    if args.alibi:
        var["alibi_slopes"] = paper_alibi_slopes(w.num_heads)
    pools = []
    k0, v0 = to_device(w.k_pool, w.dtype), to_device(w.v_pool, w.dtype)
    for r in range(args.rotate):
        pools.append((k0, v0) if r == 0 else (k0.clone(), v0.clone()))
    out = torch.empty((w.num_seqs, w.num_heads, w.head_dim), device="cuda",
                      dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16)
    psize = mode if isinstance(mode, int) else 0
    mp = max(1, max(math.ceil(int(n) / psize) for n in w.context_lens)) if psize else 1
    po = torch.empty((w.num_seqs, w.num_heads, mp, w.head_dim), device="cuda")
    pm = torch.empty((w.num_seqs, w.num_heads, mp), device="cuda")
    ps = torch.empty_like(pm)
    ws = None
    if mode == "balanced":
        ws = lib.decode_workspace(w.num_seqs, w.num_heads, w.head_dim, k_pool=k0, v_pool=v0)

    def decode(r):
        kp, vp = pools[r]
        if psize:
            lib.pa_decode_partitions(kp, vp, shared["q"], shared["tables"], shared["lens"],
                                     scale, psize, po, pm, ps, **sc)
            lib.pa_splitkv_reduce(po, pm, ps, shared["lens"], psize, out)
        else:
            lib.pa_decode(kp, vp, shared["q"], shared["tables"], shared["lens"], scale, out,
                          workspace=ws, **sc, **var)

    S = w.num_seqs
    # the fused call writes each sequence's token at its last position; a step
    # with other writes too (a copy-on-write divergence) keeps pa_kv_append
    fused = args.append == "fused" and not psize and len(w.slot_mapping) == S
    if fused:
        k_own, v_own = shared["k_new"], shared["v_new"]

    def step(r):
        kp, vp = pools[r]
        if shared["pairs"].numel():
            lib.pa_copy_blocks(kp, vp, shared["pairs"])
        if not fused:
            lib.pa_kv_append(kp, vp, shared["k_new"], shared["v_new"], shared["slots"], **sc)
            decode(r)
            return
        lib.pa_decode_append(kp, vp, shared["q"], k_own, v_own, shared["tables"], shared["lens"],
                             scale, out, workspace=ws, **sc, **var)

    def timed(fn, n):
        """Mean milliseconds per call of fn over n back-to-back calls, from HIP
        events recorded on the stream the kernels are launched on (torch's
        current stream) before the first and after the last call."""
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(n):
            fn(i % args.rotate)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / n

    if args.pmc_pass:
        # a plain copy of known size, then the decode launches being measured
        blk = tuple(k0.shape[1:])
        ck = torch.zeros((CAL_BLOCKS, *blk), dtype=k0.dtype, device="cuda")
        cv = torch.zeros_like(ck)
        half = CAL_BLOCKS // 2
        cal_pairs = torch.stack([torch.arange(half), torch.arange(half) + half], 1).cuda()
        for i in range(args.warmup):
            decode(i % args.rotate)
        lib.pa_copy_blocks(ck, cv, cal_pairs)
        for i in range(args.steps):
            decode(i % args.rotate)
        torch.cuda.synchronize()
        print(f"# pmc pass done: 1 calibration copy, {args.warmup + args.steps} decode launches",
              file=sys.stderr, flush=True)
        return 0

    warm_steps = warm_up(step, args.warmup, args.rotate)
    # timed region 1: whole steps (value, ms_per_step)
    ms_step = timed(step, args.steps)
    # timed region 2: the decode launches alone, back to back (roofline)
    warm_decode = warm_up(decode, args.warmup, args.rotate)
    dec_avg = timed(decode, args.steps)
    # per-launch spread: each launch between its own pair of events (these
    # durations include an event's own cost, ~1-2 us; the mean above has none)
    per_launch = event_times(lambda i: decode(i % args.rotate), min(args.steps, 200))
    ceiling = None
    if args.ceiling:
        # the streaming-read probe on this GPU, over a 2 GiB buffer
        src = torch.empty(1 << 31, dtype=torch.uint8, device="cuda")
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        sink = torch.empty(cus * 16, dtype=torch.uint8, device="cuda")
        probe = lambda i: lib.probe_stream_read(src, cus, sink)
        warm_up(probe, 5)
        ceiling = round(float(src.numel()) / (timed(probe, 20) * 1e-3) / 1e9, 1)
        del src
    # (a kernel trace of this run splits its dispatches by these counts)
    print(f"# regions: steps {warm_steps} warm-up + {args.steps} timed; decode {warm_decode} "
          f"warm-up + {args.steps} timed", file=sys.stderr, flush=True)

    kernels = ("decode_kernel + merge_kernel" if mode == "balanced" else
               "decode_kernel" if mode == "single" else "decode_kernel + reduce_kernel")
    kv_gbps_step = nbytes["kv"] / (ms_step * 1e-3) / 1e9
    decode_bytes = nbytes["kv"] + nbytes["q"] + nbytes["out"] + nbytes["tables"] + nbytes["lens"]
    achieved = decode_bytes / (dec_avg * 1e-3) / 1e9
    result = {
        "metric": "paged decode attention KV GB/s (% of HBM peak) + seqs/s, 8B-class batch 64",
        "value": round(kv_gbps_step, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "block_size": w.block_size, "decode_mode": str(mode),
                   "append": "fused into decode" if fused else "separate launch",
                   "context_lens": f"{int(w.context_lens.min())}..{int(w.context_lens.max())}, "
                                   f"mean {float(w.context_lens.mean()):.0f}",
                   "seed": w.seed, "rotating_caches": args.rotate,
                   "sliding_window": args.window, "alibi": bool(args.alibi)},
        "seqs_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "hbm_peak_frac_step": round(kv_gbps_step / HBM_PEAK_GBPS, 4),
        "kv_bytes": nbytes["kv"],
        "decode_us": round(dec_avg * 1e3, 2),
        "decode_us_per_launch": {"median": round(pct(per_launch, 50), 2),
                                 "p10": round(pct(per_launch, 10), 2),
                                 "p90": round(pct(per_launch, 90), 2), "launches": len(per_launch)},
        "kv_gbps_decode": round(nbytes["kv"] / (dec_avg * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "kernel": kernels, "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if variant else read_traffic(w.name, str(mode)),
                     "algorithmic_bytes_per_launch": decode_bytes,
                     "stream_ceiling_gbps": ceiling,
                     "frac_of_ceiling": round(achieved / ceiling, 4) if ceiling else None},
    }
    if w.info.get("shared_blocks") is not None:
        # shared prefix: each shared block is read by every sequence's walk;
        # the unique bytes are what a reader of every block once would move
        uniq = w.unique_kv_bytes()
        result["kv_bytes_unique"] = uniq
        result["kv_gbps_decode_unique"] = round(uniq / (dec_avg * 1e-3) / 1e9, 1)
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, args.window, args.alibi)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
