"""Benchmark of one paged-attention decode step on one MI355X.

A step is the whole hot path over one batch: copy-on-write block copies (when
the workload has any), the append of every sequence's new K/V through the slot
mapping, decode attention (split-KV), and the log-sum-exp merge.  The default
workload is the Llama-3.1-8B-class batch (32 query / 8 KV heads, head_dim 128,
bf16, 16-token blocks, 64 sequences with context lengths uniform in
[128, 4096]).

Inputs are resident in HBM before timing starts.  The step cycles through
``--rotate`` independent copies of the KV pools, so each step reads a cache
that at least (rotate-1) other caches' worth of traffic has passed since it was
last touched - more than the 256 MB Infinity Cache and the L2s hold - the way a
model's layers each read their own cache once per step.

Prints one JSON line.  ``value`` is the KV bytes the step's decode must read
divided by the step time (GB/s).
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


def to_device(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def algorithmic_bytes(w: W.Workload) -> dict:
    """Bytes the decode step must move, per component."""
    e = W.element_bytes(w.dtype)
    table_entries = sum(W.blocks_for(int(n), w.block_size) for n in w.context_lens)
    return dict(
        kv=w.kv_bytes(),
        q=w.num_seqs * w.num_heads * w.head_dim * e,
        out=w.num_seqs * w.num_heads * w.head_dim * e,
        tables=4 * table_entries,
        lens=4 * w.num_seqs,
        append=2 * 2 * len(w.slot_mapping) * w.num_kv_heads * w.head_dim * e,
    )


def cpu_baseline(w: W.Workload, budget_s: float) -> dict:
    """The float64 oracle's decode on a bounded sample of the same workload."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover - reporting only
        threads = 1
    kp, vp = oracle.copy_blocks(w.k_pool, w.v_pool, w.copy_pairs)
    kp, vp = oracle.kv_append(kp, vp, w.k_new, w.v_new, w.slot_mapping)
    scale = 1.0 / math.sqrt(w.head_dim)
    done = 0
    kv = 0
    t0 = time.perf_counter()
    while done < w.num_seqs and time.perf_counter() - t0 < budget_s:
        sl = slice(done, done + 1)
        oracle.decode(w.q[sl], kp, vp, w.block_tables[sl], w.context_lens[sl], scale, w.dtype)
        kv += int(w.context_lens[done]) * w.num_kv_heads * w.head_dim * 2 * W.element_bytes(w.dtype)
        done += 1
    dt = time.perf_counter() - t0
    return {"value": round(kv / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"float64 NumPy oracle decode (gather + two-pass softmax) of sequences "
                      f"0..{done - 1} of the same workload ({done} of {w.num_seqs}, "
                      f"{kv / 1e6:.1f} MB of KV) in {dt:.1f} s; host has {os.cpu_count()} CPUs",
            "seqs_per_s": round(done / dt, 3)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--mode", default="balanced",
                    help="balanced | single | <partition size in tokens> (split-KV + merge)")
    ap.add_argument("--rotate", type=int, default=3, help="independent copies of the KV pools")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for cpu_baseline (0 = skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; "
                                   "--gpus must be 1"}), flush=True)
        return 2
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 2
    lib.load()

    w = W.make_config(args.workload, block_size=args.block_size)
    mode = args.mode if args.mode in ("balanced", "single") else int(args.mode)
    scale = 1.0 / math.sqrt(w.head_dim)
    nbytes = algorithmic_bytes(w)
    print(f"# workload {w.name}: {w.num_seqs} seqs, KV {nbytes['kv'] / 1e6:.1f} MB, "
          f"pool {w.num_blocks} blocks, mode {mode}", file=sys.stderr, flush=True)

    shared = dict(q=to_device(w.q, w.dtype),
                  tables=torch.from_numpy(w.block_tables).cuda(),
                  lens=torch.from_numpy(w.context_lens).cuda(),
                  slots=torch.from_numpy(w.slot_mapping).cuda(),
                  pairs=torch.from_numpy(w.copy_pairs).cuda(),
                  k_new=to_device(w.k_new, w.dtype), v_new=to_device(w.v_new, w.dtype))
    pools = []
    k0, v0 = to_device(w.k_pool, w.dtype), to_device(w.v_pool, w.dtype)
    for r in range(args.rotate):
        pools.append((k0, v0) if r == 0 else (k0.clone(), v0.clone()))
    out = torch.empty((w.num_seqs, w.num_heads, w.head_dim), dtype=k0.dtype, device="cuda")
    psize = mode if isinstance(mode, int) else 0
    mp = max(1, max(math.ceil(int(n) / psize) for n in w.context_lens)) if psize else 1
    po = torch.empty((w.num_seqs, w.num_heads, mp, w.head_dim), device="cuda")
    pm = torch.empty((w.num_seqs, w.num_heads, mp), device="cuda")
    ps = torch.empty_like(pm)
    ws = None
    if mode == "balanced":
        ws = lib.decode_workspace(w.num_seqs, w.num_heads, w.head_dim)

    def step(r, ev=None):
        kp, vp = pools[r]
        if shared["pairs"].numel():
            lib.pa_copy_blocks(kp, vp, shared["pairs"])
        lib.pa_kv_append(kp, vp, shared["k_new"], shared["v_new"], shared["slots"])
        if ev is not None:
            ev[0].record()
        if psize:
            lib.pa_decode_partitions(kp, vp, shared["q"], shared["tables"], shared["lens"],
                                     scale, psize, po, pm, ps)
            if ev is not None:
                ev[1].record()
            lib.pa_splitkv_reduce(po, pm, ps, shared["lens"], psize, out)
        else:
            lib.pa_decode(kp, vp, shared["q"], shared["tables"], shared["lens"], scale, out,
                          workspace=ws)
            if ev is not None:
                ev[1].record()

    for i in range(args.warmup):
        step(i % args.rotate)
    torch.cuda.synchronize()

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(i % args.rotate, evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    dec_ms = np.array([a.elapsed_time(b) for a, b in evs])
    dec_avg = float(dec_ms.mean())

    kv_gbps_step = nbytes["kv"] / (ms_step * 1e-3) / 1e9
    decode_bytes = nbytes["kv"] + nbytes["q"] + nbytes["tables"] + nbytes["lens"]
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
                   "context_lens": f"{int(w.context_lens.min())}..{int(w.context_lens.max())}, "
                                   f"mean {float(w.context_lens.mean()):.0f}",
                   "seed": w.seed, "rotating_caches": args.rotate},
        "seqs_per_s": round(w.num_seqs / (ms_step * 1e-3), 1),
        "hbm_peak_frac_step": round(kv_gbps_step / HBM_PEAK_GBPS, 4),
        "kv_bytes": nbytes["kv"],
        "decode_us": {"mean": round(dec_avg * 1e3, 2),
                      "p10": round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                      "p50": round(float(np.percentile(dec_ms, 50)) * 1e3, 2),
                      "p90": round(float(np.percentile(dec_ms, 90)) * 1e3, 2)},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": decode_bytes},
    }
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
