"""Helpers shared by the GPU parity tests: upload a workload, run one decode
step through the C ABI, and build the oracle's expected results."""

from __future__ import annotations

import functools
import math

import numpy as np
import torch

import oracle
from paged_kv_cache_93_amd import lib
from paged_kv_cache_93_amd import workloads as W

# bf16 output for bf16 and 8-bit caches (whose values are exact in f32, like bf16)
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 2e-2}


def to_device(arr: np.ndarray, dtype: str) -> torch.Tensor:
    """Device tensor of stored values: float32, bfloat16, or uint8 E4M3 codes."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "fp8":
        return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint8)).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits of a device tensor (uint8 codes, uint16 for bf16, uint32 for f32)."""
    t = t.detach().cpu()
    if t.dtype == torch.uint8:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def bits(arr: np.ndarray, dtype: str) -> np.ndarray:
    return arr.view({"bf16": np.uint16, "fp8": np.uint8, "f32": np.uint32}[dtype])


def upload(w: W.Workload) -> dict:
    qdt = W.query_dtype(w.dtype)
    return dict(
        k_pool=to_device(w.k_pool, w.dtype), v_pool=to_device(w.v_pool, w.dtype),
        q=to_device(w.q, qdt), k_new=to_device(w.k_new, qdt),
        v_new=to_device(w.v_new, qdt),
        block_tables=torch.from_numpy(w.block_tables).cuda(),
        context_lens=torch.from_numpy(w.context_lens).cuda(),
        slot_mapping=torch.from_numpy(w.slot_mapping).cuda(),
        copy_pairs=torch.from_numpy(w.copy_pairs).cuda(),
        k_scale=w.k_scale, v_scale=w.v_scale)


def max_parts_for(w: W.Workload, partition_size: int) -> int:
    return max(1, max(math.ceil(int(n) / partition_size) for n in w.context_lens))


def run_writes(t: dict) -> None:
    if t["copy_pairs"].numel():
        lib.pa_copy_blocks(t["k_pool"], t["v_pool"], t["copy_pairs"])
    lib.pa_kv_append(t["k_pool"], t["v_pool"], t["k_new"], t["v_new"], t["slot_mapping"],
                     k_scale=t["k_scale"], v_scale=t["v_scale"])


def run_decode(t: dict, w: W.Workload, mode="balanced", out_f32: bool = False,
               lse: bool = False):
    """One decode through the C ABI; returns (out, lse or None) on the device.

    mode: "balanced" (pa_decode with a workspace), "single" (pa_decode without
    one) or a partition size in tokens (pa_decode_partitions + pa_splitkv_reduce).
    """
    scale = 1.0 / math.sqrt(w.head_dim)
    out_dt = torch.float32 if (out_f32 or w.dtype == "f32") else torch.bfloat16
    out = torch.empty((w.num_seqs, w.num_heads, w.head_dim), dtype=out_dt, device="cuda")
    lse_t = None
    if mode in ("balanced", "single"):
        ws = None
        if mode == "balanced":
            ws = lib.decode_workspace(w.num_seqs, w.num_heads, w.head_dim)
        lib.pa_decode(t["k_pool"], t["v_pool"], t["q"], t["block_tables"], t["context_lens"],
                      scale, out, workspace=ws, k_scale=t["k_scale"], v_scale=t["v_scale"])
    else:
        psize = int(mode)
        mp = max_parts_for(w, psize)
        po = torch.empty((w.num_seqs, w.num_heads, mp, w.head_dim), dtype=torch.float32,
                         device="cuda")
        pm = torch.empty((w.num_seqs, w.num_heads, mp), dtype=torch.float32, device="cuda")
        ps = torch.empty_like(pm)
        lib.pa_decode_partitions(t["k_pool"], t["v_pool"], t["q"], t["block_tables"],
                                 t["context_lens"], scale, psize, po, pm, ps,
                                 k_scale=t["k_scale"], v_scale=t["v_scale"])
        if lse:
            lse_t = torch.empty((w.num_seqs, w.num_heads), dtype=torch.float32, device="cuda")
        lib.pa_splitkv_reduce(po, pm, ps, t["context_lens"], psize, out, lse=lse_t)
    return out, lse_t


def oracle_pools(w: W.Workload):
    kp, vp = oracle.copy_blocks(w.k_pool, w.v_pool, w.copy_pairs)
    scales = (w.k_scale, w.v_scale) if w.dtype == "fp8" else None
    return oracle.kv_append(kp, vp, w.k_new, w.v_new, w.slot_mapping, fp8_scales=scales)


def oracle_out(w: W.Workload, pools=None):
    kp, vp = oracle_pools(w) if pools is None else pools
    return oracle.decode(w.q, kp, vp, w.block_tables, w.context_lens, 1.0 / math.sqrt(w.head_dim),
                         w.dtype, k_scale=w.k_scale, v_scale=w.v_scale)


@functools.lru_cache(maxsize=16)
def named(k: int, dtype: str | None = None, block_size: int | None = None,
          num_seqs: int | None = None):
    """Named workload with its oracle pools and output (cached across tests)."""
    w = W.make_config(k, dtype=dtype, block_size=block_size, num_seqs=num_seqs)
    pools = oracle_pools(w)
    return w, pools, oracle_out(w, pools)


def max_abs_err(out: torch.Tensor, ref: np.ndarray) -> float:
    got = out.float().cpu().numpy().astype(np.float64)
    assert got.shape == ref.shape
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - ref).max())
