"""8-token blocks on the MFMA decode path (a 16-row tile holds a pair of blocks).

A pair's second block is masked when it lies past the sequence or past the
partition's end, and the pairs start at the partition's (or window's) first
block.  Partitions of an odd number of blocks (24, 40 and 56 tokens) end in
the middle of a pair, so each partition's partial - output row, max and sum -
is compared with the oracle's partials one by one (a second block read across
the partition's end would add the next partition's rows to this one).
Tolerances are those of the float32-partials test: 1e-5 absolute on the rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_util import max_parts_for, run_writes, upload
from paged_kv_cache_93_amd import lib
from paged_kv_cache_93_amd import workloads as W

pytestmark = pytest.mark.gpu

LENS = [1, 7, 8, 9, 15, 16, 17, 23, 24, 25, 40, 41, 100, 257]


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("psize", [8, 16, 24, 40, 56])
@pytest.mark.parametrize("group", [1, 4, 8])
def test_partials_with_odd_partition_blocks(dtype, psize, group):
    w = W.small_random(410 + psize + group, dtype=dtype, num_seqs=len(LENS),
                       num_heads=2 * group, num_kv_heads=2, head_dim=128, block_size=8,
                       lens=LENS)
    if dtype == "fp8":
        w.k_scale, w.v_scale = 0.0137, 0.0291
    scales = (w.k_scale, w.v_scale) if dtype == "fp8" else None
    kp, vp = oracle.kv_append(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping,
                              fp8_scales=scales)
    scale = 1 / math.sqrt(128)
    mp = max_parts_for(w, psize)
    eo, em, es = oracle.decode_partitions(w.q, kp, vp, w.block_tables, w.context_lens, scale,
                                          dtype, psize, max_parts=mp, k_scale=w.k_scale,
                                          v_scale=w.v_scale)
    t = upload(w)
    run_writes(t)
    S, H = w.num_seqs, w.num_heads
    po = torch.full((S, H, mp, 128), float("nan"), device="cuda")
    pm = torch.full((S, H, mp), float("nan"), device="cuda")
    ps = torch.full((S, H, mp), float("nan"), device="cuda")
    lib.pa_decode_partitions(t["k_pool"], t["v_pool"], t["q"], t["block_tables"],
                             t["context_lens"], scale, psize, po, pm, ps,
                             k_scale=t["k_scale"], v_scale=t["v_scale"])
    torch.cuda.synchronize()
    po, pm, ps = po.cpu().double().numpy(), pm.cpu().double().numpy(), ps.cpu().double().numpy()
    for i, n in enumerate(w.context_lens):
        live = math.ceil(int(n) / psize)
        np.testing.assert_allclose(po[i, :, :live], eo[i, :, :live], rtol=0, atol=1e-5)
        np.testing.assert_allclose(pm[i, :, :live], em[i, :, :live], rtol=1e-6, atol=1e-5)
        np.testing.assert_allclose(ps[i, :, :live], es[i, :, :live], rtol=1e-5, atol=0)
        assert np.isnan(po[i, :, live:]).all()
