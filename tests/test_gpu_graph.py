"""pa_decode's balanced split captured in a HIP graph: every replay gives the
bits of the eager call.

A balanced call enqueues the decode kernel and the merge kernel of the split
sequences, both reading and writing the workspace (or the library's static
scratch); replays alternate with eager calls on the same workspace, and the
output is cleared with a fill kernel before each replay.
"""

import math

import pytest
import torch

from gpu_util import run_writes, upload
from paged_kv_cache_93_amd import lib
from paged_kv_cache_93_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("static", [False, True])
def test_graph_replays_match_eager(static):
    w = W.make_config(2, num_seqs=24)
    t = upload(w)
    run_writes(t)
    scale = 1 / math.sqrt(w.head_dim)
    ws = None if static else lib.decode_workspace(w.num_seqs, w.num_heads, w.head_dim)

    def call(out):
        args = (t["k_pool"], t["v_pool"], t["q"], t["block_tables"], t["context_lens"], scale, out)
        if static:
            lib.pa_decode_static(*args)
        else:
            lib.pa_decode(*args, workspace=ws)

    shape = (w.num_seqs, w.num_heads, w.head_dim)
    eager = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    call(eager)
    torch.cuda.synchronize()
    out = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out)
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        print(f"static={static} replay {i}", flush=True)
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), i
        again = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        call(again)
        torch.cuda.synchronize()
        assert torch.equal(again.view(torch.int16), eager.view(torch.int16)), i
