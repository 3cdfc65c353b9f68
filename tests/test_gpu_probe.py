"""The streaming-read probe reads every byte once: the XOR of what its
workgroups fold equals the XOR of all 16-byte chunks of the buffer, for the
whole chip and for XCD subsets."""

import numpy as np
import pytest
import torch

from paged_kv_cache_93_amd import lib

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("groups,mask", [(256, 0xFF), (260, 0xFF), (512, 0x01), (64, 0xA5)])
def test_probe_reads_every_chunk_once(groups, mask):
    rng = np.random.default_rng(5)
    host = rng.integers(0, 2**32, size=(1 << 20) // 4, dtype=np.uint32)  # 4 MiB
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.empty(groups * 16, dtype=torch.uint8, device="cuda")
    lib.probe_stream_read(src, groups, sink, mask)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(groups, 4), axis=0)
    want = np.bitwise_xor.reduce(host.reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)
