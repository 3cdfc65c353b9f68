"""Pins of the oracle's 8-bit cache with one scale per KV head.

The pages name 8-bit KV quantisation as halving the bytes of a block ("PagedAttention"
glossary page, section "What paging costs") and leave the granularity of the scale
open; one scale per KV head is the plain refinement of one scale per pool.  Each
function is pinned to PyTorch's float8_e4m3fn cast and binary32 division (the
append) and to the float32 decode of the dequantised values (the decode), head by
head with distinct scales, so a scale taken from the wrong head, one scale used
for every head, or K and V scales swapped all fail.
"""

import numpy as np
import pytest
import torch

import oracle


def _torch_e4m3(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _bits(x):
    return ((x.view(np.uint32) + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)


KS = np.array([2.0 ** -6, 0.0137, 0.75], dtype=np.float64)
VS = np.array([0.0291, 2.0 ** -3, 1.5], dtype=np.float64)


def test_append_quantises_each_head_with_its_own_scale():
    rng = np.random.default_rng(21)
    hkv, bs, d = 3, 4, 16
    k_pool = rng.integers(0, 256, size=(6, hkv, bs, d), dtype=np.uint8)
    v_pool = rng.integers(0, 256, size=(6, hkv, bs, d), dtype=np.uint8)
    kb = _bits(rng.standard_normal((4, hkv, d)).astype(np.float32) * 4)
    vb = _bits(rng.standard_normal((4, hkv, d)).astype(np.float32) * 4)
    slots = [3, 9, -1, 22]
    k2, v2 = oracle.kv_append(k_pool, v_pool, kb, vb, slots, fp8_scales=(KS, VS))
    for n, s in enumerate(slots):
        if s < 0:
            continue
        for g in range(hkv):
            x = (kb[n, g].astype(np.uint32) << np.uint32(16)).view(np.float32)
            y = (vb[n, g].astype(np.uint32) << np.uint32(16)).view(np.float32)
            kq = (torch.from_numpy(x) / torch.tensor(KS[g], dtype=torch.float32)).numpy()
            vq = (torch.from_numpy(y) / torch.tensor(VS[g], dtype=torch.float32)).numpy()
            assert np.array_equal(k2[s // bs, g, s % bs], _torch_e4m3(np.clip(kq, -448, 448)))
            assert np.array_equal(v2[s // bs, g, s % bs], _torch_e4m3(np.clip(vq, -448, 448)))
        k2[s // bs, :, s % bs] = k_pool[s // bs, :, s % bs]
        v2[s // bs, :, s % bs] = v_pool[s // bs, :, s % bs]
    assert np.array_equal(k2, k_pool) and np.array_equal(v2, v_pool)


def _case(rng, hkv=3, group=2, bs=4, d=8, lens=(1, 6, 11)):
    nb = sum(-(-n // bs) for n in lens) + 2
    k = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
    v = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
    for pool in (k, v):  # no NaN codes
        pool[(pool & 0x7F) == 0x7F] = 0x40
    tables = np.zeros((len(lens), 4), dtype=np.int32)
    perm, cur = rng.permutation(nb), 0
    for i, n in enumerate(lens):
        for j in range(-(-n // bs)):
            tables[i, j] = perm[cur]
            cur += 1
    q = _bits(rng.standard_normal((len(lens), hkv * group, d)).astype(np.float32))
    return q, k, v, tables, np.array(lens, dtype=np.int32)


def test_decode_is_the_float32_decode_of_each_heads_dequantised_values():
    rng = np.random.default_rng(22)
    q, k, v, tables, lens = _case(rng)
    ks = np.array([2.0 ** -5, 2.0 ** -2, 2.0 ** 1])  # powers of two: exact in float32
    vs = np.array([2.0 ** 3, 2.0 ** -4, 1.0])
    got = oracle.decode(q, k, v, tables, lens, 0.3, "fp8", k_scale=ks, v_scale=vs)
    k32 = (oracle.fp8_to_f64(k) * ks[None, :, None, None]).astype(np.float32)
    v32 = (oracle.fp8_to_f64(v) * vs[None, :, None, None]).astype(np.float32)
    q32 = oracle.to_f64(q, "bf16").astype(np.float32)
    assert np.array_equal(got, oracle.decode(q32, k32, v32, tables, lens, 0.3, "f32"))


def test_decode_heads_equal_the_single_scale_decode_with_their_scale():
    rng = np.random.default_rng(23)
    q, k, v, tables, lens = _case(rng)
    got = oracle.decode(q, k, v, tables, lens, 0.3, "fp8", k_scale=KS, v_scale=VS)
    group = q.shape[1] // k.shape[1]
    for g in range(k.shape[1]):
        one = oracle.decode(q, k, v, tables, lens, 0.3, "fp8", k_scale=KS[g], v_scale=VS[g])
        heads = slice(g * group, (g + 1) * group)
        assert np.array_equal(got[:, heads], one[:, heads])
    # equal per-head scales are the single scale, bit for bit
    same = oracle.decode(q, k, v, tables, lens, 0.3, "fp8", k_scale=np.full(3, 0.5),
                         v_scale=np.full(3, 0.25))
    assert np.array_equal(same, oracle.decode(q, k, v, tables, lens, 0.3, "fp8", k_scale=0.5,
                                              v_scale=0.25))


def test_prefill_and_partitions_follow_the_same_scales():
    rng = np.random.default_rng(24)
    q, k, v, tables, lens = _case(rng)
    ref = oracle.decode(q, k, v, tables, lens, 0.3, "fp8", k_scale=KS, v_scale=VS)
    po, pm, ps = oracle.decode_partitions(q, k, v, tables, lens, 0.3, "fp8", 4, k_scale=KS,
                                          v_scale=VS)
    merged, _ = oracle.splitkv_merge(po, pm, ps, lens, 4)
    np.testing.assert_allclose(merged, ref, rtol=1e-12, atol=1e-12)
    # a decode batch through prefill: one query row per sequence, at its last position
    qs = np.arange(len(lens) + 1, dtype=np.int32)
    pf = oracle.prefill(q, k, v, tables, qs, lens, 0.3, "fp8", k_scale=KS, v_scale=VS)
    np.testing.assert_allclose(pf, ref, rtol=1e-12, atol=1e-12)


class _OneScaleForAll:
    """Planted mistake: head 0's scale for every head."""

    def __enter__(self):
        self.saved = oracle.paged_attention.head_scale
        oracle.paged_attention.head_scale = lambda s, g: self.saved(s, 0)

    def __exit__(self, *exc):
        oracle.paged_attention.head_scale = self.saved


def test_planted_mistake_one_scale_for_every_head_is_caught():
    with _OneScaleForAll():
        with pytest.raises(AssertionError):
            test_decode_heads_equal_the_single_scale_decode_with_their_scale()
