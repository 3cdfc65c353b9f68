"""Pins of the oracle's mixed-batch (prefill) attention, ``oracle.prefill``.

* PyTorch float64 SDPA (a library routine) over contiguous K/V with an explicit
  causal mask offset by the cached context: query j of a sequence with n query
  tokens and L context tokens may see keys 0..L-n+j.
* A prompt computed in one pass or in slices (chunked prefill) gives the same
  rows bit for bit; a sequence's last row is the decode result bit for bit.
* Pure-Python brute force on tiny shapes.
* Planted mistakes (positions counted from the slice's start, the token not
  seeing itself, one future token seen) are caught.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.paged_attention as pa
from test_oracle import paged_from_contiguous


def mixed_case(rng, lens, nq, hkv, group, d, block_size):
    keys = [rng.standard_normal((hkv, n, d)).astype(np.float32) for n in lens]
    values = [rng.standard_normal((hkv, n, d)).astype(np.float32) for n in lens]
    q = rng.standard_normal((int(sum(nq)), hkv * group, d)).astype(np.float32)
    kp, vp, tables, ctx = paged_from_contiguous(keys, values, block_size, rng)
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    return q, keys, values, kp, vp, tables, ctx, qs


def sdpa_causal(q, keys, values, qs, scale):
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(len(keys)):
        n, L = qs[i + 1] - qs[i], keys[i].shape[1]
        if n == 0:
            continue
        qt = torch.from_numpy(q[qs[i]:qs[i + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(keys[i].astype(np.float64))[None]
        vt = torch.from_numpy(values[i].astype(np.float64))[None]
        pos = torch.arange(L - n, L)[:, None]
        mask = torch.arange(L)[None, :] <= pos                     # [n][L]
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                           enable_gqa=True)
        out[qs[i]:qs[i + 1]] = o[0].permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("seed", range(12))
def test_prefill_matches_torch_sdpa_with_a_causal_offset(seed):
    rng = np.random.default_rng(400 + seed)
    bs = [1, 2, 3, 16][seed % 4]
    group = [1, 2, 4, 8, 3, 16, 5, 7][seed % 8]
    lens = rng.integers(1, 40, size=4)
    nq = [int(rng.integers(1, n + 1)) for n in lens]
    nq[0] = int(lens[0])                     # one whole prompt
    nq[1] = 1                                # one decode row
    q, keys, values, kp, vp, tables, ctx, qs = mixed_case(rng, lens, nq, 2, group, 8, bs)
    scale = 1 / math.sqrt(8)
    got = oracle.prefill(q, kp, vp, tables, qs, ctx, scale, "f32")
    want = sdpa_causal(q, keys, values, qs, scale)
    assert np.abs(got - want).max() <= 1e-12


def test_slices_equal_one_pass_and_last_row_is_decode():
    rng = np.random.default_rng(7)
    L, hkv, group, d, bs = 37, 2, 4, 8, 4
    q, keys, values, kp, vp, tables, ctx, _ = mixed_case(rng, [L], [L], hkv, group, d, bs)
    scale = 0.3
    whole = oracle.prefill(q, kp, vp, tables, [0, L], ctx, scale, "f32")
    # the same prompt in slices of 10, 10, 10, 7: slice k sees context up to its end
    start = 0
    for n in (10, 10, 10, 7):
        part = oracle.prefill(q[start:start + n], kp, vp, tables, [0, n],
                              np.array([start + n], np.int32), scale, "f32")
        assert np.array_equal(part, whole[start:start + n])
        start += n
    last = oracle.decode(q[L - 1:L], kp, vp, tables, ctx, scale, "f32")
    assert np.array_equal(last, whole[L - 1:L])


def test_brute_force_tiny():
    rng = np.random.default_rng(11)
    lens, nq = [5, 3, 6], [2, 3, 1]
    q, keys, values, kp, vp, tables, ctx, qs = mixed_case(rng, lens, nq, 1, 2, 3, 2)
    got = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.7, "f32")
    for i, (L, n) in enumerate(zip(lens, nq)):
        for j in range(n):
            p = L - n + j
            for h in range(2):
                qv = [float(x) for x in q[qs[i] + j, h]]
                s = [0.7 * math.fsum(a * float(b) for a, b in zip(qv, keys[i][0, t]))
                     for t in range(p + 1)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = math.fsum(w)
                for c in range(3):
                    want = math.fsum(w[t] * float(values[i][0, t, c]) for t in range(p + 1)) / tot
                    assert abs(got[qs[i] + j, h, c] - want) <= 1e-12 * max(1.0, abs(want))


def test_conventions():
    rng = np.random.default_rng(3)
    q, keys, values, kp, vp, tables, ctx, qs = mixed_case(rng, [4, 6], [2, 0], 1, 1, 4, 2)
    out = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.5, "f32")
    assert out.shape == (2, 1, 4)
    # more query tokens than context: the rows before position 0 stay zero
    q3 = rng.standard_normal((3, 1, 4)).astype(np.float32)
    out = oracle.prefill(q3, kp, vp, tables[:1], [0, 3], np.array([2], np.int32), 0.5, "f32")
    assert not out[0].any() and out[1:].any()
    with pytest.raises(ValueError):
        oracle.prefill(q, kp, vp, tables, [0, 3, 2], ctx, 0.5, "f32")


@pytest.mark.parametrize("name,target,mutant", [
    ("positions from the slice start", "query_position", lambda L, n, j: j),
    ("token does not see itself", "visible_keys", lambda p: p),
    ("one future token seen", "visible_keys", lambda p: p + 2),
])
def test_planted_prefill_mistakes_are_caught(monkeypatch, name, target, mutant):
    monkeypatch.setattr(pa, target, mutant)
    failures = 0
    for seed in range(8):
        try:
            test_prefill_matches_torch_sdpa_with_a_causal_offset(seed)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    assert failures > 0, f"planted mistake '{name}' went unnoticed"
