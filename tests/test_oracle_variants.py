"""Pins of the oracle's attention variants: sliding window and ALiBi.

The pages only name the variants ("Paged Attention as a Memory Manager",
section "When It Falls Down"); their definitions are the published ones, and
each is pinned to a library routine or a closed form that does not share the
oracle's code:

* window: float64 PyTorch SDPA over contiguous K/V with a boolean band mask
  (causal and at most W keys back); W >= L or W = 0 gives the plain result bit
  for bit; W = 1 returns the token's own value row exactly;
* ALiBi: float64 SDPA with an additive float mask slope_h * (t - p); zero
  slopes give the plain result bit for bit; the paper's slopes for 8 heads are
  1/2, 1/4, ..., 1/256;
* planted mistakes (window one key too wide, bias sign, one slope for every
  head) are caught.  (A bias measured from the sequence start instead of the
  query is no mistake: it differs by a constant per query row, which the
  softmax cancels.)
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.paged_attention as pa
from test_oracle import paged_from_contiguous
from test_oracle_prefill import mixed_case


def sdpa_masked(q, keys, values, qs, scale, window=0, slopes=None):
    out = np.zeros(q.shape, dtype=np.float64)
    for i in range(len(keys)):
        n, L = qs[i + 1] - qs[i], keys[i].shape[1]
        if n == 0:
            continue
        qt = torch.from_numpy(q[qs[i]:qs[i + 1]].astype(np.float64)).permute(1, 0, 2)[None]
        kt = torch.from_numpy(keys[i].astype(np.float64))[None]
        vt = torch.from_numpy(values[i].astype(np.float64))[None]
        pos = torch.arange(L - n, L, dtype=torch.float64)[:, None]          # [n][1]
        t = torch.arange(L, dtype=torch.float64)[None, :]                    # [1][L]
        allowed = t <= pos
        if window:
            allowed &= t > pos - window
        hq = q.shape[1]
        bias = torch.zeros((hq, n, L), dtype=torch.float64)
        if slopes is not None:
            bias = torch.from_numpy(np.asarray(slopes, np.float64))[:, None, None] * (t - pos)[None]
        mask = torch.where(allowed[None], bias, torch.tensor(-math.inf, dtype=torch.float64))
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask[None], scale=scale,
                                           enable_gqa=True)
        out[qs[i]:qs[i + 1]] = o[0].permute(1, 0, 2).numpy()
    return out


def case(seed, group=2):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 45, size=4)
    nq = [int(rng.integers(1, n + 1)) for n in lens]
    nq[1] = 1
    return mixed_case(rng, lens, nq, 2, group, 8, [1, 2, 4, 16][seed % 4])


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("window", [1, 3, 8, 20])
def test_window_matches_sdpa_with_a_band_mask(seed, window):
    q, keys, values, kp, vp, tables, ctx, qs = case(800 + seed)
    got = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32", window=window)
    want = sdpa_masked(q, keys, values, qs, 0.4, window=window)
    assert np.abs(got - want).max() <= 1e-12


def test_window_special_cases():
    q, keys, values, kp, vp, tables, ctx, qs = case(7)
    plain = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32")
    big = int(ctx.max())
    assert np.array_equal(oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32", window=big), plain)
    one = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32", window=1)
    for i in range(len(keys)):
        n, L = qs[i + 1] - qs[i], keys[i].shape[1]
        for j in range(n):
            v = values[i][:, L - n + j, :].astype(np.float64)        # [Hkv][D]
            assert np.array_equal(one[qs[i] + j], np.repeat(v, q.shape[1] // v.shape[0], axis=0))
    # the decode oracle applies the same window to its single query
    d = oracle.decode(q[qs[1]:qs[1] + 1], kp, vp, tables[1:2], ctx[1:2], 0.4, "f32", window=3)
    assert np.array_equal(d, oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32",
                                            window=3)[qs[1]:qs[1] + 1])


@pytest.mark.parametrize("seed", range(6))
def test_alibi_matches_sdpa_with_an_additive_bias(seed):
    q, keys, values, kp, vp, tables, ctx, qs = case(900 + seed, group=4)
    slopes = oracle.alibi_slopes(q.shape[1])
    got = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32", alibi_slopes=slopes)
    want = sdpa_masked(q, keys, values, qs, 0.4, slopes=slopes)
    assert np.abs(got - want).max() <= 1e-12
    both = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32", window=5, alibi_slopes=slopes)
    assert np.abs(both - sdpa_masked(q, keys, values, qs, 0.4, window=5, slopes=slopes)).max() <= 1e-12


def test_alibi_special_cases():
    q, keys, values, kp, vp, tables, ctx, qs = case(5, group=4)
    plain = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32")
    zero = oracle.prefill(q, kp, vp, tables, qs, ctx, 0.4, "f32", alibi_slopes=np.zeros(8))
    assert np.array_equal(zero, plain)
    # the paper's slopes for 8 heads: 1/2, 1/4, ..., 1/256
    assert np.array_equal(oracle.alibi_slopes(8), 0.5 ** np.arange(1, 9))


@pytest.mark.parametrize("name,target,mutant", [
    ("window one too wide", "attended_range",
     lambda p, w=0: (max(0, p - w) if w else 0, p + 1)),
    ("bias sign", "alibi_bias",
     lambda s, h, lo, hi, p: 0.0 if s is None else -float(s[h]) * (np.arange(lo, hi) - p)),
    ("one slope for every head", "alibi_bias",
     lambda s, h, lo, hi, p: 0.0 if s is None else float(s[0]) * (np.arange(lo, hi) - p)),
])
def test_planted_variant_mistakes_are_caught(monkeypatch, name, target, mutant):
    monkeypatch.setattr(pa, target, mutant)
    failures = 0
    for seed in range(6):
        for check in (lambda: test_window_matches_sdpa_with_a_band_mask(seed, 3),
                      lambda: test_alibi_matches_sdpa_with_an_additive_bias(seed)):
            try:
                check()
            except AssertionError:
                failures += 1
    assert failures > 0, f"planted mistake '{name}' went unnoticed"
