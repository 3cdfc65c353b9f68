"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test fixes part of ``oracle.paged_attention`` against something the oracle
does not compute itself: values printed on the pages (``tests/golden``), a
library routine (PyTorch's float64 scaled-dot-product attention, SciPy's
logsumexp, PyTorch's bfloat16 widening), closed forms, and invariants the
pages state (non-contiguous storage and sharing are invisible to the result).
The last test plants plausible mistakes in the oracle and checks that these
pins catch each one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle
from oracle import paged_attention as pa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
NAN32 = np.float32(np.nan)


# ---------------------------------------------------------------------------
# helpers: build paged inputs from contiguous per-sequence K/V (test-side only)
# ---------------------------------------------------------------------------

def paged_from_contiguous(keys, values, block_size, rng, extra_blocks=3, poison=True):
    """Scatter per-sequence contiguous K/V ([Hkv][L][D] float32 each) into pools.

    Physical blocks are a random permutation; every slot no sequence owns, and
    every table entry past a sequence's last block, points at NaN data.
    """
    hkv, _, d = keys[0].shape
    counts = [-(-k.shape[1] // block_size) for k in keys]
    nb = sum(counts) + extra_blocks
    perm = rng.permutation(nb)
    fill = NAN32 if poison else np.float32(0)
    k_pool = np.full((nb, hkv, block_size, d), fill, dtype=np.float32)
    v_pool = np.full((nb, hkv, block_size, d), fill, dtype=np.float32)
    width = max(counts + [1]) + 2
    spare = int(perm[-1])  # never assigned: stays poisoned
    tables = np.full((len(keys), width), spare, dtype=np.int32)
    cursor = 0
    for i, (k, v) in enumerate(zip(keys, values)):
        length = k.shape[1]
        for j in range(counts[i]):
            phys = int(perm[cursor])
            cursor += 1
            tables[i, j] = phys
            lo, hi = j * block_size, min(length, (j + 1) * block_size)
            k_pool[phys, :, : hi - lo, :] = k[:, lo:hi, :]
            v_pool[phys, :, : hi - lo, :] = v[:, lo:hi, :]
    lens = np.array([k.shape[1] for k in keys], dtype=np.int32)
    return k_pool, v_pool, tables, lens


def random_case(rng, num_seqs, hkv, group, d, lens):
    q = rng.standard_normal((num_seqs, hkv * group, d)).astype(np.float32)
    keys = [rng.standard_normal((hkv, n, d)).astype(np.float32) for n in lens]
    values = [rng.standard_normal((hkv, n, d)).astype(np.float32) for n in lens]
    return q, keys, values


def sdpa_reference(q, keys, values, scale):
    """PyTorch float64 SDPA over contiguous K/V (library routine), GQA by enable_gqa."""
    outs = []
    for i in range(q.shape[0]):
        qt = torch.from_numpy(q[i].astype(np.float64))[None, :, None, :]      # [1,Hq,1,D]
        kt = torch.from_numpy(keys[i].astype(np.float64))[None]               # [1,Hkv,L,D]
        vt = torch.from_numpy(values[i].astype(np.float64))[None]
        o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=True)
        outs.append(o[0, :, 0, :].numpy())
    return np.stack(outs)


# ---------------------------------------------------------------------------
# value decoding
# ---------------------------------------------------------------------------

def test_bf16_widening_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.to_f64(bits, "bf16")
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# the pages' worked example and printed counts
# ---------------------------------------------------------------------------

def test_worked_example_slot_mapping():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    bs = g["block_size"]
    for p in range(g["num_tokens"]):
        slot = oracle.slot_of(g["block_table"], p, bs)
        assert slot // bs == g["token_physical_block"][p]
        assert slot % bs == g["token_row_in_block"][p]
    assert oracle.blocks_needed(g["num_tokens"], bs) == len(g["block_table"])


def test_worked_example_attention_is_contiguous_attention():
    """Paged attention over the example's table equals attention over t0..t4."""
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    bs, n, d = g["block_size"], g["num_tokens"], 8
    rng = np.random.default_rng(7)
    k_tok = rng.standard_normal((n, d)).astype(np.float32)
    v_tok = rng.standard_normal((n, d)).astype(np.float32)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k_pool = np.full((12, 1, bs, d), NAN32, dtype=np.float32)
    v_pool = np.full((12, 1, bs, d), NAN32, dtype=np.float32)
    for p in range(n):
        b, r = g["token_physical_block"][p], g["token_row_in_block"][p]
        k_pool[b, 0, r] = k_tok[p]
        v_pool[b, 0, r] = v_tok[p]
    table = np.array([g["block_table"] + [0]], dtype=np.int32)  # entry 3 never read
    lens = np.array([n], dtype=np.int32)
    scale = 1 / math.sqrt(d)
    got = oracle.decode(q, k_pool, v_pool, table, lens, scale, "f32")
    ref = sdpa_reference(q, [k_tok[None]], [v_tok[None]], scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)
    # same data stored contiguously (blocks 0,1,2 in order) gives the same bits
    kc = np.full((3, 1, bs, d), NAN32, dtype=np.float32)
    vc = np.full((3, 1, bs, d), NAN32, dtype=np.float32)
    for p in range(n):
        kc[p // bs, 0, p % bs] = k_tok[p]
        vc[p // bs, 0, p % bs] = v_tok[p]
    again = oracle.decode(q, kc, vc, np.array([[0, 1, 2]], dtype=np.int32), lens, scale, "f32")
    assert np.array_equal(got, again)


def test_block_counts_printed_on_the_pages():
    cases = json.load(open(os.path.join(GOLDEN, "block_counts.json")))["cases"]
    for c in cases:
        bs = c["block_size"]
        if "blocks" in c:
            assert oracle.blocks_needed(c["tokens"], bs) == c["blocks"], c["what"]
        if "full_blocks" in c:
            assert c["tokens"] // bs == c["full_blocks"], c["what"]
            total = oracle.blocks_needed(c["of_total_tokens"], bs)
            assert total - c["full_blocks"] == c["new_blocks"], c["what"]
        if "utilisation_percent" in c:
            used = c["tokens"] / (oracle.blocks_needed(c["tokens"], bs) * bs)
            assert round(100 * used) == c["utilisation_percent"], c["what"]
        if "max_slack" in c:
            worst = max(oracle.last_block_waste(t, bs) for t in range(1, 10 * bs))
            assert worst == c["max_slack"], c["what"]


# ---------------------------------------------------------------------------
# library pin: PyTorch float64 SDPA on random tiny shapes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(40))
def test_decode_matches_torch_sdpa(seed):
    rng = np.random.default_rng(1000 + seed)
    num_seqs = int(rng.integers(1, 4))
    hkv = int(rng.choice([1, 2, 3]))
    group = int(rng.choice([1, 2, 3, 4, 5, 7, 16]))
    d = int(rng.choice([4, 8, 16, 64]))
    bs = int(rng.choice([1, 2, 4, 16]))
    lens = [int(x) for x in rng.integers(1, 41, size=num_seqs)]
    q, keys, values = random_case(rng, num_seqs, hkv, group, d, lens)
    k_pool, v_pool, tables, lens_arr = paged_from_contiguous(keys, values, bs, rng)
    scale = 1 / math.sqrt(d)
    got = oracle.decode(q, k_pool, v_pool, tables, lens_arr, scale, "f32")
    ref = sdpa_reference(q, keys, values, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def _single(q_vec, k_rows, v_rows, bs=4, scale=None):
    d = q_vec.shape[-1]
    rng = np.random.default_rng(3)
    k_pool, v_pool, tables, lens = paged_from_contiguous([k_rows[None]], [v_rows[None]], bs, rng)
    scale = 1 / math.sqrt(d) if scale is None else scale
    return oracle.decode(q_vec.reshape(1, 1, d), k_pool, v_pool, tables, lens, scale, "f32")[0, 0]


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(11)
    for d in (4, 64, 128):
        k = rng.standard_normal((1, d)).astype(np.float32)
        v = rng.standard_normal((1, d)).astype(np.float32)
        q = rng.standard_normal(d).astype(np.float32)
        assert np.array_equal(_single(q, k, v), v[0].astype(np.float64))


def test_zero_query_is_the_mean_of_values():
    rng = np.random.default_rng(12)
    k = rng.standard_normal((37, 16)).astype(np.float32)
    v = rng.standard_normal((37, 16)).astype(np.float32)
    got = _single(np.zeros(16, np.float32), k, v)
    np.testing.assert_allclose(got, v.astype(np.float64).mean(axis=0), rtol=0, atol=1e-14)


def test_constant_values_and_affine_values():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((29, 8)).astype(np.float32)
    q = rng.standard_normal(8).astype(np.float32)
    c = np.float32(-2.5)
    got = _single(q, k, np.full((29, 8), c, dtype=np.float32))
    np.testing.assert_allclose(got, np.full(8, float(c)), rtol=0, atol=1e-14)
    # multiples of 2^-10 keep 2v + 0.5 exact in float32
    v = (np.round(rng.standard_normal((29, 8)) * 1024) / 1024).astype(np.float32)
    base = _single(q, k, v)
    shifted = _single(q, k, (np.float32(2) * v + np.float32(0.5)).astype(np.float32))
    np.testing.assert_allclose(shifted, 2 * base + 0.5, rtol=0, atol=1e-13)


def test_two_tokens_logistic_closed_form():
    rng = np.random.default_rng(14)
    d = 16
    k = rng.standard_normal((2, d)).astype(np.float32)
    v = rng.standard_normal((2, d)).astype(np.float32)
    q = rng.standard_normal(d).astype(np.float32)
    scale = 1 / math.sqrt(d)
    k64, v64, q64 = k.astype(np.float64), v.astype(np.float64), q.astype(np.float64)
    delta = scale * (float(np.dot(q64, k64[0])) - float(np.dot(q64, k64[1])))
    w0 = 1 / (1 + math.exp(-delta))
    expect = w0 * v64[0] + (1 - w0) * v64[1]
    np.testing.assert_allclose(_single(q, k, v, bs=1), expect, rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(15)
    d = 32
    k = rng.standard_normal((20, d)).astype(np.float32)
    v = rng.standard_normal((20, d)).astype(np.float32)
    j = 13
    q = np.zeros(d, np.float32)
    q[0] = 1.0
    k[:, 0] = 0.0
    k[j, 0] = 400.0  # score gap 400/sqrt(32) ~ 70.7, so every other weight is < e^-70
    np.testing.assert_allclose(_single(q, k, v), v[j].astype(np.float64), rtol=0, atol=1e-25)


# ---------------------------------------------------------------------------
# invariants the pages state
# ---------------------------------------------------------------------------

def test_physical_permutation_is_invisible_bit_for_bit():
    rng = np.random.default_rng(21)
    q, keys, values = random_case(rng, 3, 2, 4, 32, [50, 17, 64])
    k1, v1, t1, lens = paged_from_contiguous(keys, values, 16, np.random.default_rng(1))
    k2, v2, t2, _ = paged_from_contiguous(keys, values, 16, np.random.default_rng(2))
    assert not np.array_equal(t1, t2)
    a = oracle.decode(q, k1, v1, t1, lens, 0.17, "f32")
    b = oracle.decode(q, k2, v2, t2, lens, 0.17, "f32")
    assert np.array_equal(a, b)


def test_shared_prefix_equals_private_copies():
    """Tables pointing at shared prefix blocks give the same bits as private copies."""
    rng = np.random.default_rng(22)
    hkv, group, d, bs = 2, 2, 16, 4
    prefix = [rng.standard_normal((hkv, 12, d)).astype(np.float32) for _ in range(2)]  # K, V
    suffix_lens = [3, 9, 1, 5]
    keys = [np.concatenate([prefix[0], rng.standard_normal((hkv, n, d)).astype(np.float32)], axis=1)
            for n in suffix_lens]
    values = [np.concatenate([prefix[1], rng.standard_normal((hkv, n, d)).astype(np.float32)], axis=1)
              for n in suffix_lens]
    q = rng.standard_normal((4, hkv * group, d)).astype(np.float32)
    k_priv, v_priv, t_priv, lens = paged_from_contiguous(keys, values, bs, rng)
    private = oracle.decode(q, k_priv, v_priv, t_priv, lens, 0.25, "f32")
    # shared layout: sequences 1..3 point their first 3 logical blocks at sequence 0's
    t_shared = t_priv.copy()
    k_sh, v_sh = k_priv.copy(), v_priv.copy()
    for i in range(1, 4):
        for j in range(3):
            k_sh[t_priv[i, j]] = NAN32  # the private copy is gone
            v_sh[t_priv[i, j]] = NAN32
            t_shared[i, j] = t_priv[0, j]
    shared = oracle.decode(q, k_sh, v_sh, t_shared, lens, 0.25, "f32")
    assert np.array_equal(private, shared)


@pytest.mark.parametrize("bs", [1, 2, 3, 16, 32])
def test_block_size_is_invisible_bit_for_bit(bs):
    rng = np.random.default_rng(23)
    q, keys, values = random_case(rng, 2, 2, 2, 16, [45, 70])
    k16, v16, t16, lens = paged_from_contiguous(keys, values, 16, np.random.default_rng(4))
    kb, vb, tb, _ = paged_from_contiguous(keys, values, bs, np.random.default_rng(5))
    a = oracle.decode(q, k16, v16, t16, lens, 0.3, "f32")
    b = oracle.decode(q, kb, vb, tb, lens, 0.3, "f32")
    assert np.array_equal(a, b)


def test_poisoned_unowned_slots_do_not_matter():
    rng = np.random.default_rng(24)
    q, keys, values = random_case(rng, 3, 1, 2, 8, [5, 16, 33])
    kp, vp, t, lens = paged_from_contiguous(keys, values, 16, np.random.default_rng(6), poison=True)
    kz, vz, _, _ = paged_from_contiguous(keys, values, 16, np.random.default_rng(6), poison=False)
    a = oracle.decode(q, kp, vp, t, lens, 0.35, "f32")
    b = oracle.decode(q, kz, vz, t, lens, 0.35, "f32")
    assert np.isfinite(a).all() and np.array_equal(a, b)


# ---------------------------------------------------------------------------
# split-KV partials and their merge
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("psize", [1, 2, 5, 16, 48, 512])
def test_partition_merge_equals_unsplit(psize):
    rng = np.random.default_rng(31)
    q, keys, values = random_case(rng, 3, 2, 2, 16, [1, 47, 130])
    kp, vp, t, lens = paged_from_contiguous(keys, values, 16, rng)
    scale = 0.25
    full = oracle.decode(q, kp, vp, t, lens, scale, "f32")
    po, pm, ps = oracle.decode_partitions(q, kp, vp, t, lens, scale, "f32", psize)
    merged, lse = oracle.splitkv_merge(po, pm, ps, lens, psize)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-13)
    # lse against SciPy's logsumexp of the scores
    for i in range(3):
        for h in range(4):
            k64 = keys[i][h // 2].astype(np.float64)
            scores = scale * (k64 @ q[i, h].astype(np.float64))
            assert abs(lse[i, h] - logsumexp(scores)) < 1e-12


def test_single_partition_is_the_unsplit_result():
    rng = np.random.default_rng(32)
    q, keys, values = random_case(rng, 2, 1, 4, 8, [20, 31])
    kp, vp, t, lens = paged_from_contiguous(keys, values, 4, rng)
    full = oracle.decode(q, kp, vp, t, lens, 0.4, "f32")
    po, pm, ps = oracle.decode_partitions(q, kp, vp, t, lens, 0.4, "f32", 64)
    assert np.array_equal(po[:, :, 0, :], full)
    merged, _ = oracle.splitkv_merge(po, pm, ps, lens, 64)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-15)


def test_merge_closed_form_and_unused_partitions():
    o = np.zeros((1, 1, 4, 3))
    o[0, 0, 0] = [1.0, 2.0, 3.0]
    o[0, 0, 1] = [-1.0, 0.0, 5.0]
    o[0, 0, 2:] = np.nan  # past the sequence's partitions: never read
    m = np.array([[[0.7, 0.7, np.nan, np.nan]]])
    s = np.array([[[3.0, 1.0, np.nan, np.nan]]])
    out, lse = oracle.splitkv_merge(o, m, s, [20], 10)  # 20 tokens, 10 per partition
    np.testing.assert_allclose(out[0, 0], (3 * o[0, 0, 0] + 1 * o[0, 0, 1]) / 4, rtol=0, atol=1e-15)
    assert abs(lse[0, 0] - (0.7 + math.log(4.0))) < 1e-15
    # a partition whose max is far below the others gets a weight of exp(-gap)
    m2 = np.array([[[0.0, -50.0, np.nan, np.nan]]])
    out2, _ = oracle.splitkv_merge(o, m2, s, [20], 10)
    w1 = 1.0 * math.exp(-50.0)
    np.testing.assert_allclose(out2[0, 0], (3 * o[0, 0, 0] + w1 * o[0, 0, 1]) / (3 + w1), rtol=1e-15)


def test_empty_sequence_conventions():
    q = np.ones((1, 2, 4), np.float32)
    pool = np.full((2, 1, 4, 4), NAN32, np.float32)
    t = np.zeros((1, 1), np.int32)
    lens = np.zeros(1, np.int32)
    assert np.array_equal(oracle.decode(q, pool, pool, t, lens, 0.5, "f32"), np.zeros((1, 2, 4)))
    po, pm, ps = oracle.decode_partitions(q, pool, pool, t, lens, 0.5, "f32", 4, max_parts=1)
    assert np.isneginf(pm).all() and (ps == 0).all() and (po == 0).all()
    out, lse = oracle.splitkv_merge(po, pm, ps, lens, 4)
    assert (out == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------------------
# byte-exact writes
# ---------------------------------------------------------------------------

def test_append_places_rows_at_slots_and_nothing_else():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    bs = g["block_size"]
    rng = np.random.default_rng(41)
    k_pool = rng.integers(0, 1 << 16, size=(12, 3, bs, 8), dtype=np.uint16)
    v_pool = rng.integers(0, 1 << 16, size=(12, 3, bs, 8), dtype=np.uint16)
    k_new = rng.integers(0, 1 << 16, size=(2, 3, 8), dtype=np.uint16)
    v_new = rng.integers(0, 1 << 16, size=(2, 3, 8), dtype=np.uint16)
    # token t4 of the worked example, and a token with no slot
    slot = oracle.slot_of(g["block_table"], 4, bs)
    k2, v2 = oracle.kv_append(k_pool, v_pool, k_new, v_new, [slot, -1])
    assert np.array_equal(k2[11, :, 0, :], k_new[0]) and np.array_equal(v2[11, :, 0, :], v_new[0])
    mask = np.ones(k_pool.shape, bool)
    mask[11, :, 0, :] = False
    assert np.array_equal(k2[mask], k_pool[mask]) and np.array_equal(v2[mask], v_pool[mask])
    with pytest.raises(ValueError):
        oracle.kv_append(k_pool, v_pool, k_new, v_new, [slot, slot])


def test_copy_on_write_semantics():
    """Copy a shared block, remap one table, write into the copy; the others
    still read the original ("Paged Attention as a Memory Manager", section
    "Prefix Caching and Copy-on-Write")."""
    rng = np.random.default_rng(42)
    bs, d = 4, 8
    k_pool = rng.standard_normal((6, 1, bs, d)).astype(np.float32)
    v_pool = rng.standard_normal((6, 1, bs, d)).astype(np.float32)
    k_pool[5] = NAN32
    v_pool[5] = NAN32
    tables = np.array([[0, 1], [0, 2]], dtype=np.int32)  # block 0 shared
    lens = np.array([8, 8], dtype=np.int32)
    q = rng.standard_normal((2, 1, d)).astype(np.float32)
    before = oracle.decode(q, k_pool, v_pool, tables, lens, 0.3, "f32")
    k2, v2 = oracle.copy_blocks(k_pool, v_pool, [(0, 5)])
    assert np.array_equal(k2[5], k_pool[0]) and np.array_equal(k2[:5], k_pool[:5])
    tables[1, 0] = 5
    same = oracle.decode(q, k2, v2, tables, lens, 0.3, "f32")
    assert np.array_equal(same, before)  # a copy changes no result
    knew = rng.standard_normal((1, 1, d)).astype(np.float32)
    vnew = rng.standard_normal((1, 1, d)).astype(np.float32)
    k3, v3 = oracle.kv_append(k2, v2, knew, vnew, [oracle.slot_of(tables[1], 3, bs)])
    after = oracle.decode(q, k3, v3, tables, lens, 0.3, "f32")
    assert np.array_equal(after[0], before[0])      # the other sequence is untouched
    assert not np.array_equal(after[1], before[1])  # the diverged one sees its write
    with pytest.raises(ValueError):
        oracle.copy_blocks(k_pool, v_pool, [(0, 5), (5, 4)])


# ---------------------------------------------------------------------------
# the 8-bit (E4M3) cache
# ---------------------------------------------------------------------------

def _torch_e4m3(values_f32):
    """PyTorch's float32 -> float8_e4m3fn cast (round to nearest even; NaN past 464)."""
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_table_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = oracle.fp8_to_f64(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    keep = ~np.isnan(ref)
    assert np.array_equal(ref[keep], got[keep])
    assert np.array_equal(np.signbit(ref[keep]), np.signbit(got[keep]))


def test_e4m3_closed_forms():
    v = oracle.e4m3_value
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) < 0
    assert v(0x01) == 2.0 ** -9 and v(0x07) == 7 * 2.0 ** -9   # subnormals m/8 * 2^-6
    assert v(0x08) == 2.0 ** -6                                 # smallest normal
    assert v(0x30) == 0.5 and v(0x38) == 1.0 and v(0x40) == 2.0 and v(0xB8) == -1.0
    assert v(0x7E) == 448.0 == oracle.E4M3_MAX and v(0xFE) == -448.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert v(0x78) == 256.0 and v(0x3F) == 1.875


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(7)
    finite = oracle.fp8_to_f64(np.arange(0x7F))  # 0 .. 448, increasing
    mids = (finite[:-1] + finite[1:]) / 2          # every tie between neighbours
    mags = np.exp(rng.uniform(math.log(2.0 ** -12), math.log(460.0), 30000))
    vals = np.concatenate([finite, mids, mags, [464.0]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    assert np.array_equal(oracle.fp8_encode(vals.astype(np.float64)), _torch_e4m3(vals))


def test_e4m3_encode_saturates_and_keeps_nan():
    enc = lambda x: int(oracle.fp8_encode(np.array([x]))[0])
    for x in (448.0, 448.5, 464.0, 465.0, 1.0e30, math.inf):
        assert enc(x) == 0x7E and enc(-x) == 0xFE
    assert enc(math.nan) == 0x7F
    assert enc(-0.0) == 0x80 and enc(-1e-10) == 0x80 and enc(1e-10) == 0x00
    # the library clamps where PyTorch's cast gives NaN
    assert math.isnan(torch.tensor(465.0).to(torch.float8_e4m3fn).float().item())


def test_e4m3_round_trip_of_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.fp8_encode(oracle.fp8_to_f64(codes)), codes)


@pytest.mark.parametrize("scale", [2.0 ** -6, 0.0123, 3.0])
def test_fp8_quantize_divides_in_binary32(scale):
    rng = np.random.default_rng(11)
    x = rng.standard_normal(4000).astype(np.float32)
    bits = ((x.view(np.uint32) + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)
    x32 = torch.from_numpy((bits.astype(np.uint32) << np.uint32(16)).view(np.float32))
    quot = (x32 / torch.tensor(scale, dtype=torch.float32)).numpy()
    quot = np.clip(quot, -448.0, 448.0)
    assert np.array_equal(oracle.fp8_quantize(bits, scale), _torch_e4m3(quot))


def _fp8_case(rng, bs=4, d=8, hkv=2, group=2, lens=(1, 5, 9, 13)):
    nb = sum(-(-n // bs) for n in lens) + 2
    k_codes = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
    v_codes = rng.integers(0, 256, size=(nb, hkv, bs, d), dtype=np.uint8)
    for pool in (k_codes, v_codes):  # no NaN codes where rows are read
        pool[(pool & 0x7F) == 0x7F] = 0x38
    perm = rng.permutation(nb)
    tables = np.zeros((len(lens), 8), dtype=np.int32)
    cursor = 0
    for i, n in enumerate(lens):
        for j in range(-(-n // bs)):
            tables[i, j] = perm[cursor]
            cursor += 1
    qf = rng.standard_normal((len(lens), hkv * group, d)).astype(np.float32)
    q_bits = ((qf.view(np.uint32) + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)
    return q_bits, k_codes, v_codes, tables, np.array(lens, dtype=np.int32)


def test_fp8_decode_is_decode_of_the_dequantised_values():
    rng = np.random.default_rng(5)
    q_bits, k_codes, v_codes, tables, lens = _fp8_case(rng)
    ks, vs = 2.0 ** -5, 2.0 ** 3  # powers of two: the dequantised values are float32
    got = oracle.decode(q_bits, k_codes, v_codes, tables, lens, 0.25, "fp8", k_scale=ks, v_scale=vs)
    k32 = (oracle.fp8_to_f64(k_codes) * ks).astype(np.float32)
    v32 = (oracle.fp8_to_f64(v_codes) * vs).astype(np.float32)
    q32 = oracle.to_f64(q_bits, "bf16").astype(np.float32)
    ref = oracle.decode(q32, k32, v32, tables, lens, 0.25, "f32")
    assert np.array_equal(got, ref)
    # and the scales act where they should: scores see k_scale, outputs scale with v_scale
    swapped = oracle.decode(q_bits, k_codes, v_codes, tables, lens, 0.25, "fp8", k_scale=vs, v_scale=ks)
    assert not np.allclose(swapped, got)
    doubled = oracle.decode(q_bits, k_codes, v_codes, tables, lens, 0.25, "fp8", k_scale=ks, v_scale=2 * vs)
    assert np.array_equal(doubled, 2 * got)
    po, pm, ps = oracle.decode_partitions(q_bits, k_codes, v_codes, tables, lens, 0.25, "fp8", 4,
                                          k_scale=ks, v_scale=vs)
    merged, _ = oracle.splitkv_merge(po, pm, ps, lens, 4)
    np.testing.assert_allclose(merged, got, rtol=1e-12, atol=1e-12)


def test_fp8_append_writes_quantised_rows():
    rng = np.random.default_rng(9)
    bs, d, hkv = 4, 16, 2
    k_pool = rng.integers(0, 256, size=(5, hkv, bs, d), dtype=np.uint8)
    v_pool = rng.integers(0, 256, size=(5, hkv, bs, d), dtype=np.uint8)
    xk = rng.standard_normal((3, hkv, d)).astype(np.float32) * 8
    xv = rng.standard_normal((3, hkv, d)).astype(np.float32) * 8
    to_bits = lambda x: ((x.view(np.uint32) + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16)
    kb, vb = to_bits(xk), to_bits(xv)
    slots = [6, -1, 17]
    ks, vs = 0.05, 2.0 ** -4
    k2, v2 = oracle.kv_append(k_pool, v_pool, kb, vb, slots, fp8_scales=(ks, vs))
    for n, s in enumerate(slots):
        if s < 0:
            continue
        kq = (torch.from_numpy(oracle.to_f64(kb[n], "bf16").astype(np.float32)) /
              torch.tensor(ks, dtype=torch.float32)).numpy()
        vq = (torch.from_numpy(oracle.to_f64(vb[n], "bf16").astype(np.float32)) /
              torch.tensor(vs, dtype=torch.float32)).numpy()
        # saturation at 448 (PyTorch's cast would give NaN past 464)
        assert np.array_equal(k2[s // bs, :, s % bs], _torch_e4m3(np.clip(kq, -448, 448)))
        assert np.array_equal(v2[s // bs, :, s % bs], _torch_e4m3(np.clip(vq, -448, 448)))
        k2[s // bs, :, s % bs] = k_pool[s // bs, :, s % bs]
        v2[s // bs, :, s % bs] = v_pool[s // bs, :, s % bs]
    assert np.array_equal(k2, k_pool) and np.array_equal(v2, v_pool)  # nothing else moved


# ---------------------------------------------------------------------------
# planted mistakes are caught by the pins above
# ---------------------------------------------------------------------------

def _gather_off_by_one_row(pool, table_row, length, block_size, kv_head):
    rows = [pool[int(table_row[p // block_size]), kv_head, (p + 1) % block_size] for p in range(length)]
    return np.stack(rows) if rows else pool[:0, kv_head, 0, :]


def _gather_ignores_table(pool, table_row, length, block_size, kv_head):
    rows = [pool[p // block_size, kv_head, p % block_size] for p in range(length)]
    return np.stack(rows) if rows else pool[:0, kv_head, 0, :]


def _gather_drops_last_token(pool, table_row, length, block_size, kv_head):
    return _real_gather(pool, table_row, max(length - 1, 1), block_size, kv_head)


def _softmax_unnormalised(scores, values):
    m = scores.max()
    w = np.exp(scores - m)
    return w @ values, m, w.sum()


def _softmax_wrong_sign(scores, values):
    m = (-scores).max()
    w = np.exp(-scores - m)
    return (w @ values) / w.sum(), m, w.sum()


_real_gather = pa.gather_rows


@pytest.mark.parametrize("name,target,mutant", [
    ("row offset", "gather_rows", _gather_off_by_one_row),
    ("table ignored", "gather_rows", _gather_ignores_table),
    ("last token dropped", "gather_rows", _gather_drops_last_token),
    ("no normalisation", "_softmax_weighted_sum", _softmax_unnormalised),
    ("sign of scores", "_softmax_weighted_sum", _softmax_wrong_sign),
])
def test_planted_mistakes_are_caught(monkeypatch, name, target, mutant):
    monkeypatch.setattr(pa, target, mutant)
    failures = 0
    for seed in range(6):
        try:
            test_decode_matches_torch_sdpa(seed)
        except AssertionError:
            failures += 1
    try:
        test_worked_example_attention_is_contiguous_attention()
    except AssertionError:
        failures += 1
    assert failures > 0, f"planted mistake '{name}' went unnoticed"


def _e4m3_table_bias8():
    out = []
    for c in range(256):
        e, m = (c >> 3) & 0xF, c & 7
        sign = -1.0 if c & 0x80 else 1.0
        out.append(sign * (math.ldexp(m, -10) if e == 0 else math.ldexp(8 + m, e - 11)))
    return np.array(out)


def _encode_ties_toward_zero(values):
    y = np.asarray(values, dtype=np.float64)
    mags = pa._E4M3_MAGNITUDES
    out = []
    for v in y.reshape(-1):
        a = min(abs(v), 448.0)
        idx = int(np.argmin(np.abs(mags - a)))  # the first of two equally near: the smaller
        out.append((0x80 if math.copysign(1, v) < 0 else 0) | idx)
    return np.array(out, dtype=np.uint8).reshape(y.shape)


def _quantize_multiplies(bf16_bits, scale):
    x32 = pa.to_f64(bf16_bits, "bf16").astype(np.float32)
    return pa.fp8_encode((x32 * np.float32(scale)).astype(np.float64))


def _kv_f64_swapped(rows, dtype, scale):
    return pa.fp8_to_f64(rows) / float(scale) if dtype == "fp8" else pa.to_f64(rows, dtype)


@pytest.mark.parametrize("name,target,mutant,checks", [
    ("E4M3 bias 8", "_E4M3_TABLE", _e4m3_table_bias8(),
     ["test_e4m3_decode_table_matches_torch"]),
    ("ties toward zero", "fp8_encode", _encode_ties_toward_zero,
     ["test_e4m3_encode_matches_torch_in_range"]),
    ("scale multiplies", "fp8_quantize", _quantize_multiplies,
     ["test_fp8_append_writes_quantised_rows"]),
    ("scale divides on read", "_kv_f64", _kv_f64_swapped,
     ["test_fp8_decode_is_decode_of_the_dequantised_values"]),
])
def test_planted_fp8_mistakes_are_caught(monkeypatch, name, target, mutant, checks):
    monkeypatch.setattr(pa, target, mutant)
    if target == "fp8_encode":
        monkeypatch.setattr(oracle, "fp8_encode", mutant)
    if target == "fp8_quantize":
        monkeypatch.setattr(oracle, "fp8_quantize", mutant)
    failures = 0
    for check in checks:
        try:
            globals()[check]()
        except AssertionError:
            failures += 1
    assert failures > 0, f"planted mistake '{name}' went unnoticed"
