"""Seeded synthetic decode workloads (the input side shared by tests, bench and oracle).

This module only *makes inputs*: random values, block allocation through a
free-list block manager, block tables, context lengths and slot mappings.  It
computes no attention and imports neither the HIP binding nor the oracle.

Block management follows the pages' description of the engine around the
kernel: a pool of fixed-size blocks held in a free list, where allocation pops
and freeing pushes ("How Paged Attention and Continuous Batching Actually
Work", section "Paged attention: virtual memory for the KV cache"); per-sequence
block tables; reference-counted shared prefix blocks and copy-on-write of a
shared block that one sequence writes ("Paged Attention as a Memory Manager",
section "Prefix Caching and Copy-on-Write"; "LLM paged attention arch", section
"The architecture: every piece explained").  The slot mapping of each new token
is the scheduler's output here, as in the engine step of "How Paged Attention
and Continuous Batching Actually Work", section "One step, end to end".

Storage layout of every pool: ``[num_blocks][num_kv_heads][block_size][head_dim]``;
bf16 values are carried as ``numpy.uint16`` bit patterns, f32 values as
``numpy.float32``.  An 8-bit (``"fp8"``) workload stores E4M3 codes
(``numpy.uint8``) with dequantisation scale ``FP8_SCALE`` for both pools; its
queries and new tokens are bf16.  The codes come from PyTorch's float8_e4m3fn
cast of the scaled draws (a library conversion, not this library's).  Slots a sequence does not own (unallocated blocks, the
unfilled tail of a last block, and this step's new-token slots before the
append) hold NaN, so any read outside the attended range shows up in results.

Every workload is a pure function of its seed.  The five named workloads use
master seed ``9300 + k`` (k = 1..5).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

NAN_F32_BITS = np.uint32(0x7FC00000)
NAN_BF16_BITS = np.uint16(0x7FC0)
NAN_FP8_BITS = np.uint8(0x7F)  # E4M3 NaN
# Dequantisation scale of both pools of the 8-bit workloads: stored codes hold
# N(0,1) draws times 64, well inside E4M3's +-448.
FP8_SCALE = 2.0 ** -6

# Named workloads (the shapes the pages' examples use: Llama-3.1-8B-class and
# Llama-3-70B-class attention head layouts, 16-token blocks).
CONFIGS = {
    1: dict(name="tiny_f32", dtype="f32", num_heads=2, num_kv_heads=1, head_dim=64,
            block_size=16),
    2: dict(name="llama8b_batch64", dtype="bf16", num_heads=32, num_kv_heads=8,
            head_dim=128, block_size=16, num_seqs=64, len_lo=128, len_hi=4096),
    3: dict(name="llama8b_batch256_fragmented", dtype="bf16", num_heads=32,
            num_kv_heads=8, head_dim=128, block_size=16, num_seqs=256,
            lognormal_median=200.0, lognormal_sigma=1.0, len_cap=4096,
            churn_steps=1000),
    4: dict(name="llama70b_shared_prefix_cow", dtype="bf16", num_heads=64,
            num_kv_heads=8, head_dim=128, block_size=16, num_seqs=60,
            prefix_tokens=1008, suffix_lo=1, suffix_hi=1000),
    5: dict(name="llama8b_32k_splitkv", dtype="bf16", num_heads=32, num_kv_heads=8,
            head_dim=128, block_size=16, num_seqs=8, context=32768,
            partition_size=512),
}

# Streams spawned from a master seed, one per independent random quantity.
_STREAMS = ("lengths", "placement", "q", "pool", "new", "divergent", "churn", "extra")


# ---------------------------------------------------------------------------
# Values
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Finite inputs only (the generator draws N(0,1)).  Same rounding as a
    bfloat16 cast of finite float32 values in PyTorch.
    """
    return _round_bf16_inplace(np.array(x, dtype=np.float32, copy=True)).astype(np.uint16)


def _round_bf16_inplace(x: np.ndarray) -> np.ndarray:
    """uint32 view of ``x`` whose low 16 bits hold the rounded bfloat16 (x is clobbered)."""
    u = x.view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    lsb += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bfloat16 bit patterns."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) drawn in float32; bf16 storage rounds each draw once."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def nan_bits(dtype: str):
    return {"f32": NAN_F32_BITS, "bf16": NAN_BF16_BITS, "fp8": NAN_FP8_BITS}[dtype]


def storage_dtype(dtype: str):
    return {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]


def bits_dtype(dtype: str):
    """Unsigned integer type with the storage's width (for writing bit patterns)."""
    return {"f32": np.uint32, "bf16": np.uint16, "fp8": np.uint8}[dtype]


def element_bytes(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "fp8": 1}[dtype]


def query_dtype(dtype: str) -> str:
    """Dtype of q and of the new tokens: bf16 for an 8-bit cache, else the cache's."""
    return "bf16" if dtype == "fp8" else dtype


def fp8_codes(x: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes of float32 draws divided by ``scale`` (PyTorch's cast; |x/scale| <= 448)."""
    import torch

    y = np.clip(np.asarray(x, dtype=np.float32) / np.float32(scale), -448.0, 448.0)
    return torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------------------
# Block manager (host bookkeeping only)
# ---------------------------------------------------------------------------

class BlockPool:
    """LIFO free list of physical block ids with per-block reference counts."""

    def __init__(self, num_blocks: int, order=None):
        self.num_blocks = int(num_blocks)
        ids = list(range(self.num_blocks)) if order is None else [int(b) for b in order]
        if sorted(ids) != list(range(self.num_blocks)):
            raise ValueError("order must be a permutation of the pool")
        # the first pop returns ids[0]
        self.free = ids[::-1]
        self.refcount = np.zeros(self.num_blocks, dtype=np.int32)

    def num_free(self) -> int:
        return len(self.free)

    def alloc(self) -> int:
        if not self.free:
            raise MemoryError("block pool exhausted")
        b = self.free.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def share(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError("sharing a free block")
        self.refcount[b] += 1

    def release(self, b: int) -> None:
        if self.refcount[b] <= 0:
            raise ValueError("releasing a free block")
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.free.append(b)

    def release_all(self, blocks) -> None:
        for b in reversed(list(blocks)):
            self.release(b)


def blocks_for(num_tokens: int, block_size: int) -> int:
    """Number of blocks a sequence of num_tokens tokens occupies."""
    return -(-int(num_tokens) // int(block_size))


def contiguity_ratio(tables, lens, block_size: int) -> float:
    """Fraction of logically adjacent block pairs that are physically adjacent."""
    adjacent = pairs = 0
    for row, n in zip(tables, lens):
        nb = blocks_for(n, block_size)
        for j in range(1, nb):
            pairs += 1
            adjacent += int(row[j]) == int(row[j - 1]) + 1
    return adjacent / pairs if pairs else 1.0


# ---------------------------------------------------------------------------
# Workload container
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    """Inputs of one decode step.

    The step runs, in order: ``copy_pairs`` block copies (copy-on-write), the
    append of ``k_new``/``v_new`` at ``slot_mapping``, then decode attention of
    ``q`` over ``context_lens`` tokens per sequence through ``block_tables``.
    The pools hold the state *before* the step.
    """

    name: str
    seed: int
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    slot_mapping: np.ndarray
    copy_pairs: np.ndarray
    refcount: np.ndarray
    info: dict
    k_scale: float = 1.0  # dequantisation scales of an 8-bit cache
    v_scale: float = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_bytes(self, window: int = 0) -> int:
        """Bytes of K and V that decode must read: sum_i L_i * Hkv * D * 2 * e,
        with L_i capped at ``window`` for a sliding window (0: none)."""
        e = element_bytes(self.dtype)
        lens = self.context_lens.astype(np.int64)
        if window > 0:
            lens = np.minimum(lens, window)
        return int(lens.sum()) * self.num_kv_heads * self.head_dim * 2 * e

    def unique_kv_bytes(self) -> int:
        """K/V bytes of distinct (physical block, row) pairs decode reads."""
        e = element_bytes(self.dtype)
        seen = set()
        rows = 0
        for row, n in zip(self.block_tables, self.context_lens):
            n = int(n)
            for j in range(blocks_for(n, self.block_size)):
                b = int(row[j])
                if b in seen:
                    continue
                seen.add(b)
                rows += min(self.block_size, n - j * self.block_size)
        return rows * self.num_kv_heads * self.head_dim * 2 * e


# ---------------------------------------------------------------------------
# Building a workload from a placement
# ---------------------------------------------------------------------------

def _fill_pools(seed_seq, num_blocks, hkv, bs, d, dtype, chunk_blocks=1024):
    """Two pools of independent N(0,1) values.

    Each chunk of blocks has its own generator spawned from ``seed_seq``, so the
    values do not depend on how many threads draw them.
    """
    from concurrent.futures import ThreadPoolExecutor

    pools = [np.empty((num_blocks, hkv, bs, d), dtype=storage_dtype(dtype)) for _ in range(2)]
    starts = list(range(0, num_blocks, chunk_blocks))
    children = seed_seq.spawn(2 * len(starts))

    def work(job):
        p, c = divmod(job, len(starts))
        b0 = starts[c]
        b1 = min(num_blocks, b0 + chunk_blocks)
        rng = np.random.default_rng(children[job])
        x = rng.standard_normal(size=(b1 - b0, hkv, bs, d), dtype=np.float32)
        if dtype == "fp8":
            pools[p][b0:b1] = fp8_codes(x, FP8_SCALE)
        else:
            pools[p][b0:b1] = x if dtype == "f32" else _round_bf16_inplace(x)

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(work, range(2 * len(starts))))
    return pools


def _assemble(name, seed, cfg, dtype, streams, num_blocks, seq_blocks, lens,
              max_blocks, refcount, extra_writes=(), copy_pairs=(), info=None):
    """Draw values, poison everything outside the owned rows, emit the step.

    ``seq_blocks[i]`` lists sequence i's physical blocks in logical order
    (after any copy-on-write remap); ``lens[i]`` includes this step's token,
    which the append writes at row (lens[i]-1) of the sequence.
    ``extra_writes`` are additional (physical block, row) writes of this step,
    each with its own new K/V (the copy-on-write divergence).
    """
    hq, hkv, d, bs = cfg["num_heads"], cfg["num_kv_heads"], cfg["head_dim"], cfg["block_size"]
    num_seqs = len(lens)
    k_pool, v_pool = _fill_pools(streams["pool_seq"], num_blocks, hkv, bs, d, dtype)
    poison = nan_bits(dtype)

    owned_rows = np.zeros((num_blocks, bs), dtype=bool)
    for blocks, n in zip(seq_blocks, lens):
        for j, b in enumerate(blocks):
            owned_rows[b, : min(bs, int(n) - j * bs)] = True
    # a copy source must hold real rows wherever its copy will be read
    for src, dst in copy_pairs:
        owned_rows[src] |= owned_rows[dst]

    # New-token rows: physical (block, row) of position lens[i]-1 of each sequence.
    writes = []
    for blocks, n in zip(seq_blocks, lens):
        last = int(n) - 1
        writes.append((blocks[last // bs], last - (last // bs) * bs))
    writes.extend(extra_writes)
    slot_mapping = np.array([b * bs + r for b, r in writes], dtype=np.int64)
    if len(set(slot_mapping.tolist())) != len(slot_mapping):
        raise AssertionError("generator produced a repeated slot")

    # Poison: unowned rows, plus the rows this step writes (before the append).
    dead = ~owned_rows
    for b, r in writes:
        dead[b, r] = True
    # copy destinations are written by the copy step; before it they hold poison
    for _src, dst in copy_pairs:
        dead[dst, :] = True
    bidx, ridx = np.nonzero(dead)
    for pool in (k_pool, v_pool):
        pool.view(bits_dtype(dtype))[bidx, :, ridx, :] = poison

    qdt = query_dtype(dtype)
    q = draw_values(streams["q"], (num_seqs, hq, d), qdt)
    k_new = draw_values(streams["new"], (len(writes), hkv, d), qdt)
    v_new = draw_values(streams["new"], (len(writes), hkv, d), qdt)

    # Table rows past a sequence's last block point at a poisoned block when one
    # exists, so reading them would show up as NaN in the output.
    unowned = np.nonzero(~owned_rows.any(axis=1))[0]
    filler = int(unowned[0]) if len(unowned) else 0
    tables = np.full((num_seqs, max_blocks), filler, dtype=np.int32)
    for i, blocks in enumerate(seq_blocks):
        tables[i, : len(blocks)] = blocks

    scale = FP8_SCALE if dtype == "fp8" else 1.0
    return Workload(
        name=name, seed=seed, dtype=dtype, k_scale=scale, v_scale=scale,
        num_heads=hq, num_kv_heads=hkv,
        head_dim=d, block_size=bs, q=q, k_pool=k_pool, v_pool=v_pool,
        block_tables=tables, context_lens=np.asarray(lens, dtype=np.int32),
        k_new=k_new, v_new=v_new, slot_mapping=slot_mapping,
        copy_pairs=np.asarray(list(copy_pairs), dtype=np.int64).reshape(-1, 2),
        refcount=refcount, info=dict(info or {}))


def _streams(seed: int):
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    streams = {k: np.random.default_rng(c) for k, c in zip(_STREAMS, children)}
    streams["pool_seq"] = children[_STREAMS.index("pool")]
    return streams


def _scatter_placement(rng, lens, bs, slack=1.25, extra_blocks=0, num_blocks=None):
    """Pool of ceil(slack * need) blocks, assigned by a seeded shuffle in logical order."""
    need = sum(blocks_for(n, bs) for n in lens)
    if num_blocks is None:
        num_blocks = int(math.ceil(slack * need)) + extra_blocks
    order = rng.permutation(num_blocks)
    pool = BlockPool(num_blocks, order)
    seq_blocks = [[pool.alloc() for _ in range(blocks_for(n, bs))] for n in lens]
    return num_blocks, pool, seq_blocks


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------

def make_config(k: int, dtype: str | None = None, block_size: int | None = None,
                num_seqs: int | None = None, context: int | None = None,
                head_dim: int | None = None) -> Workload:
    """Workload k (1..5) with master seed 9300 + k.

    ``dtype``/``block_size``/``num_seqs``/``context``/``head_dim`` override the
    named shape (same seed), e.g. float32 copies of the bf16 shapes, block size
    32 for workload 5, 64-dim heads, or fewer sequences for quick tests.
    """
    cfg = dict(CONFIGS[k])
    seed = 9300 + k
    if block_size is not None:
        cfg["block_size"] = int(block_size)
    if head_dim is not None:
        cfg["head_dim"] = int(head_dim)
    dt = dtype or cfg["dtype"]
    s = _streams(seed)
    bs = cfg["block_size"]
    name = cfg["name"] + ("" if dt == cfg["dtype"] else f"_{dt}") + (
        "" if block_size in (None, CONFIGS[k]["block_size"]) else f"_bs{bs}") + (
        "" if head_dim in (None, CONFIGS[k]["head_dim"]) else f"_d{cfg['head_dim']}")

    if k == 1:
        lens = [5, 37]
        num_blocks = 8
        order = s["placement"].permutation(num_blocks)
        pool = BlockPool(num_blocks, order)
        seq_blocks = [[pool.alloc() for _ in range(blocks_for(n, bs))] for n in lens]
        return _assemble(name, seed, cfg, dt, s, num_blocks, seq_blocks, lens,
                         max_blocks=blocks_for(max(lens), bs), refcount=pool.refcount,
                         info=dict(pool_order=order.tolist()))

    if k == 2:
        n = num_seqs or cfg["num_seqs"]
        lens = s["lengths"].integers(cfg["len_lo"], cfg["len_hi"] + 1, size=cfg["num_seqs"])[:n]
        if context is not None:
            lens = np.minimum(lens, context)
        lens = [int(x) for x in lens]
        num_blocks, pool, seq_blocks = _scatter_placement(s["placement"], lens, bs)
        return _assemble(name, seed, cfg, dt, s, num_blocks, seq_blocks, lens,
                         max_blocks=blocks_for(cfg["len_hi"], bs), refcount=pool.refcount)

    if k == 3:
        return _fragmented(cfg, seed, s, dt, name, num_seqs or cfg["num_seqs"])

    if k == 4:
        return _shared_prefix(cfg, seed, s, dt, name, num_seqs or cfg["num_seqs"])

    if k == 5:
        n = num_seqs or cfg["num_seqs"]
        ctx = context or cfg["context"]
        lens = [ctx] * n
        num_blocks, pool, seq_blocks = _scatter_placement(s["placement"], lens, bs)
        return _assemble(name, seed, cfg, dt, s, num_blocks, seq_blocks, lens,
                         max_blocks=blocks_for(ctx, bs), refcount=pool.refcount,
                         info=dict(partition_size=cfg["partition_size"]))
    raise ValueError(f"no workload {k}")


def lognormal_lengths(rng, n, median, sigma, cap):
    z = rng.standard_normal(n)
    return [int(min(cap, max(1, round(median * math.exp(sigma * float(v)))))) for v in z]


def _fragmented(cfg, seed, s, dt, name, num_seqs):
    """Batch of log-normal lengths placed after a continuous-batching churn.

    The pool (ceil(1.25 * need) blocks, LIFO free list) first serves
    ``churn_steps`` simulated engine steps: up to ``num_seqs`` running
    sequences each gain one token per step, taking a block at every block
    boundary; finished sequences return their blocks; arrivals refill the batch
    while blocks last; when a running sequence needs a block and none is free,
    the latest-arrived sequence is preempted and returns its blocks.  After the
    last step every simulated sequence is released in a seeded order, and the
    measured batch then takes its blocks from the fragmented free list.
    """
    bs = cfg["block_size"]
    med, sig, cap = cfg["lognormal_median"], cfg["lognormal_sigma"], cfg["len_cap"]
    lens = lognormal_lengths(s["lengths"], num_seqs, med, sig, cap)
    need = sum(blocks_for(n, bs) for n in lens)
    num_blocks = int(math.ceil(1.25 * need))
    pool = BlockPool(num_blocks)
    rng = s["churn"]
    running = []  # arrival order; dicts with target, length, blocks, alive
    preemptions = finished = 0

    def preempt(seq):
        nonlocal preemptions
        seq["alive"] = False
        running.remove(seq)
        pool.release_all(seq["blocks"])
        preemptions += 1

    for _step in range(cfg["churn_steps"]):
        # admit arrivals while the batch has room and blocks last
        while len(running) < num_seqs:
            target = lognormal_lengths(rng, 1, med, sig, cap)[0]
            start = int(rng.integers(1, target + 1))
            nb = blocks_for(start, bs)
            if nb > pool.num_free():
                break
            running.append(dict(target=target, length=start, alive=True,
                                blocks=[pool.alloc() for _ in range(nb)]))
        # every running sequence gains one token
        for seq in list(running):
            if not seq["alive"]:
                continue
            seq["length"] += 1
            if seq["length"] <= len(seq["blocks"]) * bs:
                continue
            while pool.num_free() == 0 and running[-1] is not seq:
                preempt(running[-1])
            if pool.num_free() == 0:
                preempt(seq)
                continue
            seq["blocks"].append(pool.alloc())
        # finished sequences return their blocks
        for seq in list(running):
            if seq["length"] >= seq["target"]:
                running.remove(seq)
                pool.release_all(seq["blocks"])
                finished += 1
    for j in rng.permutation(len(running)):
        pool.release_all(running[int(j)]["blocks"])
    assert pool.num_free() == num_blocks
    seq_blocks = [[pool.alloc() for _ in range(blocks_for(n, bs))] for n in lens]
    tables_for_ratio = [list(b) for b in seq_blocks]
    info = dict(preemptions=preemptions, finished=finished,
                contiguity=contiguity_ratio(tables_for_ratio, lens, bs))
    return _assemble(name, seed, cfg, dt, s, num_blocks, seq_blocks, lens,
                     max_blocks=max(blocks_for(n, bs) for n in lens), refcount=pool.refcount,
                     info=info)


def _shared_prefix(cfg, seed, s, dt, name, num_seqs):
    """Shared system prefix (refcounted blocks) plus private suffixes, with one COW.

    Every sequence's first prefix_tokens / B logical blocks point at the same
    physical blocks (refcount = number of sequences).  One seeded sequence d
    diverges at the last prefix position: before its write, the block manager
    takes a fresh block, schedules a copy of the shared block into it, points
    d's table entry at the copy and drops the shared block's refcount by one;
    the append then writes d's new K/V for that position into the copy.
    """
    bs = cfg["block_size"]
    prefix = cfg["prefix_tokens"]
    if prefix % bs:
        raise ValueError("prefix must fill whole blocks")
    n_prefix_blocks = prefix // bs
    suffix = [int(x) for x in s["lengths"].integers(cfg["suffix_lo"], cfg["suffix_hi"] + 1,
                                                     size=cfg["num_seqs"])[:num_seqs]]
    lens = [prefix + x for x in suffix]
    need = n_prefix_blocks + sum(blocks_for(x, bs) for x in suffix)
    num_blocks = int(math.ceil(1.25 * need)) + 1
    order = s["placement"].permutation(num_blocks)
    pool = BlockPool(num_blocks, order)
    shared = [pool.alloc() for _ in range(n_prefix_blocks)]
    for b in shared:
        for _ in range(num_seqs - 1):
            pool.share(b)
    seq_blocks = [list(shared) + [pool.alloc() for _ in range(blocks_for(x, bs))] for x in suffix]
    d = int(s["divergent"].integers(0, num_seqs))
    src = shared[-1]
    dst = pool.alloc()
    pool.release(src)
    seq_blocks[d][n_prefix_blocks - 1] = dst
    # d's rewrite of its last prefix position lands in the copy
    extra = [(dst, (prefix - 1) - (n_prefix_blocks - 1) * bs)]
    info = dict(divergent_seq=d, cow_src=src, cow_dst=dst, shared_blocks=shared)
    return _assemble(name, seed, cfg, dt, s, num_blocks, seq_blocks, lens,
                     max_blocks=blocks_for(prefix + cfg["suffix_hi"], bs), refcount=pool.refcount,
                     extra_writes=extra, copy_pairs=[(src, dst)], info=info)


def small_random(seed: int, *, dtype="f32", num_seqs=3, num_heads=4, num_kv_heads=2,
                 head_dim=64, block_size=16, len_lo=1, len_hi=100, slack=1.5,
                 lens=None) -> Workload:
    """Small scattered workload for quick parity cases (ragged lengths)."""
    cfg = dict(num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
               block_size=block_size)
    s = _streams(seed)
    if lens is None:
        lens = [int(x) for x in s["lengths"].integers(len_lo, len_hi + 1, size=num_seqs)]
    num_blocks, pool, seq_blocks = _scatter_placement(s["placement"], lens, block_size,
                                                      slack=slack, extra_blocks=1)
    return _assemble(f"small_{seed}", seed, cfg, dtype, s, num_blocks, seq_blocks, lens,
                     max_blocks=max(1, max(blocks_for(n, block_size) for n in lens)),
                     refcount=pool.refcount)


def random_partials(seed: int, num_seqs: int, num_heads: int, head_dim: int,
                    max_parts: int, context_lens, partition_size: int):
    """Synthetic split-KV partials: per (seq, head, partition) an output row,
    a running max and a positive weight sum; partitions past a sequence's
    last are filled with NaN (they must not be read)."""
    s = _streams(seed)
    rng = s["extra"]
    out = rng.standard_normal((num_seqs, num_heads, max_parts, head_dim), dtype=np.float32)
    mx = (rng.standard_normal((num_seqs, num_heads, max_parts)) * 4.0).astype(np.float32)
    sm = rng.uniform(0.5, 64.0, size=(num_seqs, num_heads, max_parts)).astype(np.float32)
    for i, n in enumerate(context_lens):
        live = blocks_for(int(n), partition_size)
        out[i, :, live:] = np.nan
        mx[i, :, live:] = np.nan
        sm[i, :, live:] = np.nan
    return out, mx, sm


# ---------------------------------------------------------------------------
# Mixed-batch (prefill) workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillWorkload:
    """Inputs of one mixed-batch attention call (pa_prefill).

    Sequence i owns query rows ``query_start[i] .. query_start[i+1]-1`` of ``q``
    (its last n_i positions); its ``context_lens[i]`` rows are in the pools
    already (this step's writes included).  Everything outside the owned rows
    is NaN, and table entries past a sequence's last block point at a poisoned
    block.
    """

    name: str
    seed: int
    dtype: str
    k_scale: float
    v_scale: float
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    q: np.ndarray              # [num_tokens][num_heads][head_dim], bf16 bits
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_tables: np.ndarray   # int32 [num_seqs][max_blocks]
    query_start: np.ndarray    # int32 [num_seqs + 1]
    context_lens: np.ndarray   # int32 [num_seqs]

    @property
    def num_seqs(self) -> int:
        return len(self.context_lens)

    @property
    def num_tokens(self) -> int:
        return int(self.query_start[-1])

    def flops(self, window: int = 0) -> int:
        """Algorithmic flops: 4 * head_dim per (query row, head, visible key);
        a query at position p sees p + 1 keys, or min(p + 1, window) with a window."""
        total = 0
        for i in range(self.num_seqs):
            n, L = int(self.query_start[i + 1] - self.query_start[i]), int(self.context_lens[i])
            seen = np.arange(L - n + 1, L + 1, dtype=np.int64)   # keys seen by each query token
            if window:
                seen = np.minimum(seen, window)
            total += int(seen.sum())
        return 4 * self.head_dim * self.num_heads * total


def prefill_batch(name: str, seed: int, lens, nq, num_heads: int = 32, num_kv_heads: int = 8,
                  head_dim: int = 128, block_size: int = 16, dtype: str = "bf16",
                  zero_query: bool = False, slack: float = 1.1) -> PrefillWorkload:
    """A mixed batch: sequence i has context lens[i] and nq[i] query tokens."""
    lens = [int(x) for x in lens]
    nq = [int(x) for x in nq]
    if len(lens) != len(nq) or any(n < 0 or n > L for n, L in zip(nq, lens)):
        raise ValueError("need 0 <= nq[i] <= lens[i]")
    streams = _streams(seed)
    num_blocks, _pool, seq_blocks = _scatter_placement(streams["placement"], lens, block_size,
                                                       slack=slack, extra_blocks=1)
    k_pool, v_pool = _fill_pools(streams["pool_seq"], num_blocks, num_kv_heads, block_size,
                                 head_dim, dtype)
    owned = np.zeros((num_blocks, block_size), dtype=bool)
    for blocks, n in zip(seq_blocks, lens):
        for j, b in enumerate(blocks):
            owned[b, : min(block_size, n - j * block_size)] = True
    bidx, ridx = np.nonzero(~owned)
    for pool in (k_pool, v_pool):
        pool.view(bits_dtype(dtype))[bidx, :, ridx, :] = nan_bits(dtype)
    unowned = np.nonzero(~owned.any(axis=1))[0]
    filler = int(unowned[0]) if len(unowned) else 0
    width = max(blocks_for(n, block_size) for n in lens) + 1
    tables = np.full((len(lens), width), filler, dtype=np.int32)
    for i, blocks in enumerate(seq_blocks):
        tables[i, : len(blocks)] = blocks
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    qdt = query_dtype(dtype)
    q = draw_values(streams["q"], (int(qs[-1]), num_heads, head_dim), qdt)
    if zero_query:
        q = np.zeros_like(q)
    scale = FP8_SCALE if dtype == "fp8" else 1.0
    return PrefillWorkload(name=name, seed=seed, dtype=dtype, k_scale=scale, v_scale=scale,
                           num_heads=num_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
                           block_size=block_size, q=q, k_pool=k_pool, v_pool=v_pool,
                           block_tables=tables, query_start=qs,
                           context_lens=np.asarray(lens, dtype=np.int32))


def prefill_config(name: str, dtype: str = "bf16", block_size: int = 16) -> PrefillWorkload:
    """Named mixed-batch workloads at the 8B-class head layout (32 / 8 heads, dim 128).

    * ``cached_preamble``: 16 requests of 1,200-token prompts whose first 896
      tokens (56 blocks) are already cached, so 304 tokens each are computed -
      the worked example of "LLM paged attention arch", section "End-to-end
      flow", sixteen times (seed 9311);
    * ``long_prompts``: 4 prompts of 4,096 tokens computed from scratch (9312);
    * ``mixed_step``: a chunked-prefill step under an 8,192-token budget - 60
      decodes with contexts U{128..4096}, one 2,048-token slice of a prompt
      whose first 2,048 tokens were computed in an earlier step, and one
      1,024-token prompt from scratch (9313).
    """
    if name == "cached_preamble":
        return prefill_batch(name, 9311, [1200] * 16, [304] * 16, dtype=dtype,
                             block_size=block_size)
    if name == "long_prompts":
        return prefill_batch(name, 9312, [4096] * 4, [4096] * 4, dtype=dtype,
                             block_size=block_size)
    if name == "mixed_step":
        rng = np.random.default_rng(9313)
        lens = [int(x) for x in rng.integers(128, 4097, 60)] + [4096, 1024]
        nq = [1] * 60 + [2048, 1024]
        return prefill_batch(name, 9313, lens, nq, dtype=dtype, block_size=block_size)
    raise ValueError(f"unknown prefill workload {name!r}")
