"""Pins of the block-manager oracle (``oracle/block_manager.py``).

Nothing on the pages prints a block table, so the oracle is pinned by:

* the scenarios the pages work through with numbers (``golden/block_manager_cases.json``):
  a prompt of 1,200 tokens of which a 900-token preamble is cached (75 blocks,
  56 shared, 19 new, ~300 tokens to prefill), 100 conversations sharing one
  5,000-token prompt (313 blocks, 160 GB against 1.6 GB), a 17-token sequence
  (2 blocks, ~53 % used), ceil(t/16) blocks for t tokens;
* the behaviour the pages state in words: copy-on-write takes a fresh block,
  copies, re-points one table and drops one reference; the youngest request is
  preempted when the pool runs dry and shared blocks only lose a reference; a
  preempted request is recomputed (or swapped back) when blocks free up; a
  finished request's blocks serve the very next step; admission keeps a margin;
  long prompts are fed in budget-sized slices after the running decodes;
* brute force on random traces: a content model replays every plan's copies
  and writes on arrays of prefix identities, and every request must read its
  own token prefixes back through its table, every cached block must hold the
  prefix its key names, and no write may land in a shared block;
* planted mistakes, each of which one of the above must catch.
"""

from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np
import pytest

from bm_trace import ContentModel, Trace
from oracle import blocks_needed
from oracle.block_manager import (RECOMPUTE, RUNNING, SWAP, SWAPPED, WAITING, BlockManager)

GOLDEN = json.loads((Path(__file__).parent / "golden" / "block_manager_cases.json").read_text())


# ---------------------------------------------------------------------------
# invariants and the checked trace runner
# ---------------------------------------------------------------------------

def check_invariants(m: BlockManager) -> None:
    holders = [0] * m.num_gpu_blocks
    cpu_held = []
    for r in m.requests.values():
        assert len(set(r.blocks)) == len(r.blocks), "a block twice in one table"
        for b in r.blocks:
            holders[b] += 1
        if r.state == RUNNING:
            assert len(r.blocks) == blocks_needed(r.computed, m.B) and not r.cpu_blocks
        elif r.state == SWAPPED:
            assert not r.blocks and len(r.cpu_blocks) == blocks_needed(r.computed, m.B)
            cpu_held += r.cpu_blocks
        else:
            assert r.state == WAITING and not r.blocks and not r.cpu_blocks and r.computed == 0
    assert holders == m.refcount, "reference counts differ from the tables"
    assert len(set(m.free)) == len(m.free)
    assert set(m.free) == {b for b in range(m.num_gpu_blocks) if m.refcount[b] == 0}
    assert sorted(m.cpu_free + cpu_held) == list(range(m.num_cpu_blocks))
    assert {b: k for k, b in m.cache.items()} == m.block_key


def holders(m: BlockManager) -> dict:
    out = {}
    for r in m.requests.values():
        for b in r.blocks:
            out.setdefault(b, set()).add(r.rid)
    return out


def check_content(m: BlockManager, cm: ContentModel, plan, tokens_at, held_before) -> None:
    """``held_before``: block -> requests holding it before the step."""
    B = m.B
    held_now = holders(m)
    for k, rid in enumerate(plan.seq_ids):
        L = plan.context_lens[k]
        assert cm.read(plan.block_tables[k], L) == cm.expected(tokens_at[rid], L), \
            f"request {rid} reads a wrong prefix through its plan table"
        for s in plan.slot_mapping[plan.query_start[k]:plan.query_start[k + 1]]:
            b = s // B
            still = held_before.get(b, set()) & held_now.get(b, set())
            assert still <= {rid}, "a write landed in a block shared before the step"
    for r in m.requests.values():
        if r.state == RUNNING:
            assert cm.read(r.blocks, r.computed) == cm.expected(r.tokens, r.computed), \
                f"running request {r.rid} lost its KV"
        elif r.state == SWAPPED:
            assert cm.read(r.cpu_blocks, r.computed, cpu=True) == cm.expected(r.tokens, r.computed), \
                f"swapped request {r.rid} lost its KV"
    for key, b in m.cache.items():
        got = [int(x) for x in cm.gpu[b]]
        want = [cm.ids.of(key, len(key) - B + i) for i in range(B)]
        assert got == want, f"cached block {b} does not hold the prefix of its key"


TRACE_SETTINGS = [
    # (gpu blocks, cpu blocks, block size, prefix caching, preempt mode, watermark, vocab, fork prob)
    (24, 16, 4, True, RECOMPUTE, 0, 3, 0.1),
    (24, 16, 4, True, SWAP, 0, 3, 0.1),
    (12, 6, 2, True, SWAP, 1, 2, 0.2),
    (40, 40, 8, False, SWAP, 0, 4, 0.05),
    (16, 0, 1, True, SWAP, 0, 2, 0.15),
    (30, 10, 16, True, RECOMPUTE, 2, 3, 0.1),
]


def run_checked(factory, seed: int, setting, steps: int = 60) -> dict:
    g, c, B, pc, mode, wm, vocab, fork = setting
    m = factory(g, c, B, prefix_caching=pc, preempt_mode=mode, watermark_blocks=wm)
    trace = Trace(seed, g, c, B, vocab=vocab, fork_prob=fork, watermark=wm)
    cm = ContentModel(g, c, B)
    seen = dict(preempt=0, swap=0, cow=0, hits=0)

    held, waiting = {}, set()

    def check(plans):
        plan, = plans
        cm.apply(plan, trace.tokens_at_schedule.__getitem__)
        check_content(m, cm, plan, trace.tokens_at_schedule, held)
        check_invariants(m)
        seen["preempt"] += len(plan.preempted)
        seen["swap"] += len(plan.swap_out) + len(plan.swap_in)
        seen["cow"] += len(plan.cow_pairs)
        for k, rid in enumerate(plan.seq_ids):
            n = plan.query_start[k + 1] - plan.query_start[k]
            if rid in waiting and plan.context_lens[k] > n:
                seen["hits"] += 1          # admitted with a cached prefix

    for _ in range(steps):
        held = holders(m)
        waiting = {r.rid for r in m.requests.values() if r.state == WAITING}
        trace.step([m], on_plans=check)
        check_invariants(m)
    return seen


# ---------------------------------------------------------------------------
# scenarios with numbers on the pages
# ---------------------------------------------------------------------------

def test_prefix_cache_worked_example():
    g = GOLDEN["prefix_hit"]
    B = g["block_size"]
    rng = np.random.default_rng(93)
    preamble = [int(t) for t in rng.integers(0, 32000, g["preamble_tokens"])]
    m = BlockManager(200, 0, B)
    m.add_request(0, preamble + [int(t) for t in rng.integers(0, 32000, 100)])
    m.schedule(4096)
    m.add_request(1, preamble + [int(t) for t in rng.integers(0, 32000, g["prompt_tokens"] - g["preamble_tokens"])])
    plan = m.schedule(4096)
    assert plan.seq_ids == [1]
    table = plan.block_tables[0]
    n = plan.query_start[1]
    cached = plan.context_lens[0] - n
    assert plan.context_lens[0] == g["prompt_tokens"] and len(table) == g["blocks"]
    assert cached == g["cached_blocks"] * B
    assert table[:g["cached_blocks"]] == m.table(0)[:g["cached_blocks"]]
    assert all(m.refcount[b] == 2 for b in table[:g["cached_blocks"]])
    fresh = table[g["cached_blocks"]:]
    assert len(fresh) == g["new_blocks"] and not set(fresh) & set(m.table(0))
    assert abs(n - g["prefill_tokens_about"]) < B
    st = m.stats()
    assert st["prefix_hit_tokens"] == cached and st["admitted_tokens"] == 1000 + g["prompt_tokens"]
    # the 1,201st token is the first one of the 76th block
    m.append_token(1, 7)
    plan = m.schedule(4096)
    assert plan.seq_ids == [1] and len(plan.block_tables[0]) == g["blocks"] + 1
    assert plan.slot_mapping == [plan.block_tables[0][g["blocks"]] * B]
    # on completion the private blocks return, the shared ones lose a reference,
    # and the preamble stays warm for the next request
    shared = table[:g["cached_blocks"]]
    m.finish(1)
    assert all(m.refcount[b] == 1 for b in shared)
    m.finish(0)
    assert all(m.refcount[b] == 0 for b in shared)
    m.add_request(2, preamble + [5] * 40)
    plan = m.schedule(4096)
    assert plan.block_tables[0][:g["cached_blocks"]] == shared
    check_invariants(m)


def test_blocks_held_are_ceil_of_tokens():
    B = 16
    m = BlockManager(64, 0, B, prefix_caching=False)
    m.add_request(0, [3])
    for t in range(1, 400):
        m.schedule(1)
        assert len(m.table(0)) == math.ceil(t / 16)
        assert len(m.table(0)) * B - t <= 15
        m.append_token(0, t % 5)
    g = GOLDEN["sequence_17"]
    m = BlockManager(8, 0, g["block_size"])
    m.add_request(0, list(range(g["tokens"])))
    plan = m.schedule(100)
    assert len(plan.block_tables[0]) == g["blocks"]
    assert round(100 * g["tokens"] / (g["blocks"] * g["block_size"])) == g["utilisation_percent"]


def test_fork_shares_every_block_then_copies_on_write():
    g = GOLDEN["fork_share"]
    B, n_conv = g["block_size"], g["conversations"]
    m = BlockManager(g["shared_blocks"] + 2 * n_conv, 0, B, prefix_caching=False)
    m.add_request(0, [int(t) for t in np.random.default_rng(5).integers(0, 32000, g["prompt_tokens"])])
    m.schedule(g["prompt_tokens"])
    for child in range(1, n_conv):
        m.fork(0, child)
    table = m.table(0)
    assert len(table) == g["shared_blocks"]
    assert all(m.table(c) == table for c in range(n_conv))
    assert all(m.refcount[b] == n_conv for b in table)
    block_bytes = B * g["kb_per_token"] * 1e3
    assert len({b for c in range(n_conv) for b in m.table(c)}) * block_bytes / 1e9 == \
        pytest.approx(g["shared_gb"], rel=0.01)
    assert n_conv * g["prompt_tokens"] * g["kb_per_token"] * 1e3 / 1e9 == pytest.approx(g["separate_gb"])
    # every conversation diverges: each writer but the last copies the shared partial block
    for c in range(n_conv):
        m.append_token(c, 1000 + c)
    plan = m.schedule(4 * n_conv)
    last = table[-1]
    assert g["prompt_tokens"] % B != 0
    assert len(plan.cow_pairs) == n_conv - 1
    assert all(src == last for src, _ in plan.cow_pairs)
    assert len({dst for _, dst in plan.cow_pairs}) == n_conv - 1
    assert m.refcount[last] == 1 and m.table(n_conv - 1)[-1] == last
    assert m.stats()["cow_copies"] == n_conv - 1
    check_invariants(m)


def test_copy_on_write_steps():
    """Fresh block, copy, one table re-pointed, one reference dropped."""
    m = BlockManager(16, 0, 4, prefix_caching=False)
    m.add_request(0, [1, 2, 3, 4, 5, 6])          # block 1 holds positions 4, 5
    m.schedule(64)
    m.fork(0, 1)
    old = m.table(0)[1]
    assert m.refcount[old] == 2
    first_free = m.free[0]
    m.append_token(0, 7)
    m.append_token(1, 8)
    plan = m.schedule(64)
    assert plan.cow_pairs == [(old, first_free)]
    assert m.table(0) == [m.table(1)[0], first_free] and m.table(1)[1] == old
    assert m.refcount[old] == 1 and m.refcount[first_free] == 1
    assert plan.slot_mapping == [first_free * 4 + 2, old * 4 + 2]


def _three_sharing_requests(mode: str, cpu_blocks: int, cls=BlockManager):
    """Three requests share a one-block preamble and grow until the pool runs dry."""
    m = cls(7, cpu_blocks, 4, preempt_mode=mode)
    pre = [9, 9, 9, 9]
    for rid, tail in enumerate([[1], [2, 2], [3, 3, 3]]):
        m.add_request(rid, pre + tail)
    plan = m.schedule(64)
    assert plan.seq_ids == [0, 1, 2]
    shared = m.table(0)[0]
    assert m.table(1)[0] == shared == m.table(2)[0]
    for step in range(40):
        for rid in list(m.requests):
            if m.requests[rid].state == RUNNING:
                m.append_token(rid, step % 4)
        before = {rid: list(r.blocks) for rid, r in m.requests.items()}
        plan = m.schedule(64)
        if plan.preempted:
            return m, plan, shared, before
    raise AssertionError("the pool never ran dry")


def _check_youngest_preempted(cls):
    m, plan, shared, before = _three_sharing_requests(RECOMPUTE, 0, cls)
    assert plan.preempted == [(2, RECOMPUTE)]
    return m, plan, shared, before


def test_preemption_takes_the_youngest_and_shared_blocks_lose_a_reference():
    m, plan, shared, before = _check_youngest_preempted(BlockManager)
    assert plan.seq_ids == [0, 1]               # the older requests keep decoding
    assert m.requests[2].state == WAITING and m.requests[2].computed == 0
    assert m.refcount[shared] == 2 and shared not in m.free
    private = [b for b in before[2] if b != shared]
    assert all(m.refcount[b] == 0 or any(b in t for t in plan.block_tables) for b in private)
    # the victim is recomputed once blocks free up
    m.finish(0)
    plan = m.schedule(64)
    assert plan.seq_ids[-1] == 2
    r = m.requests[2]
    assert plan.context_lens[-1] == len(r.tokens) == r.computed
    assert plan.block_tables[-1][0] == shared  # the preamble is taken from the cache
    check_invariants(m)


def test_swap_out_and_back_in():
    m, plan, shared, before = _three_sharing_requests(SWAP, 8)
    assert plan.preempted == [(2, SWAP)]
    assert [g for g, _ in plan.swap_out] == before[2]
    cpu = [c for _, c in plan.swap_out]
    assert m.requests[2].state == SWAPPED and m.requests[2].cpu_blocks == cpu
    assert m.refcount[shared] == 2
    m.finish(0)
    plan = m.schedule(64)
    assert [c for c, _ in plan.swap_in] == cpu
    assert m.requests[2].state == RUNNING
    assert m.table(2)[:len(cpu)] == [g for _, g in plan.swap_in]
    assert sorted(m.cpu_free) == list(range(8))
    check_invariants(m)


def test_swap_falls_back_to_recompute_without_cpu_blocks():
    m, plan, _, before = _three_sharing_requests(SWAP, 1)
    assert plan.preempted == [(2, RECOMPUTE)] and not plan.swap_out


def test_finished_request_frees_blocks_for_the_next_step():
    m = BlockManager(4, 0, 4, prefix_caching=False)
    m.add_request(0, list(range(16)))            # all four blocks
    m.add_request(1, [1, 2, 3])
    plan = m.schedule(64)
    assert plan.seq_ids == [0] and m.requests[1].state == WAITING
    m.finish(0)
    plan = m.schedule(64)
    assert plan.seq_ids == [1]


def _copy_source_freed_in_its_step(cls):
    """R0 copies its shared block X; the pool is then dry for C's copy, and the
    victim R1 drops the last other reference to X."""
    m = cls(5, 0, 4, prefix_caching=False)
    m.add_request(0, [1, 2, 3, 4, 5, 6])         # R0: b0, X
    m.add_request(1, [7, 8, 9, 10, 11, 12])      # C: c0, Y
    m.schedule(64)
    x, y = m.table(0)[1], m.table(1)[1]
    m.fork(1, 2)                                 # D shares C's blocks
    m.fork(0, 3)                                 # R1 shares R0's blocks, latest arrival
    for rid in range(4):
        m.append_token(rid, 20 + rid)
    plan = m.schedule(64)
    srcs = {a for a, _ in plan.cow_pairs}
    assert not srcs & {b for _, b in plan.cow_pairs}, "a copy source reused as a copy destination"
    return m, plan, x, y


def test_copy_source_freed_in_its_step_waits_for_the_step_end():
    m, plan, x, y = _copy_source_freed_in_its_step(BlockManager)
    assert plan.preempted == [(3, RECOMPUTE), (2, RECOMPUTE)]
    assert [a for a, _ in plan.cow_pairs] == [x] and plan.seq_ids == [0, 1]
    assert m.free[-1] == x                       # rejoined the queue at the step end
    check_invariants(m)


def test_reusing_a_copy_source_at_once_is_caught():
    with pytest.raises(AssertionError):
        _copy_source_freed_in_its_step(_ReuseCopySourceAtOnce)


def test_admission_keeps_a_margin():
    m = BlockManager(10, 0, 4, prefix_caching=False, watermark_blocks=2)
    m.add_request(0, list(range(24)))            # 6 blocks, 4 left >= 2
    m.add_request(1, list(range(12)))            # 3 more would leave 1 < 2
    plan = m.schedule(100)
    assert plan.seq_ids == [0] and m.requests[1].state == WAITING
    m2 = BlockManager(10, 0, 4, prefix_caching=False, watermark_blocks=1)
    m2.add_request(0, list(range(24)))
    m2.add_request(1, list(range(12)))
    assert m2.schedule(100).seq_ids == [0, 1]


def test_decodes_first_then_prompt_slices_within_the_budget():
    m = BlockManager(32, 0, 4, prefix_caching=False)
    m.add_request(0, [1, 2, 3])
    m.schedule(10)
    m.append_token(0, 4)
    m.add_request(1, list(range(25)))
    sizes = []
    for _ in range(3):
        plan = m.schedule(10)
        assert plan.seq_ids[0] == 0 and plan.query_start[1] == 1   # the decode goes first
        sizes.append(plan.query_start[2] - plan.query_start[1])
        m.append_token(0, 5)
    assert sizes == [9, 9, 7]
    assert m.requests[1].computed == 25


def test_admitted_prompt_always_computes_its_last_token():
    m = BlockManager(16, 0, 4)
    m.add_request(0, [1] * 8)
    m.schedule(64)
    m.add_request(1, [1] * 8)                    # both blocks are cached
    plan = m.schedule(64)
    assert plan.seq_ids == [1] and plan.context_lens == [8]
    assert plan.query_start[1] >= 1              # the last prompt token is computed
    assert plan.block_tables[0][0] == m.table(0)[0]


# ---------------------------------------------------------------------------
# brute force: content model over random traces
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("setting", TRACE_SETTINGS)
def test_random_traces_keep_every_prefix(setting):
    seen = dict(preempt=0, swap=0, cow=0, hits=0)
    for seed in range(6):
        got = run_checked(BlockManager, 1000 + seed, setting)
        for k in seen:
            seen[k] += got[k]
    # the traces reach the machinery they are meant to check
    assert seen["preempt"] > 0
    if setting[2] > 1:                 # one-token blocks are never partial
        assert seen["cow"] > 0
    if setting[4] == SWAP and setting[1] > 0:
        assert seen["swap"] > 0
    if setting[3]:
        assert seen["hits"] > 0


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

class _NoCopyOnWrite(BlockManager):
    def _shared_write_block(self, r):
        return False


class _UnchainedKeys(BlockManager):
    """Keys a block by its own tokens only, not chained with the prefix before it."""

    def _key(self, tokens, j):
        return tuple(tokens[j * self.B:(j + 1) * self.B])


class _PriorityInverted(BlockManager):
    """Serves the latest arrival first, so the oldest request becomes the victim."""

    def _by_arrival(self, state):
        got = super()._by_arrival(state)
        return got[::-1] if state == RUNNING else got


class _KeyOutlivesNewContent(BlockManager):
    def _pop_gpu(self):
        b = self.free.pop(0)
        self.refcount[b] = 1
        return b


class _CowKeepsReference(BlockManager):
    def _schedule(self, r, n, plan):
        shared = self._shared_write_block(r)
        old = r.blocks[r.computed // self.B] if shared else None
        super()._schedule(r, n, plan)
        if shared:
            self.refcount[old] += 1


class _ReuseCopySourceAtOnce(BlockManager):
    def _release(self, r):
        self._cow_sources = set()
        super()._release(r)


class _FloorPlusOneBlocks(BlockManager):
    def _blocks_for(self, num_tokens):
        return num_tokens // self.B + 1


def _fails_somewhere(factory, settings=TRACE_SETTINGS, seeds=range(6)) -> bool:
    for setting in settings:
        for seed in seeds:
            try:
                run_checked(factory, 1000 + seed, setting)
            except (AssertionError, IndexError, KeyError, ValueError):
                return True
    return False


@pytest.mark.parametrize("mutant", [_NoCopyOnWrite, _UnchainedKeys, _KeyOutlivesNewContent,
                                    _CowKeepsReference, _FloorPlusOneBlocks])
def test_random_traces_catch_planted_mistakes(mutant):
    assert _fails_somewhere(mutant)


def test_inverted_priority_is_caught():
    with pytest.raises(AssertionError):
        _check_youngest_preempted(_PriorityInverted)
