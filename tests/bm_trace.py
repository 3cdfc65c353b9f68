"""Seeded random request traces for block-manager tests, and a content model.

Holds none of the block manager's logic.  ``Trace`` draws a reproducible stream
of operations (add a request, schedule a step, append sampled tokens, fork,
finish) and applies the same stream to any object with the block manager's
methods.  ``ContentModel`` replays a step plan's copies and writes on plain
arrays of *prefix identities* (an integer naming the whole token prefix that a
KV row was computed from) and checks that every request reads back its own
prefixes through its table.
"""

from __future__ import annotations

import math

import numpy as np


def oracle_plan(p) -> dict:
    """An oracle step plan as plain lists, for comparison."""
    return dict(seq_ids=list(p.seq_ids), query_start=list(p.query_start),
                context_lens=list(p.context_lens), slot_mapping=list(p.slot_mapping),
                block_tables=[list(t) for t in p.block_tables],
                cow=[tuple(x) for x in p.cow_pairs], swap_out=[tuple(x) for x in p.swap_out],
                swap_in=[tuple(x) for x in p.swap_in], preempted=list(p.preempted))


def native_plan(p, block_size: int) -> dict:
    """A native step plan (numpy arrays, padded tables) in the same form."""
    tables = []
    for k, L in enumerate(p.context_lens.tolist()):
        n = math.ceil(L / block_size)
        assert not p.block_tables[k, n:].any(), "table padding must be 0"
        tables.append(p.block_tables[k, :n].tolist())
    return dict(seq_ids=p.seq_ids.tolist(), query_start=p.query_start.tolist(),
                context_lens=p.context_lens.tolist(), slot_mapping=p.slot_mapping.tolist(),
                block_tables=tables, cow=[tuple(x) for x in p.cow_pairs.tolist()],
                swap_out=[tuple(x) for x in p.swap_out.tolist()],
                swap_in=[tuple(x) for x in p.swap_in.tolist()], preempted=list(p.preempted))


class PrefixIds:
    """Interns token prefixes: the identity of position p of ``tokens``."""

    def __init__(self):
        self._ids = {}

    def of(self, tokens, p: int) -> int:
        key = tuple(tokens[:p + 1])
        return self._ids.setdefault(key, len(self._ids))


class ContentModel:
    """GPU and CPU pools of prefix identities (-1 = never written)."""

    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int, block_size: int):
        self.B = block_size
        self.gpu = np.full((num_gpu_blocks, block_size), -1, dtype=np.int64)
        self.cpu = np.full((max(num_cpu_blocks, 1), block_size), -1, dtype=np.int64)
        self.ids = PrefixIds()

    def apply(self, plan, tokens_of) -> None:
        """Run a plan's copies and writes in their execution order."""
        for g, c in plan.swap_out:
            self.cpu[c] = self.gpu[g]
        for c, g in plan.swap_in:
            self.gpu[g] = self.cpu[c]
        srcs = {s for s, _ in plan.cow_pairs}
        dsts = [d for _, d in plan.cow_pairs]
        assert len(set(dsts)) == len(dsts) and not (srcs & set(dsts)), "copy hazard"
        before = self.gpu.copy()
        for s, d in plan.cow_pairs:
            self.gpu[d] = before[s]
        slots = list(plan.slot_mapping)
        assert len(set(slots)) == len(slots), "a slot written twice"
        for k, rid in enumerate(plan.seq_ids):
            toks = tokens_of(rid)
            start = plan.context_lens[k] - (plan.query_start[k + 1] - plan.query_start[k])
            for i, p in enumerate(range(start, plan.context_lens[k])):
                s = slots[plan.query_start[k] + i]
                self.gpu[s // self.B, s % self.B] = self.ids.of(toks, p)

    def read(self, table, length: int, cpu: bool = False) -> list:
        pool = self.cpu if cpu else self.gpu
        return [int(pool[table[p // self.B], p % self.B]) for p in range(length)]

    def expected(self, tokens, length: int) -> list:
        return [self.ids.of(tokens, p) for p in range(length)]


class Trace:
    """A seeded stream of block-manager operations on a small pool."""

    def __init__(self, seed: int, num_gpu_blocks: int = 24, num_cpu_blocks: int = 16,
                 block_size: int = 4, vocab: int = 3, max_new_requests: int = 2,
                 fork_prob: float = 0.1, finish_prob: float = 0.08, watermark: int = 0):
        self.rng = np.random.default_rng(seed)
        self.B = block_size
        self.vocab = vocab
        self.max_new = max_new_requests
        self.fork_prob = fork_prob
        self.finish_prob = finish_prob
        # longest request that can always be admitted on an empty pool
        self.max_len = (num_gpu_blocks - watermark) * block_size - 1
        self.preambles = [list(self.rng.integers(0, vocab, int(self.rng.integers(1, 3 * block_size))))
                          for _ in range(3)]
        self.next_rid = 0
        self.live = {}   # rid -> token list, mirrored from the driver's own ops

    def _prompt(self) -> list:
        head = self.preambles[int(self.rng.integers(0, len(self.preambles)))] \
            if self.rng.random() < 0.6 else []
        tail = list(self.rng.integers(0, self.vocab, int(self.rng.integers(1, 2 * self.B + 2))))
        return [int(t) for t in (head + tail)][:max(1, self.max_len // 2)]

    def step(self, managers, budget_max: int = 48, on_plans=None):
        """One iteration on every manager; returns the plans (one per manager).

        ``on_plans(plans)`` runs right after scheduling, before any request of
        this step samples, forks or finishes.
        """
        for _ in range(int(self.rng.integers(0, self.max_new + 1))):
            rid, toks = self.next_rid, self._prompt()
            self.next_rid += 1
            self.live[rid] = list(toks)
            for m in managers:
                m.add_request(rid, toks)
        budget = int(self.rng.integers(1, budget_max + 1))
        plans = [m.schedule(budget) for m in managers]
        self.tokens_at_schedule = {rid: list(t) for rid, t in self.live.items()}
        if on_plans is not None:
            on_plans(plans)
        ref = managers[0]
        # requests whose KV now covers all their tokens sample one more
        for rid in sorted(self.live):
            info = ref.request_info(rid)
            if info["state"] != "running" or info["computed"] != len(self.live[rid]):
                continue
            if len(self.live[rid]) >= self.max_len or self.rng.random() < self.finish_prob:
                del self.live[rid]
                for m in managers:
                    m.finish(rid)
                continue
            if self.rng.random() < self.fork_prob:
                child = self.next_rid
                self.next_rid += 1
                self.live[child] = list(self.live[rid])
                for m in managers:
                    m.fork(rid, child)
                tok = int(self.rng.integers(0, self.vocab))
                self.live[child].append(tok)
                for m in managers:
                    m.append_token(child, tok)
            tok = int(self.rng.integers(0, self.vocab))
            self.live[rid].append(tok)
            for m in managers:
                m.append_token(rid, tok)
        # now and then a waiting or swapped request is aborted
        for rid in sorted(self.live):
            if ref.request_info(rid)["state"] != "running" and self.rng.random() < self.finish_prob / 2:
                del self.live[rid]
                for m in managers:
                    m.finish(rid)
        return plans
