"""Plain CPU oracle of the paged KV block manager and its per-step scheduler.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module.  It shares no code with the native library and imports
nothing from it.

What it models, and the passages each part follows:

* The block pool and its free list.  Memory is cut into fixed-size blocks kept
  in a free list; allocation pops a block from it and freeing pushes the block
  back, and a request holding t tokens holds ceil(t/B) blocks ("How Paged
  Attention and Continuous Batching Actually Work", section "Paged attention:
  virtual memory for the KV cache").
* Block tables.  Entry j of a request's table is the physical block behind its
  logical tokens [jB, jB+B) ("LLM paged attention arch", section "The
  architecture: every piece explained"); the flat slot of position p is
  table[p // B] * B + p % B.
* Prefix cache.  Every full block is keyed by its token ids chained with the
  key of the prefix before it; a new prompt whose leading blocks match keys
  already resident points its table at those blocks and bumps their reference
  counts, and their prefill is skipped.  Freed blocks keep their key, so a
  shared preamble "stays warm" for the next request (same page and section,
  and its section "End-to-end flow").
* Copy-on-write.  A write into a block whose reference count exceeds one takes
  a fresh block, copies the old content into it, points the writer's table at
  it and drops the old block's count ("Paged Attention as a Memory Manager",
  section "Prefix Caching and Copy-on-Write").
* The step.  Each iteration first walks the running requests granting each the
  slots for the tokens it needs this step (``allocate_slots``), then admits
  waiting requests while a per-step token budget lasts; a long prompt is fed in
  budget-sized slices (chunked prefill).  When the pool runs dry the
  lowest-priority request is preempted and returns its blocks ("How Paged
  Attention and Continuous Batching Actually Work", sections "Continuous
  batching: schedule steps, not batches" and "One step, end to end").
  Priority is arrival: the victim is the latest-arrived request, whose KV is
  either copied to CPU blocks (swap) for a later swap-in or dropped and
  recomputed from its tokens; shared blocks only lose a reference ("LLM paged
  attention arch", sections "The architecture: every piece explained" and
  "End-to-end flow").  Admission asks whether the pool holds the prompt's
  blocks plus a margin (same page, admission row of the architecture).

Where the pages leave a step open, this module takes the readings below (each
is one plain choice; none is claimed by the pages):

1. The free list is a queue: allocation takes its front, a freed block joins
   its back; at start it holds blocks 0, 1, ..., N-1 in that order.  The same
   holds for the CPU pool used by swapping.
2. A request releases its blocks last block first, so its leading blocks (the
   ones a later prompt is most likely to share) are the last to be reused.
3. Priority is arrival order (earlier is higher).  Running requests are served
   in arrival order; the preemption victim is the latest-arrived running
   request not yet served in this step, which may be the one asking.
4. A prefix key is the whole token prefix through the end of the block (the
   chained hash of the pages, without the hash); only full blocks are keyed;
   matching stops at the first block not found; at most floor((len-1)/B)
   blocks are taken from the cache, so at least the last prompt token is
   computed (its output is what the first sample is drawn from).
5. A key stays with its block after the block is freed and leaves the cache
   when the block is popped for new content.  A block whose key is already
   cached (filled by another request with the same prefix) stays unkeyed.
6. Copy-on-write triggers when the first position a request writes this step
   lies inside an existing partial block with reference count > 1 (after a
   fork); full blocks are never written.
7. A block freed during a step that is the source of one of that step's
   copy-on-write copies rejoins the free queue only when the step ends, so no
   block is both a copy source and a copy destination within one step.
8. Swap-out needs one CPU block per GPU block of the victim; without enough CPU
   blocks the victim is recomputed instead.  Swapped-in blocks are private and
   unkeyed.
9. Swapped requests (first) and waiting requests (then) are taken in arrival
   order, and only in a step in which nobody was preempted; taking stops at the
   first one that does not fit.  Admission of a waiting request checks the
   blocks of its whole prompt (plus the margin); only the blocks of the
   scheduled slice are allocated.  Swap-in checks the blocks it allocates.
10. A fork copies the parent's tokens, computed count and table; every block
    gains a reference; the child arrives after every earlier request.

The step plan lists, in this order of execution on the device: swap-out copies
(GPU block -> CPU block), swap-in copies (CPU block -> GPU block), copy-on-write
copies (GPU block -> GPU block), then the KV writes of every scheduled token
through ``slot_mapping``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .paged_attention import blocks_needed, slot_of

WAITING, RUNNING, SWAPPED = "waiting", "running", "swapped"
RECOMPUTE, SWAP = "recompute", "swap"


@dataclass
class Request:
    rid: int
    arrival: int
    tokens: list
    state: str = WAITING
    blocks: list = field(default_factory=list)      # GPU block table
    cpu_blocks: list = field(default_factory=list)  # CPU blocks while swapped
    computed: int = 0                               # tokens whose KV is in the cache


@dataclass
class StepPlan:
    """What one step asks of the device, in execution order (see module doc)."""
    seq_ids: list = field(default_factory=list)      # scheduled requests, in order
    query_start: list = field(default_factory=lambda: [0])  # token offsets, len S+1
    context_lens: list = field(default_factory=list)  # tokens attended after the writes
    slot_mapping: list = field(default_factory=list)  # one slot per scheduled token
    block_tables: list = field(default_factory=list)  # each scheduled request's table
    cow_pairs: list = field(default_factory=list)     # (src GPU block, dst GPU block)
    swap_out: list = field(default_factory=list)      # (GPU block, CPU block)
    swap_in: list = field(default_factory=list)       # (CPU block, GPU block)
    preempted: list = field(default_factory=list)     # (rid, RECOMPUTE | SWAP)


class BlockManager:
    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int, block_size: int,
                 prefix_caching: bool = True, preempt_mode: str = RECOMPUTE,
                 watermark_blocks: int = 0):
        if num_gpu_blocks <= 0 or num_cpu_blocks < 0 or block_size <= 0 or watermark_blocks < 0:
            raise ValueError("bad block manager sizes")
        if preempt_mode not in (RECOMPUTE, SWAP):
            raise ValueError("preempt_mode is 'recompute' or 'swap'")
        self.B = block_size
        self.num_gpu_blocks = num_gpu_blocks
        self.num_cpu_blocks = num_cpu_blocks
        self.prefix_caching = prefix_caching
        self.preempt_mode = preempt_mode
        self.watermark = watermark_blocks
        self.free = list(range(num_gpu_blocks))      # reading 1
        self.cpu_free = list(range(num_cpu_blocks))
        self.refcount = [0] * num_gpu_blocks
        self.cache = {}        # prefix tuple -> GPU block
        self.block_key = {}    # GPU block -> prefix tuple
        self.requests = {}     # rid -> Request
        self._arrivals = 0
        self._cow_sources = set()   # reading 7, per step
        self._deferred = []
        # running totals: the telemetry the pages name (block use, preemption
        # rate, prefix hit rate; "LLM paged attention arch", section "The
        # architecture: every piece explained")
        self.totals = dict(preemptions=0, swapped_out_blocks=0, swapped_in_blocks=0,
                           cow_copies=0, prefix_hit_tokens=0, admitted_tokens=0)

    # -- request lifecycle ---------------------------------------------------

    def add_request(self, rid: int, tokens) -> None:
        tokens = [int(t) for t in tokens]
        if rid in self.requests:
            raise ValueError(f"request {rid} exists")
        if not tokens:
            raise ValueError("empty prompt")
        if self._blocks_for(len(tokens)) > self.num_gpu_blocks - self.watermark:
            raise ValueError("prompt can never fit the pool")
        self.requests[rid] = Request(rid, self._arrivals, tokens)
        self._arrivals += 1

    def append_token(self, rid: int, token: int) -> None:
        self._get(rid).tokens.append(int(token))

    def fork(self, parent: int, child: int) -> None:
        p = self._get(parent)
        if p.state != RUNNING:
            raise ValueError("only a running request can be forked")
        if child in self.requests:
            raise ValueError(f"request {child} exists")
        c = Request(child, self._arrivals, list(p.tokens), RUNNING, list(p.blocks), [], p.computed)
        self._arrivals += 1
        for b in c.blocks:
            self.refcount[b] += 1
        self.requests[child] = c

    def finish(self, rid: int) -> None:
        """A finished (or aborted) request pushes its blocks back at once."""
        r = self._get(rid)
        self._release(r)
        for cb in reversed(r.cpu_blocks):
            self.cpu_free.append(cb)
        del self.requests[rid]

    # -- the step ------------------------------------------------------------

    def schedule(self, token_budget: int) -> StepPlan:
        if token_budget <= 0:
            raise ValueError("token_budget must be positive")
        plan = StepPlan()
        budget = token_budget
        self._cow_sources, self._deferred = set(), []

        # 1. running requests, highest priority (earliest arrival) first
        order = self._by_arrival(RUNNING)
        end = len(order)
        i = 0
        while i < end:
            r = order[i]
            n = min(len(r.tokens) - r.computed, budget)
            if n == 0:
                i += 1
                continue
            preempted_self = False
            while self._blocks_to_grow(r, n) > len(self.free):
                victim = order[end - 1]
                end -= 1
                self._preempt(victim, plan)
                if victim is r:
                    preempted_self = True
                    break
            if preempted_self:
                break
            self._schedule(r, n, plan)
            budget -= n
            i += 1

        # 2. swapped, then waiting requests, only if nobody was preempted;
        #    taking stops at the first request that does not fit (reading 9)
        if not plan.preempted:
            stopped = False
            for r in self._by_arrival(SWAPPED):
                n = min(len(r.tokens) - r.computed, budget)
                if budget == 0 or len(self.free) - self._blocks_for(r.computed + n) < self.watermark:
                    stopped = True
                    break
                self._swap_in(r, plan)
                if n:
                    self._schedule(r, n, plan)
                    budget -= n
            for r in ([] if stopped else self._by_arrival(WAITING)):
                if budget == 0:
                    break
                hits = self._prefix_hits(r.tokens)
                cached = len(hits) * self.B
                n = min(len(r.tokens) - cached, budget)
                taken_from_free = sum(1 for b in hits if self.refcount[b] == 0)
                need = self._blocks_for(len(r.tokens)) - len(hits) + taken_from_free
                if len(self.free) - need < self.watermark:
                    break
                for b in hits:
                    if self.refcount[b] == 0:
                        self.free.remove(b)
                    self.refcount[b] += 1
                r.blocks = list(hits)
                r.computed = cached
                r.state = RUNNING
                self.totals["prefix_hit_tokens"] += cached
                self.totals["admitted_tokens"] += len(r.tokens)
                self._schedule(r, n, plan)
                budget -= n

        self.free.extend(self._deferred)
        self._cow_sources, self._deferred = set(), []
        return plan

    # -- internals -------------------------------------------------------------

    def _get(self, rid: int) -> Request:
        if rid not in self.requests:
            raise KeyError(f"no request {rid}")
        return self.requests[rid]

    def _by_arrival(self, state: str) -> list:
        return sorted((r for r in self.requests.values() if r.state == state),
                      key=lambda r: r.arrival)

    def _blocks_for(self, num_tokens: int) -> int:
        """Blocks that hold ``num_tokens`` tokens: ceil(t / B)."""
        return blocks_needed(num_tokens, self.B)

    def _key(self, tokens, j: int) -> tuple:
        """Reading 4: the key of logical block j is the token prefix through its end."""
        return tuple(tokens[:(j + 1) * self.B])

    def _pop_gpu(self) -> int:
        b = self.free.pop(0)
        key = self.block_key.pop(b, None)   # reading 5: new content evicts the key
        if key is not None:
            del self.cache[key]
        self.refcount[b] = 1
        return b

    def _release(self, r: Request) -> None:
        for b in reversed(r.blocks):        # reading 2
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                if b in self._cow_sources:  # reading 7
                    self._deferred.append(b)
                else:
                    self.free.append(b)
        r.blocks = []

    def _shared_write_block(self, r: Request) -> bool:
        """Reading 6: the first position to write lies in a shared partial block."""
        c = r.computed
        return c % self.B != 0 and self.refcount[r.blocks[c // self.B]] > 1

    def _blocks_to_grow(self, r: Request, n: int) -> int:
        grow = self._blocks_for(r.computed + n) - len(r.blocks)
        return grow + (1 if self._shared_write_block(r) else 0)

    def _schedule(self, r: Request, n: int, plan: StepPlan) -> None:
        """allocate_slots for positions computed .. computed+n-1, then record them."""
        c = r.computed
        if self._shared_write_block(r):
            j = c // self.B
            old, new = r.blocks[j], self._pop_gpu()
            self.refcount[old] -= 1
            r.blocks[j] = new
            plan.cow_pairs.append((old, new))
            self._cow_sources.add(old)
            self.totals["cow_copies"] += 1
        while len(r.blocks) < self._blocks_for(c + n):
            r.blocks.append(self._pop_gpu())
        if self.prefix_caching:
            for j in range(c // self.B, (c + n) // self.B):   # blocks that become full
                key = self._key(r.tokens, j)
                b = r.blocks[j]
                if key not in self.cache and b not in self.block_key:
                    self.cache[key] = b
                    self.block_key[b] = key
        r.computed = c + n
        plan.seq_ids.append(r.rid)
        plan.slot_mapping.extend(slot_of(r.blocks, p, self.B) for p in range(c, c + n))
        plan.query_start.append(plan.query_start[-1] + n)
        plan.context_lens.append(r.computed)
        plan.block_tables.append(list(r.blocks))

    def _prefix_hits(self, tokens) -> list:
        if not self.prefix_caching:
            return []
        hits = []
        for j in range((len(tokens) - 1) // self.B):          # reading 4
            b = self.cache.get(self._key(tokens, j))
            if b is None:
                break
            hits.append(b)
        return hits

    def _preempt(self, r: Request, plan: StepPlan) -> None:
        self.totals["preemptions"] += 1
        if self.preempt_mode == SWAP and len(self.cpu_free) >= len(r.blocks):
            for b in r.blocks:
                cb = self.cpu_free.pop(0)
                r.cpu_blocks.append(cb)
                plan.swap_out.append((b, cb))
            self.totals["swapped_out_blocks"] += len(r.blocks)
            self._release(r)
            r.state = SWAPPED
            plan.preempted.append((r.rid, SWAP))
        else:                                                    # reading 8
            self._release(r)
            r.computed = 0
            r.state = WAITING
            plan.preempted.append((r.rid, RECOMPUTE))

    def _swap_in(self, r: Request, plan: StepPlan) -> None:
        for cb in r.cpu_blocks:
            b = self._pop_gpu()
            r.blocks.append(b)
            plan.swap_in.append((cb, b))
        self.totals["swapped_in_blocks"] += len(r.cpu_blocks)
        for cb in reversed(r.cpu_blocks):
            self.cpu_free.append(cb)
        r.cpu_blocks = []
        r.state = RUNNING

    # -- views used by tests ---------------------------------------------------

    def table(self, rid: int) -> list:
        return list(self._get(rid).blocks)

    def request_info(self, rid: int) -> dict:
        r = self._get(rid)
        return dict(state=r.state, computed=r.computed, num_tokens=len(r.tokens),
                    arrival=r.arrival, num_blocks=len(r.blocks), num_cpu_blocks=len(r.cpu_blocks))

    def stats(self) -> dict:
        states = [r.state for r in self.requests.values()]
        return dict(free_gpu_blocks=len(self.free), free_cpu_blocks=len(self.cpu_free),
                    cached_blocks=len(self.cache), running=states.count(RUNNING),
                    waiting=states.count(WAITING), swapped=states.count(SWAPPED), **self.totals)


def swap_blocks(dst_pool, src_pool, pairs):
    """Destination pool after copying block src to block dst for every pair.

    The data movement of a swap: a victim's blocks are copied to pinned CPU
    memory and back ("LLM paged attention arch", section "The architecture:
    every piece explained").  Pools are arrays ``[num_blocks][...]``; every
    byte of block ``src`` of ``src_pool`` lands in block ``dst`` of the copy of
    ``dst_pool``; destinations must be distinct.
    """
    out = np.array(dst_pool, copy=True)
    pairs = [(int(a), int(b)) for a, b in pairs]
    dsts = [b for _, b in pairs]
    if len(set(dsts)) != len(dsts):
        raise ValueError("swap pairs need distinct destinations")
    for src, dst in pairs:
        out[dst] = src_pool[src]
    return out
