"""Plain-Python oracle of the host block manager and the iteration-level scheduler.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix, and what this module restates:
  * Static batching launches a fixed batch and releases it only when its
    slowest member finishes; finished members leave their slot idle ("Module 4
    · Batching, Scheduling, and Paging", section "Static batching: the batch
    waits for its slowest member").
  * Continuous batching reschedules every iteration: finished sequences leave
    and waiting requests are admitted into the freed slots (same page, section
    "Continuous batching: reschedule every iteration"; worksonmygpu.com post,
    section "Iteration-level scheduling").
  * Orca avoids running out of KV memory by reserving the maximum response
    length for every admitted request (Module 4, "Continuous batching", the
    tradeoff note; "Paging the KV Cache", section "The waste hiding inside
    memory").
  * Under PagedAttention a sequence gets a new block at the moment its last
    one is full, returns all of its blocks when it ends, and is pushed out
    (dropped, to be recomputed) when device memory runs short (Module 4,
    section "PagedAttention").
  * The samples of one prompt point at the prompt's blocks; a shared block is
    duplicated before a write that would make the samples differ, and a count
    of sharers per block decides when it is free again (Module 4, section
    "Block sharing").
  * Prefill and decode share an iteration under a policy that bounds the work
    of one iteration (worksonmygpu.com post, section "The prefill/decode mix").

Where the pages leave a step open, the reading taken here (each is listed in
the design notes):
  * one iteration has a token budget: decode tokens first (one per running
    sample), then prefill chunks of at most ``max_chunk`` tokens, continuing
    requests before admitting new ones;
  * admission is first come, first served and never skips the head of the
    queue; a request with n samples takes n batch slots from admission on;
    continuous batching admits only while the iteration's token budget lasts,
    while a static batch is formed whole (its later members start their
    prefill in the following iterations);
  * a decode sequence appends the KV of its previous token and produces the
    next; a prompt's last prefill chunk produces every sample's first token;
  * the free list is a stack: blocks are taken in ``free_order`` at first and
    a released block is the next one taken;
  * paged eviction: before any append of an iteration, while the free blocks
    cannot cover what the running requests need this iteration (one block per
    decode sample whose last block is full or shared, plus the blocks of each
    continuing prefill chunk), the most recently admitted running request is
    evicted: its blocks are released and it restarts from its prompt at the
    head of the queue; an iteration that evicted admits nobody;
  * reservation (Orca, and static batching) holds ceil(max_len / bs) blocks per
    sample from admission until that sample finishes (static: until the batch
    ends); without paging, samples do not share, so the prompt's blocks are
    copied into each further sample's reservation before its first decode;
  * swapping (paged, when host blocks are configured): an evicted request that
    is decoding and whose blocks fit the free host blocks is swapped out
    instead of dropped -- each of its distinct blocks goes to one host block
    (first appearance in sample, then table order; host blocks are a stack
    like the device ones) -- and keeps its progress. Back at the head of the
    queue it is swapped in when its samples fit the free slots and its blocks
    the free device blocks: one new device block per host block, the samples'
    sharing kept, the host blocks released in the same order. A swapped-in
    request needs no prefill and takes no token budget; it decodes from the
    next iteration on. In one iteration the GPU runs the swap-outs, then the
    swap-ins, then the copies, appends and attention;
  * prefix caching (paged, when enabled; "Module 4", section "Block sharing",
    its note on sharing identical prefixes across requests): a request may
    name a prefix -- (prefix id, length): its first `length` prompt tokens
    equal those of every request naming the same id. A full block inside the
    prefix, once prefilled, is entered in a cache under (prefix id, block
    index), and the cache holds a reference to it. An admitted request takes
    the cached blocks of its prefix from block 0 up to the first miss (never
    its whole prompt: the last prompt token is always computed) and starts
    its prefill after them. Cache entries are kept in least-recently-used
    order (a hit or an entry moves a key to the back); when a block is needed
    and none is free, the oldest entry that only the cache still holds gives
    up its block. Those blocks count as free in every fit test.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field

POLICIES = ("paged", "reserve", "static")


@dataclass
class SchedConfig:
    num_blocks: int
    block_size: int
    max_seqs: int      # batch slots: samples that may run at once
    max_tokens: int    # tokens one iteration may process (decode + prefill)
    max_chunk: int     # longest prefill chunk
    max_len: int       # longest context a sample may reach (prompt + output - 1)
    policy: str = "paged"
    num_host_blocks: int = 0   # paged: host blocks for swapping (0: evictions recompute)
    prefix_caching: bool = False   # paged: reuse full prefix blocks across requests


@dataclass
class Plan:
    """What one iteration does, in launch order: copies, then appends, then attention."""
    iteration: int
    copies: list = field(default_factory=list)    # (src, dst) block pairs
    slots: list = field(default_factory=list)     # prefill tokens (chunk order), then decode tokens
    chunks: list = field(default_factory=list)    # (req, q_start, length, context_len, table)
    decodes: list = field(default_factory=list)   # (req, sample, context_len, table)
    admitted: list = field(default_factory=list)
    preempted: list = field(default_factory=list)
    finished: list = field(default_factory=list)
    generated: int = 0
    swap_out: list = field(default_factory=list)  # (device block, host block), first
    swap_in: list = field(default_factory=list)   # (host block, device block), second


class _Sample:
    def __init__(self, table, ntok, out):
        self.table = table
        self.ntok = ntok      # tokens whose KV is cached
        self.gen = 1          # tokens produced (the prefill produced the first)
        self.out = out
        self.done = out == 1
        self.released = False
        self.host_table = None  # host blocks while swapped out


class _Request:
    def __init__(self, rid, prompt, outs, arrival, prefix_id=-1, prefix_len=0):
        self.rid = rid
        self.prompt = int(prompt)
        self.outs = [int(o) for o in outs]
        self.arrival = int(arrival)
        self.prefix_id = int(prefix_id)
        self.prefix_len = int(prefix_len) if prefix_id >= 0 else 0
        self.reset()
        self.evictions = 0

    def reset(self):
        self.state = "waiting"
        self.prefilled = 0
        self.table = []        # the prompt's table while it is prefilled
        self.reserved = []     # reservation tables of samples 1 .. n-1
        self.samples = []

    @property
    def n(self):
        return len(self.outs)


def _cdiv(a, b):
    return -(-a // b)


class Scheduler:
    """Drives requests through prefill and decode, one ``step()`` per iteration.

    ``requests`` is a list of (prompt_len, [output_len per sample], arrival_iteration)
    or (prompt_len, [output_len per sample], arrival_iteration, prefix_id, prefix_len),
    in arrival order; ``free_order`` lists every block id once.
    """

    def __init__(self, cfg: SchedConfig, free_order, requests):
        if cfg.policy not in POLICIES:
            raise ValueError(f"unknown policy {cfg.policy!r}")
        if cfg.num_host_blocks < 0 or (cfg.num_host_blocks > 0 and cfg.policy != "paged"):
            raise ValueError("host blocks serve the paged policy's evictions only")
        if cfg.prefix_caching and cfg.policy != "paged":
            raise ValueError("prefix caching needs the paged policy")
        self.cfg = cfg
        order = [int(b) for b in free_order]
        if sorted(order) != list(range(cfg.num_blocks)):
            raise ValueError("free_order must list every block id once")
        self.free = order[::-1]               # a stack: free[-1] is taken next
        self.ref = [0] * cfg.num_blocks
        self.host_free = list(range(cfg.num_host_blocks))[::-1]   # host block 0 first
        self.cache = {}    # (prefix id, block index) -> block
        self.lru = []      # cache keys, least recently used first
        self.reqs = []
        for i, req in enumerate(requests):
            r = _Request(i, *req)
            if r.prompt < 1 or r.n < 1 or min(r.outs) < 1:
                raise ValueError(f"request {i}: empty prompt or output")
            if not 0 <= r.prefix_len <= r.prompt:
                raise ValueError(f"request {i}: prefix longer than the prompt")
            if r.prompt + max(r.outs) - 1 > cfg.max_len:
                raise ValueError(f"request {i} exceeds max_len")
            worst = r.n * _cdiv(cfg.max_len if cfg.policy != "paged"
                                else r.prompt + max(r.outs) - 1, cfg.block_size)
            if worst > cfg.num_blocks or r.n > cfg.max_seqs:
                raise ValueError(f"request {i} can never fit")
            self.reqs.append(r)
        self.pending = deque(range(len(self.reqs)))
        self.waiting = deque()
        self.running = []          # admission order
        self.slots_used = 0
        self.pending_copies = []   # prompt copies into reservations, for the next iteration
        self.it = 0

    # -- block manager ---------------------------------------------------------------
    def _alloc(self):
        if not self.free:   # the oldest cache entry nobody else holds gives up its block
            key = next(k for k in self.lru if self.ref[self.cache[k]] == 1)
            self.lru.remove(key)
            b = self.cache.pop(key)
            self.ref[b] = 0
            self.free.append(b)
        b = self.free.pop()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _available(self):
        """Blocks an allocation can get: free ones and cached ones only the cache holds."""
        return len(self.free) + sum(1 for b in self.cache.values() if self.ref[b] == 1)

    def _prefix_hits(self, r):
        """Cached blocks of r's prefix from block 0 up to the first miss."""
        if not self.cfg.prefix_caching or r.prefix_id < 0:
            return []
        bs, hits = self.cfg.block_size, []
        limit = min(r.prefix_len, r.prompt - 1)
        while (len(hits) + 1) * bs <= limit and (r.prefix_id, len(hits)) in self.cache:
            hits.append(self.cache[(r.prefix_id, len(hits))])
        return hits

    def _touch(self, key):
        if key in self.lru:
            self.lru.remove(key)
        self.lru.append(key)

    def _release_table(self, table):
        for b in table:
            self.ref[b] -= 1
            assert self.ref[b] >= 0
            if self.ref[b] == 0:
                self.free.append(b)

    def _write_slot(self, table, pos, copies):
        """Slot of logical position ``pos``; allocates on fill, copies a shared block."""
        bs = self.cfg.block_size
        j = pos // bs
        if j == len(table):
            table.append(self._alloc())
        elif self.ref[table[j]] > 1:
            new = self._alloc()
            copies.append((table[j], new))
            self.ref[table[j]] -= 1
            table[j] = new
        return table[j] * bs + pos % bs

    # -- eviction ----------------------------------------------------------------------
    def _swap_out(self, r, plan):
        """Swap a decoding request's blocks to host blocks; False if they do not fit."""
        live = [q for q in r.samples if not q.released]
        uniq = []
        for q in live:
            for b in q.table:
                if b not in uniq:
                    uniq.append(b)
        if len(uniq) > len(self.host_free):
            return False
        where = {}
        for b in uniq:
            where[b] = self.host_free.pop()
            plan.swap_out.append((b, where[b]))
        for q in live:
            q.host_table = [where[b] for b in q.table]
            self._release_table(q.table)
            q.table = None
            self.slots_used -= 1
        r.state = "swapped"
        return True

    def _swap_in(self, r, plan):
        live = [q for q in r.samples if not q.released]
        uniq = []
        for q in live:
            for h in q.host_table:
                if h not in uniq:
                    uniq.append(h)
        if self.slots_used + len(live) > self.cfg.max_seqs or len(uniq) > self._available():
            return False
        where = {}
        for h in uniq:
            where[h] = self._alloc()
            plan.swap_in.append((h, where[h]))
        for q in live:
            q.table = [where[h] for h in q.host_table]
            q.host_table = None
        for b in where.values():   # the samples share blocks as before
            self.ref[b] = sum(q.table.count(b) for q in live)
        for h in uniq:
            self.host_free.append(h)
        self.slots_used += len(live)
        r.state = "decode"
        return True

    def _evict(self, rid, plan):
        r = self.reqs[rid]
        if r.state == "decode" and self.cfg.num_host_blocks > 0 and self._swap_out(r, plan):
            r.evictions += 1
            self.running.remove(rid)
            self.waiting.appendleft(rid)
            plan.preempted.append(rid)
            return
        if r.state == "prefill":
            self._release_table(r.table)
            for t in r.reserved:
                self._release_table(t)
            self.slots_used -= r.n
        else:
            for s in r.samples:
                if not s.released:
                    self._release_table(s.table)
                    self.slots_used -= 1
        r.reset()
        r.evictions += 1
        self.running.remove(rid)
        self.waiting.appendleft(rid)
        plan.preempted.append(rid)

    def _need(self, budget):
        """Blocks the running requests may take this iteration (an upper bound)."""
        cfg, n, b = self.cfg, 0, budget
        for _, _, s in self._decode_samples():
            if b == 0:
                break
            b -= 1
            if s.ntok % cfg.block_size == 0 or self.ref[s.table[-1]] > 1:
                n += 1
        for rid in self.running:
            r = self.reqs[rid]
            if r.state == "prefill":
                L = min(r.prompt - r.prefilled, cfg.max_chunk, b)
                if L <= 0:
                    break
                n += _cdiv(r.prefilled + L, cfg.block_size) - len(r.table)
                b -= L
        return n

    def _decode_samples(self):
        for rid in self.running:
            r = self.reqs[rid]
            if r.state == "decode":
                for k, s in enumerate(r.samples):
                    if not s.done:
                        yield rid, k, s

    # -- prefill -----------------------------------------------------------------------
    def _chunk(self, rid, plan, budget, pre_slots):
        """Schedule the next prefill chunk of ``rid`` (its blocks are available); its length."""
        cfg, r = self.cfg, self.reqs[rid]
        L = min(r.prompt - r.prefilled, cfg.max_chunk, budget)
        if L <= 0:
            return 0
        q_start = len(pre_slots)
        for pos in range(r.prefilled, r.prefilled + L):
            pre_slots.append(self._write_slot(r.table, pos, plan.copies))
        before = r.prefilled
        r.prefilled += L
        if cfg.prefix_caching and r.prefix_id >= 0:   # full prefix blocks this chunk completed
            bs = cfg.block_size
            for j in range(before // bs, r.prefilled // bs):
                key = (r.prefix_id, j)
                if (j + 1) * bs <= r.prefix_len and key not in self.cache:
                    self.cache[key] = r.table[j]
                    self.ref[r.table[j]] += 1
                    self._touch(key)
        plan.chunks.append((rid, q_start, L, r.prefilled, list(r.table)))
        if r.prefilled == r.prompt:          # the prompt's last chunk: fork into samples
            r.state = "decode"
            r.samples = [_Sample(r.table, r.prompt, r.outs[0])]
            for k in range(1, r.n):
                if cfg.policy == "paged":
                    for b in r.table:
                        self.ref[b] += 1
                    t = list(r.table)
                else:
                    t = r.reserved[k - 1]
                    for j in range(_cdiv(r.prompt, cfg.block_size)):
                        self.pending_copies.append((r.table[j], t[j]))
                r.samples.append(_Sample(t, r.prompt, r.outs[k]))
            r.reserved = []
            plan.generated += r.n
        return L

    # -- one iteration ---------------------------------------------------------------
    def done(self):
        return not self.pending and not self.waiting and not self.running

    def step(self):
        """Plan and apply one iteration; None once every request has finished."""
        if self.done():
            return None
        cfg = self.cfg
        plan = Plan(self.it)
        plan.copies.extend(self.pending_copies)
        self.pending_copies = []
        while self.pending and self.reqs[self.pending[0]].arrival <= self.it:
            self.waiting.append(self.pending.popleft())
        batch_empty = not self.running
        budget = cfg.max_tokens
        # eviction until the running requests' appends of this iteration fit
        if cfg.policy == "paged":
            while self._need(budget) > self._available():
                if len(self.running) <= 1:
                    raise AssertionError("a lone request does not fit the pool")
                self._evict(self.running[-1], plan)
        dec_slots = []
        for rid, k, s in list(self._decode_samples()):
            if budget == 0:
                break
            dec_slots.append(self._write_slot(s.table, s.ntok, plan.copies))
            s.ntok += 1
            s.gen += 1
            s.done = s.gen == s.out
            plan.decodes.append((rid, k, s.ntok, list(s.table)))
            plan.generated += 1
            budget -= 1
        pre_slots = []
        for rid in list(self.running):
            if self.reqs[rid].state == "prefill":
                budget -= self._chunk(rid, plan, budget, pre_slots)
        admitting = not plan.preempted and (cfg.policy != "static" or batch_empty)
        # a static batch is formed whole; continuous batching admits only what
        # this iteration's budget can start on
        while admitting and self.waiting and (budget > 0 or cfg.policy == "static"):
            rid = self.waiting[0]
            r = self.reqs[rid]
            if r.state == "swapped":   # back in, with its progress
                if not self._swap_in(r, plan):
                    break
                self.waiting.popleft()
                self.running.append(rid)
                plan.admitted.append(rid)
                continue
            if self.slots_used + r.n > cfg.max_seqs:
                break
            hits = []
            if cfg.policy == "paged":
                hits = self._prefix_hits(r)
                got = len(hits) * cfg.block_size
                first = min(r.prompt - got, cfg.max_chunk, budget)
                held_by_cache_only = sum(1 for b in hits if self.ref[b] == 1)
                if _cdiv(got + first, cfg.block_size) - len(hits) > \
                        self._available() - held_by_cache_only:
                    break
            else:
                R = _cdiv(cfg.max_len, cfg.block_size)
                if r.n * R > len(self.free):
                    break
                r.table = [self._alloc() for _ in range(R)]
                r.reserved = [[self._alloc() for _ in range(R)] for _ in range(r.n - 1)]
            self.waiting.popleft()
            self.running.append(rid)
            self.slots_used += r.n
            r.state = "prefill"
            plan.admitted.append(rid)
            for j, b in enumerate(hits):   # the cached prefix blocks: no prefill
                self.ref[b] += 1
                r.table.append(b)
                self._touch((r.prefix_id, j))
            r.prefilled = len(hits) * cfg.block_size
            budget -= self._chunk(rid, plan, budget, pre_slots)
        plan.slots = pre_slots + dec_slots
        # release what finished in this iteration (after its kernels have run)
        if cfg.policy == "static":
            if self.running and all(self.reqs[rid].state == "decode" and
                                    all(s.done for s in self.reqs[rid].samples)
                                    for rid in self.running):
                for rid in self.running:
                    for s in self.reqs[rid].samples:
                        self._release_table(s.table)
                    self.reqs[rid].state = "done"
                    plan.finished.append(rid)
                self.running = []
                self.slots_used = 0
        else:
            for rid in list(self.running):
                r = self.reqs[rid]
                if r.state != "decode":
                    continue
                for s in r.samples:
                    if s.done and not s.released:
                        self._release_table(s.table)
                        s.released = True
                        self.slots_used -= 1
                if all(s.released for s in r.samples):
                    r.state = "done"
                    self.running.remove(rid)
                    plan.finished.append(rid)
        self.it += 1
        if not (plan.slots or plan.copies or plan.preempted or plan.finished or plan.swap_in) \
                and not self.pending:
            # nothing ran and nothing is yet to arrive: with the pool whole and
            # every request fitting alone, this cannot happen
            raise AssertionError(f"iteration {plan.iteration} made no progress")
        return plan

    def run(self):
        """Every plan until all requests finish."""
        plans = []
        while (p := self.step()) is not None:
            plans.append(p)
        return plans
