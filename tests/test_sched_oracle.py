"""Pins of the scheduler oracle (CPU only).

The oracle in oracle/scheduler.py is checked against facts that do not come
from itself:
  * a trace derived by hand from the pages' rules (allocate a block only when
    the previous one fills; copy a shared block on the first divergent write,
    the last sharer writing in place; free blocks when a sequence completes;
    a released block is the next one handed out) — "Module 4 · Batching,
    Scheduling, and Paging", sections "PagedAttention" and "Block sharing";
  * closed forms for the number of iterations when nothing but the output
    lengths limits the schedule: continuous batching ends after max(O)
    iterations, static batching after the sum over batches of each batch's
    max(O) ("Module 4", sections "Static batching" and "Continuous batching");
  * invariants on every iteration of random streams: blocks are conserved,
    reference counts equal the tables that hold each block, every written slot
    is the one its table and position imply and is written once, a written
    block is private, every request ends with exactly its output lengths, and
    the reservation policies never evict.
"""
import math

import numpy as np
import pytest

from oracle.scheduler import SchedConfig, Scheduler
from workloads.requests import make_request_stream


def _run(s, limit=20000):
    """Every plan of ``s``; a schedule that has not finished after ``limit``
    iterations is stuck (evicting and re-admitting forever)."""
    plans = []
    while (p := s.step()) is not None:
        plans.append(p)
        assert len(plans) <= limit, "the schedule does not finish"
    return plans


def _plans(policy, reqs, **kw):
    cfg = dict(num_blocks=64, block_size=8, max_seqs=12, max_tokens=64, max_chunk=32, max_len=160)
    cfg.update(kw)
    order = kw.pop("free_order", None)
    cfg.pop("free_order", None)
    if order is None:
        order = np.random.default_rng(7).permutation(cfg["num_blocks"])
    s = Scheduler(SchedConfig(policy=policy, **cfg), order, reqs)
    return s, _run(s)


def test_hand_derived_paged_trace():
    # bs 4, six blocks handed out first in the order 3, 1, 4, 0, 5, 2.
    # A: prompt 5, one sample of 3 tokens. B: prompt 3, two samples of 2
    # tokens. C: prompt 2, one sample of 1 token, arriving at iteration 2.
    cfg = SchedConfig(num_blocks=6, block_size=4, max_seqs=4, max_tokens=16, max_chunk=8,
                      max_len=16, policy="paged")
    s = Scheduler(cfg, [3, 1, 4, 0, 5, 2], [(5, [3], 0), (3, [2, 2], 0), (2, [1], 2)])
    p0, p1, p2 = s.step(), s.step(), s.step()
    assert s.step() is None
    # Iteration 0: A's prompt fills block 3 (slots 12..15) and opens block 1
    # (slot 4); B's prompt takes block 4 (slots 16..18); the prompts' last
    # chunks give A one token and B's two samples one each; B's samples share
    # block 4.
    assert p0.admitted == [0, 1]
    assert p0.slots == [12, 13, 14, 15, 4, 16, 17, 18]
    assert p0.chunks == [(0, 0, 5, 5, [3, 1]), (1, 5, 3, 3, [4])]
    assert p0.decodes == [] and p0.copies == [] and p0.generated == 3
    # Iteration 1: A writes position 5 in block 1 (slot 5). B's sample 0 is
    # the first to write into the shared block 4: it gets block 0 (copy
    # 4 -> 0, slot 3); sample 1 is then the last user and writes in place
    # (slot 19). Both B samples reach 2 tokens; their blocks 0 and 4 return to
    # the free list (in that order).
    assert p1.copies == [(4, 0)]
    assert p1.slots == [5, 3, 19]
    assert p1.decodes == [(0, 0, 6, [3, 1]), (1, 0, 4, [0]), (1, 1, 4, [4])]
    assert p1.finished == [1] and p1.generated == 3
    # Iteration 2: A writes slot 6 and finishes. C arrives and takes block 4,
    # the block released last (slots 16, 17); its one token comes from the
    # prefill, so it finishes at once.
    assert p2.admitted == [2]
    assert p2.slots == [16, 17, 6]
    assert p2.chunks == [(2, 0, 2, 2, [4])]
    assert p2.decodes == [(0, 0, 7, [3, 1])]
    assert p2.finished == [0, 2] and p2.generated == 2
    assert s.free == [2, 5, 0, 3, 1, 4]


def test_continuous_batching_ends_after_the_longest_output():
    rng = np.random.default_rng(3)
    outs = [int(o) for o in rng.integers(1, 60, 20)]
    reqs = [(int(rng.integers(1, 9)), [o], 0) for o in outs]
    for policy in ("paged", "reserve"):
        _, plans = _plans(policy, reqs, num_blocks=20 * 9, max_seqs=20, max_tokens=400,
                          max_chunk=16, max_len=72)
        assert len(plans) == max(outs)


def test_static_batching_waits_for_each_batch_slowest_member():
    rng = np.random.default_rng(4)
    outs = [int(o) for o in rng.integers(1, 60, 22)]
    reqs = [(int(rng.integers(1, 9)), [o], 0) for o in outs]
    B = 5
    _, plans = _plans("static", reqs, num_blocks=B * 9, max_seqs=B, max_tokens=400,
                      max_chunk=16, max_len=72)
    want = sum(max(outs[i:i + B]) for i in range(0, len(outs), B))
    assert len(plans) == want
    for p in plans:   # admissions only when a batch starts
        assert not p.admitted or p.iteration == 0 or plans[p.iteration - 1].finished


def _check_invariants(s, plans, reqs, bs):
    # replay the plans: every slot written once per iteration and consistent
    # with its table and position
    for p in plans:
        assert len(set(p.slots)) == len(p.slots)
        npre = sum(c[2] for c in p.chunks)
        pre, dec = p.slots[:npre], p.slots[npre:]
        for (rid, q0, L, ctx, table) in p.chunks:
            want = [table[t // bs] * bs + t % bs for t in range(ctx - L, ctx)]
            assert pre[q0:q0 + L] == want
        assert len(dec) == len(p.decodes)
        for slot, (rid, k, ctx, table) in zip(dec, p.decodes):
            assert slot == table[(ctx - 1) // bs] * bs + (ctx - 1) % bs
            assert len(table) == math.ceil(ctx / bs) or s.cfg.policy != "paged"
        # copy destinations are fresh, sources are not written through
        dsts = [d for _, d in p.copies]
        assert len(set(dsts)) == len(dsts)
        # one iteration stays within its token budget and its batch slots
        assert npre + len(p.decodes) <= s.cfg.max_tokens
        assert len(p.decodes) <= s.cfg.max_seqs
    # every request ends once with exactly its outputs
    fin = [r for p in plans for r in p.finished]
    assert sorted(fin) == list(range(len(reqs)))
    made = sum(p.generated for p in plans)
    want = sum(sum(r[1]) for r in reqs)
    evictions = sum(len(p.preempted) for p in plans)
    if s.cfg.policy != "paged":
        assert evictions == 0 and made == want
    else:
        assert made >= want and (evictions > 0 or made == want)
    # the pool is whole again
    assert sorted(s.free) == list(range(s.cfg.num_blocks))
    assert all(r == 0 for r in s.ref)


@pytest.mark.parametrize("policy", ["paged", "reserve", "static"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_invariants_on_random_streams(policy, seed):
    reqs = make_request_stream(seed, 40, prompt=(1, 60), output=(1, 80), multi_frac=0.3,
                               samples=3, arrival_every=2)
    s, plans = _plans(policy, reqs)
    _check_invariants(s, plans, reqs, 8)


def test_refcounts_track_tables_every_iteration():
    reqs = make_request_stream(5, 30, prompt=(1, 40), output=(1, 50), multi_frac=0.5, samples=4,
                               arrival_every=1)
    NB = 96
    cfg = SchedConfig(num_blocks=NB, block_size=4, max_seqs=10, max_tokens=40, max_chunk=12,
                      max_len=96, policy="paged")
    s = Scheduler(cfg, np.random.default_rng(1).permutation(NB), reqs)
    evicted = 0
    n = 0
    while (p := s.step()) is not None:
        n += 1
        assert n < 20000, "the schedule does not finish"
        held = {}
        for rid in s.running:
            r = s.reqs[rid]
            tables = [r.table] if r.state == "prefill" else [q.table for q in r.samples
                                                             if not q.released]
            for t in tables:
                for b in t:
                    held[b] = held.get(b, 0) + 1
        assert all(s.ref[b] == held.get(b, 0) for b in range(NB))
        assert len(s.free) + len(held) == NB
        evicted += len(p.preempted)
        # a block written this iteration is private to its writer: a decode
        # sample's block has no other user; a prompt block is shared at most
        # by the samples of its own request (forked when the prompt completes)
        npre = sum(c[2] for c in p.chunks)
        for slot in p.slots[npre:]:
            assert s.ref[slot // 4] <= 1
        for rid, q0, L, _, _ in p.chunks:
            for slot in p.slots[q0:q0 + L]:
                assert s.ref[slot // 4] <= s.reqs[rid].n
    assert evicted > 0   # the pool is tight enough to exercise eviction


def test_paged_evicts_the_latest_admitted_request():
    # a pool too small for every prompt at once: the last admitted running
    # request is evicted, goes back to the head of the queue, and all finish
    reqs = [(9, [12], 0), (9, [12], 0), (9, [12], 0)]
    cfg = SchedConfig(num_blocks=8, block_size=4, max_seqs=3, max_tokens=30, max_chunk=9,
                      max_len=20, policy="paged")
    s = Scheduler(cfg, list(range(8)), reqs)
    plans = _run(s, limit=500)
    ev = [(p.iteration, r) for p in plans for r in p.preempted]
    assert ev, "this pool must force an eviction"
    for it, r in ev:
        running_before = [x for p in plans[:it] for x in p.admitted]
        assert r == running_before[-1] or r in running_before
    first_it, first_r = ev[0]
    admitted_so_far = [x for p in plans[:first_it] for x in p.admitted]
    assert first_r == max(admitted_so_far)
    assert sorted(x for p in plans for x in p.finished) == [0, 1, 2]


def test_reservation_copies_the_prompt_into_each_sample():
    # without paging, samples do not share: the prompt's 3 blocks are copied
    # into each further sample's reservation before its first decode
    reqs = [(10, [4, 4, 4], 0)]
    cfg = SchedConfig(num_blocks=30, block_size=4, max_seqs=3, max_tokens=30, max_chunk=16,
                      max_len=16, policy="reserve")
    s = Scheduler(cfg, list(range(30)), reqs)
    p0, p1 = s.step(), s.step()
    assert p0.copies == []
    assert p1.copies == [(0, 4), (1, 5), (2, 6), (0, 8), (1, 9), (2, 10)]
    assert [d[3] for d in p1.decodes] == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]]


def test_rejects_what_can_never_fit():
    cfg = SchedConfig(num_blocks=4, block_size=4, max_seqs=2, max_tokens=8, max_chunk=8,
                      max_len=12, policy="paged")
    with pytest.raises(ValueError):
        Scheduler(cfg, range(4), [(10, [4], 0)])         # 13 tokens > max_len
    with pytest.raises(ValueError):
        Scheduler(cfg, range(4), [(4, [1, 1, 1], 0)])   # 3 samples > 2 slots
    with pytest.raises(ValueError):
        Scheduler(cfg, [0, 1, 2, 2], [(4, [1], 0)])     # not a permutation


def test_hand_derived_swap_trace():
    # bs 4, blocks handed out 0, 1, 2, ...; six host blocks, handed out 0, 1, ...
    # Three requests, prompt 9, 12 tokens each. A and B are admitted (blocks
    # 0-2 and 3-5); C does not fit. At position 12 A takes 6 and B takes 7. At
    # position 16 (iteration 8) both need a block and none is free, so B, the
    # latest admission, is swapped out: its distinct blocks 3, 4, 5, 7 go to
    # host blocks 0..3, and A takes block 7 (released last). B cannot come
    # back while A runs (4 blocks needed, 3 free), and C waits behind it.
    # A finishes at iteration 11 (blocks 0, 1, 2, 6, 7 released in that
    # order); at iteration 12 B returns into 7, 6, 2, 1 (the stack's top),
    # keeping its 16 cached tokens, and C is admitted into 0, 5, 4. At
    # iteration 13 B writes position 16, which opens a fifth block: 3.
    cfg = SchedConfig(num_blocks=8, block_size=4, max_seqs=3, max_tokens=30, max_chunk=9,
                      max_len=20, policy="paged", num_host_blocks=6)
    s = Scheduler(cfg, list(range(8)), [(9, [12], 0), (9, [12], 0), (9, [12], 0)])
    plans = _run(s, limit=200)
    p8, p12 = plans[8], plans[12]
    assert p8.preempted == [1]
    assert p8.swap_out == [(3, 0), (4, 1), (5, 2), (7, 3)]
    assert p8.decodes == [(0, 0, 17, [0, 1, 2, 6, 7])]
    assert all(not p.admitted and not p.swap_in for p in plans[9:12])
    assert plans[11].finished == [0]
    assert p12.admitted == [1, 2]
    assert p12.swap_in == [(0, 7), (1, 6), (2, 2), (3, 1)]
    assert p12.chunks == [(2, 0, 9, 9, [0, 5, 4])]
    assert plans[13].decodes[0] == (1, 0, 17, [7, 6, 2, 1, 3])   # B resumes at position 16
    # nothing was recomputed
    assert sum(p.generated for p in plans) == 36
    assert sorted(s.host_free) == list(range(6))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_swapping_keeps_progress_and_returns_every_block(seed):
    reqs = make_request_stream(seed, 40, prompt=(1, 60), output=(1, 90), multi_frac=0.3,
                               samples=3, arrival_every=1)
    cfg = SchedConfig(num_blocks=60, block_size=8, max_seqs=12, max_tokens=64, max_chunk=32,
                      max_len=160, policy="paged", num_host_blocks=64)
    s = Scheduler(cfg, np.random.default_rng(seed).permutation(60), reqs)
    plans = _run(s)
    outs = sum(len(p.swap_out) for p in plans)
    assert outs > 0 and outs == sum(len(p.swap_in) for p in plans)
    # every decoding victim was swapped (64 host blocks hold any request), so
    # no token was generated twice (victims still in prefill restart it)
    assert sum(p.generated for p in plans) == sum(sum(o) for _, o, _ in reqs)
    # a swapped-in block receives exactly one host block, and a host block is
    # read back before it is handed out again
    held = {}
    for p in plans:
        for b, h in p.swap_out:
            assert h not in held
            held[h] = b
        for h, b in p.swap_in:
            assert h in held
            del held[h]
    assert not held
    _check_invariants(s, plans, reqs, 8)
    assert sorted(s.host_free) == list(range(64))


def test_hand_derived_prefix_cache_trace():
    # bs 4, blocks 0..9 handed out in order. A and B name prefix 0 of 9
    # tokens (two full blocks); prompts of 12, two tokens each; B arrives at
    # iteration 1. A's prefill enters blocks 0 and 1 in the cache (block 2
    # holds token 8, past the last full prefix block). B takes them as hits
    # and prefills only positions 8..11, into block 4 (3 went to A's decode).
    cfg = SchedConfig(num_blocks=10, block_size=4, max_seqs=4, max_tokens=16, max_chunk=16,
                      max_len=16, policy="paged", prefix_caching=True)
    s = Scheduler(cfg, list(range(10)), [(12, [2], 0, 0, 9), (12, [2], 1, 0, 9)])
    p0, p1, p2 = s.step(), s.step(), s.step()
    assert s.step() is None
    assert p0.chunks == [(0, 0, 12, 12, [0, 1, 2])]
    assert p1.chunks == [(1, 0, 4, 12, [0, 1, 4])]
    assert p1.slots == [16, 17, 18, 19, 12]          # B's four tokens, then A's decode
    assert p1.decodes == [(0, 0, 13, [0, 1, 2, 3])]
    assert p2.decodes == [(1, 0, 13, [0, 1, 4, 3])]
    # the cache keeps its blocks after both requests are done
    assert s.cache == {(0, 0): 0, (0, 1): 1}
    assert s.ref[0] == 1 and s.ref[1] == 1
    assert sorted(s.free + [0, 1]) == list(range(10))


def test_prefix_cache_gives_up_its_least_recently_used_block():
    # bs 2, six blocks; four one-token-output requests with 4-token prefixes
    # (two full blocks) and 5-token prompts, one per iteration, prefixes
    # 0, 1, 2, 0. R2 needs a third block when none is free: the oldest entry,
    # (0, 0) -> block 0, gives it up. R3's prefix then misses at block 0, so
    # it takes no hit and prefills all five tokens, evicting (0, 1) -> 1 and
    # (1, 0) -> 2 for its second and third blocks.
    cfg = SchedConfig(num_blocks=6, block_size=2, max_seqs=2, max_tokens=8, max_chunk=8,
                      max_len=6, policy="paged", prefix_caching=True)
    reqs = [(5, [1], 0, 0, 4), (5, [1], 1, 1, 4), (5, [1], 2, 2, 4), (5, [1], 3, 0, 4)]
    s = Scheduler(cfg, list(range(6)), reqs)
    plans = _run(s, limit=20)
    chunks = [c for p in plans for c in p.chunks]
    assert chunks == [(0, 0, 5, 5, [0, 1, 2]), (1, 0, 5, 5, [2, 3, 4]),
                      (2, 0, 5, 5, [4, 5, 0]), (3, 0, 5, 5, [0, 1, 2])]


@pytest.mark.parametrize("seed", [0, 1])
def test_prefix_caching_saves_prefill_and_keeps_the_pool_whole(seed):
    reqs = make_request_stream(seed, 60, prompt=(1, 40), output=(1, 40), multi_frac=0.2,
                               samples=2, arrival_every=2, prefix_groups=3, prefix_tokens=50)
    runs = {}
    for pc in (False, True):
        cfg = SchedConfig(num_blocks=80, block_size=8, max_seqs=10, max_tokens=64, max_chunk=32,
                          max_len=140, policy="paged", prefix_caching=pc)
        s = Scheduler(cfg, np.random.default_rng(seed).permutation(80), reqs)
        plans = _run(s)
        runs[pc] = sum(sum(c[2] for c in p.chunks) for p in plans)
        fin = sorted(r for p in plans for r in p.finished)
        assert fin == list(range(len(reqs)))
        # every block is free or held by the cache alone
        assert len(s.free) + len(s.cache) == 80
        assert all(s.ref[b] == 1 for b in s.cache.values())
        if not pc:
            _check_invariants(s, plans, reqs, 8)
    assert runs[True] < runs[False]
