"""Input generator and host block manager (CPU only)."""
import hashlib

import numpy as np
import pytest

from workloads import BlockManager, PoolExhausted, make_workload
from workloads.rng import f32_to_bf16_bits, normal_values


def _digest(w):
    h = hashlib.sha256()
    for a in (w.pool, w.q, w.block_tables, w.context_lens, w.slot_mapping, w.k_new, w.v_new,
              w.copy_pairs):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_generation_is_deterministic():
    a = make_workload("mha", num_seqs=5, max_len=300)
    b = make_workload("mha", num_seqs=5, max_len=300)
    c = make_workload("mha", num_seqs=5, max_len=300, seed=99)
    assert _digest(a) == _digest(b) != _digest(c)


def test_chunked_draws_do_not_depend_on_thread_count(monkeypatch):
    import workloads.rng as r
    ss = np.random.SeedSequence(5)
    a = normal_values(ss, 3 * r.CHUNK + 17, "bf16")
    monkeypatch.setattr(r, "_threads", lambda: 1)
    b = normal_values(np.random.SeedSequence(5), 3 * r.CHUNK + 17, "bf16")
    assert np.array_equal(a, b)


def test_bf16_encoding_rounds_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.0, np.nan, 3.0e38, 1.0 + 2 ** -9], np.float32)
    # 1 + 2^-8 is a tie between 1 and 1+2^-7 -> even (1.0); 1 + 3*2^-8 ties up to 1 + 2^-6
    want = np.array([0x3F80, 0x3F80, 0x3F82, 0xC000, 0x7FC0, 0x7F62, 0x3F80], np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), want)


def test_tiny_matches_its_description():
    w = make_workload("tiny")
    assert list(w.context_lens) == [6, 18, 34, 65]
    assert w.num_blocks == 33 and w.poison_block == 32
    assert w.dtype == "f32" and w.scale == 0.125
    # sequence 3 caches 64 tokens in 4 blocks and takes a fifth for the appended token
    assert w.block_tables.shape == (4, 5)
    assert (w.block_tables[3] != 32).all()
    assert w.slot_mapping[3] == w.block_tables[3, 4] * 16
    assert np.isnan(w.pool[32]).all()


def test_unused_slots_are_poison():
    w = make_workload("gqa", num_seqs=8, median=40, hi=100, num_q_heads=4, num_kv_heads=2,
                      head_dim=8)
    nan = np.uint16(0x7FC0)
    used = set()
    for b in range(w.num_seqs):
        n = int(w.context_lens[b]) - 1  # cached before the append
        for j in range(-(-n // w.block_size)):
            used.add(int(w.block_tables[b, j]))
    for j in range(w.num_blocks):
        if j not in used:
            assert (w.pool[j] == nan).all()
    # the appended token's slot is poison before the append
    kview = w.pool.reshape(w.num_blocks, 2, 2, 1, w.block_size, 8)[:, 0]  # d = 8: one slice
    for s in w.slot_mapping:
        assert (kview[s // w.block_size, :, :, s % w.block_size] == nan).all()


def test_prefix_config_shares_and_copies():
    w = make_workload("prefix")
    assert w.num_seqs == 256
    assert w.copy_pairs.shape == (224, 2)  # 7 copies for each of 32 prompts
    # before the step every sample of a prompt points at the same 65 blocks
    assert (w.context_lens >= 1033).all() and (w.context_lens <= 1544).all()
    srcs = w.copy_pairs[:, 0]
    assert len(set(srcs.tolist())) == 32
    dsts = w.copy_pairs[:, 1]
    assert len(set(dsts.tolist())) == 224 and not set(dsts.tolist()) & set(srcs.tolist())
    # the literal 1024-token prefix fills 64 blocks exactly: nothing to copy
    w2 = make_workload("prefix", prefix_len=1024, num_prompts=2)
    assert w2.copy_pairs.shape == (0, 2)


def test_mixed_config_counts():
    w = make_workload("mixed")
    assert w.slot_mapping.shape == (16 * 512 + 240,)
    assert w.meta["prior"][0] == 0 and w.meta["prior"][1] == 2048
    assert list(w.query_start_loc) == [512 * i for i in range(17)]
    assert len(set(w.slot_mapping.tolist())) == w.slot_mapping.size


def test_block_manager_allocate_on_fill_and_free():
    bm = BlockManager(8, 4, np.random.default_rng(0))
    bm.add_sequence("a", 4)
    assert len(bm.tables["a"]) == 1
    s = bm.append_slot("a")  # position 4 needs a second block
    assert len(bm.tables["a"]) == 2 and s == bm.tables["a"][1] * 4
    for _ in range(3):
        bm.append_slot("a")
    assert len(bm.tables["a"]) == 2
    bm.check()
    bm.free_sequence("a")
    assert bm.num_free() == 8
    bm.check()


def test_block_manager_copy_on_write_and_refcounts():
    bm = BlockManager(16, 4, np.random.default_rng(1))
    bm.add_sequence("p", 6)          # blocks: full + half
    for i in range(3):
        bm.fork("p", i)
    bm.free_sequence("p")
    shared = bm.tables[0][1]
    assert bm.refcount[shared] == 3
    bm.append_slot(0)
    bm.append_slot(1)
    bm.append_slot(2)                # last sharer writes in place
    pairs = bm.take_copy_pairs()
    assert pairs.shape == (2, 2) and (pairs[:, 0] == shared).all()
    assert bm.tables[2][1] == shared and bm.refcount[shared] == 1
    bm.check()


def test_block_manager_refuses_when_exhausted():
    bm = BlockManager(2, 4, np.random.default_rng(2))
    bm.add_sequence("a", 8)
    with pytest.raises(PoolExhausted):
        bm.append_slot("a")
    with pytest.raises(PoolExhausted):
        bm.add_sequence("b", 1)
