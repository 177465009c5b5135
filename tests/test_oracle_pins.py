"""Pins of the fp64 oracle against facts other than itself (CPU only).

Each test names the oracle function it pins and the kind of fact it uses:
hand-derived examples, closed forms, a library routine on contiguous inputs,
invariants, and the independent pure-Python brute force.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import oracle.brute as brute
from tests.pool_writer import contiguous_pool, empty_pool, put_token, unshare_blocks
from workloads import build_decode_workload, make_workload

HERE = os.path.dirname(os.path.abspath(__file__))


def _decode(w, pool=None, q=None, tables=None, lens=None, scale=None):
    return oracle.decode(w.q if q is None else q, w.pool if pool is None else pool,
                         w.block_tables if tables is None else tables,
                         w.context_lens if lens is None else lens,
                         w.num_kv_heads, w.block_size, w.scale if scale is None else scale,
                         w.dtype)


def _appended(w):
    return oracle.append(w.pool, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads,
                         w.block_size, w.head_dim)


# -- golden hand-derived cases ----------------------------------------------------

def _golden_cases():
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_hand_worked(case):
    """decode / prefill / gather against hand-derived outputs."""
    Hkv, bs, d = case["num_kv_heads"], case["block_size"], case["head_dim"]
    pool = empty_pool(case["num_blocks"], Hkv, bs, d, np.float32)
    tables, lens = [], []
    for seq in case["sequences"]:
        for t, (blk, slot) in enumerate(seq["placement"]):
            # placement must be what the table implies for logical token t
            assert seq["table"][t // bs] == blk and t % bs == slot
            pad = lambda h: [np.nan if x is None else x for x in h] + [0.0] * (d - len(h))  # noqa: E731
            kk = [pad(h) for h in seq["k"][t]]
            vv = [pad(h) for h in seq["v"][t]]
            put_token(pool, blk, slot, kk, vv, Hkv, bs, d)
        tables.append(seq["table"])
        lens.append(len(seq["placement"]))
    width = max(len(t) for t in tables)
    tab = np.array([t + [0] * (width - len(t)) for t in tables], np.int32)
    q = np.array([[h + [0.0] * (d - len(h)) for h in row] for row in case["q"]], np.float32)
    if case["kind"] == "decode":
        out = oracle.decode(q, pool, tab, np.array(lens), Hkv, bs, case["scale"], "f32")
    else:
        L = case["sequences"][0]["chunk_len"]
        out = oracle.prefill(q, pool, tab, np.array(lens), np.array([0, L]), Hkv, bs,
                             case["scale"], "f32")
    exp = np.array(case["expected"], np.float64)
    assert np.abs(out - exp).max() <= case["tol"], (out, exp)


# -- element decoding ------------------------------------------------------------

def test_bf16_decoding_known_values():
    """decode_elements: bfloat16 bit patterns with textbook values."""
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F80, 0x0001, 0x4049], np.uint16)
    want = [1.0, -2.0, 1.0078125, 0.0, -0.0, math.inf, 2.0 ** -133, 3.140625]
    got = oracle.decode_elements(bits, "bf16")
    assert list(got) == want
    assert math.copysign(1.0, got[4]) == -1.0


# -- Q1 / Q2: append and copy, bitwise ------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "prefix_small"])
def test_append_bitwise_against_brute(name):
    """O4 append: bit-equal to the flat-index brute force; untouched bytes unchanged."""
    if name == "tiny":
        w = make_workload("tiny")
    else:
        w = make_workload("prefix", num_prompts=2, samples=3, prefix_len=21, max_suffix=9,
                          num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4)
    a = _appended(w)
    b = brute.append(w.pool, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads,
                     w.block_size, w.head_dim)
    view = np.uint32 if w.dtype == "f32" else np.uint16
    assert np.array_equal(a.view(view), b.view(view))
    # every element outside the written slots keeps its bits (NaN poison included)
    touched = np.zeros(w.pool.shape, bool)
    kv, vv = oracle.pool_views(touched, w.num_kv_heads, w.block_size, w.head_dim)
    for s in w.slot_mapping:
        off = s % w.block_size
        kv[s // w.block_size, :, :, off, :] = True
        vv[s // w.block_size, :, off // 4, :, off % 4] = True
    assert np.array_equal(a.view(view)[~touched], w.pool.view(view)[~touched])
    assert touched.sum() == len(w.slot_mapping) * 2 * w.num_kv_heads * w.head_dim


def test_append_skips_negative_slots():
    w = make_workload("tiny")
    sm = w.slot_mapping.copy()
    sm[1] = -1
    a = oracle.append(w.pool, w.k_new, w.v_new, sm, w.num_kv_heads, w.block_size, w.head_dim)
    b = brute.append(w.pool, w.k_new, w.v_new, sm, w.num_kv_heads, w.block_size, w.head_dim)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_append_places_token_where_gather_reads_it():
    """After append, gathering position n-1 returns exactly the appended rows."""
    w = make_workload("tiny")
    a = _appended(w)
    for i, (kind, row, pos) in enumerate(w.append_owner):
        for g in range(w.num_kv_heads):
            K, V = oracle.gather(a, w.dtype, w.block_tables[row], pos + 1, g, w.num_kv_heads,
                                 w.block_size, w.head_dim)
            assert np.array_equal(K[pos], w.k_new[i, g].astype(np.float64))
            assert np.array_equal(V[pos], w.v_new[i, g].astype(np.float64))


def test_slots_consistent_with_tables():
    """check_slots accepts the generator's slots and rejects a corrupted one."""
    for w in (make_workload("tiny"),
              make_workload("prefix", num_prompts=2, samples=3, prefix_len=21, max_suffix=9,
                            num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4)):
        oracle.check_slots(w.slot_mapping, w.append_owner, w.block_tables, w.block_size)
        bad = w.slot_mapping.copy()
        bad[0] += 1
        with pytest.raises(AssertionError):
            oracle.check_slots(bad, w.append_owner, w.block_tables, w.block_size)


def test_copy_blocks_snapshot_semantics():
    """O5 copy: dst equals src as it was before the call; other blocks unchanged."""
    w = make_workload("prefix", num_prompts=2, samples=3, prefix_len=21, max_suffix=9,
                      num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4)
    assert w.copy_pairs.shape[0] == 2 * 2  # all but the last sharer copy
    c = oracle.copy_blocks(w.pool, w.copy_pairs)
    b = brute.copy_blocks(w.pool, w.copy_pairs)
    assert np.array_equal(c.view(np.uint16), b.view(np.uint16))
    dst = set(int(x) for x in w.copy_pairs[:, 1])
    for src, d in w.copy_pairs:
        assert np.array_equal(c[d].view(np.uint16), w.pool[src].view(np.uint16))
    for j in range(w.pool.shape[0]):
        if j not in dst:
            assert np.array_equal(c[j].view(np.uint16), w.pool[j].view(np.uint16))
    # swapping two blocks in one call reads the pre-call state of both
    x, y = int(w.block_tables[0, 0]), int(w.block_tables[-1, 0])
    assert not np.array_equal(w.pool[x].view(np.uint16), w.pool[y].view(np.uint16))
    sw = oracle.copy_blocks(w.pool, np.array([[x, y], [y, x]]))
    assert np.array_equal(sw[x].view(np.uint16), w.pool[y].view(np.uint16))
    assert np.array_equal(sw[y].view(np.uint16), w.pool[x].view(np.uint16))


def test_swap_blocks_moves_whole_blocks_and_round_trips():
    """Swap out copies device blocks to host blocks flat index by flat index;
    swapping back with the pairs reversed restores the pool exactly; blocks
    no pair names are untouched on both sides."""
    w = make_workload("tiny")
    rng = np.random.default_rng(8)
    nh = 6
    host = np.full((nh, w.pool.shape[1]), np.nan, np.float32)
    src = rng.choice(w.pool.shape[0] - 1, 4, replace=False)
    dst = rng.choice(nh, 4, replace=False)
    pairs = np.stack([src, dst], 1)
    pool2, host2 = oracle.swap_blocks(w.pool, host, pairs, 0)
    assert np.array_equal(pool2.view(np.uint32), w.pool.view(np.uint32))
    E = w.pool.shape[1]
    flat_pool, flat_host = list(w.pool.reshape(-1)), host.reshape(-1).copy()
    for s_, d_ in pairs:   # element by element, by flat index
        for e in range(E):
            flat_host[d_ * E + e] = flat_pool[s_ * E + e]
    assert np.array_equal(host2.reshape(-1).view(np.uint32), flat_host.view(np.uint32))
    untouched = [j for j in range(nh) if j not in set(dst.tolist())]
    assert np.isnan(host2[untouched]).all()
    # back in, into blocks cleared to zero first
    cleared = w.pool.copy()
    cleared[src] = 0.0
    pool3, host3 = oracle.swap_blocks(cleared, host2, pairs[:, ::-1], 1)
    assert np.array_equal(pool3.view(np.uint32), w.pool.view(np.uint32))
    assert np.array_equal(host3.view(np.uint32), host2.view(np.uint32))


# -- Q3, Q4: closed forms --------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_context_returns_v_exactly(dtype):
    """Q3: with one key the softmax weight is exactly 1, so o = V[0] exactly."""
    w = build_decode_workload("one", 7, [1] * 5, 4, 2, 16, 16, dtype, scale=0.25)
    a = _appended(w)
    out = _decode(w, pool=a)
    G = w.num_q_heads // w.num_kv_heads
    for b in range(w.num_seqs):
        for h in range(w.num_q_heads):
            want = oracle.decode_elements(w.v_new[b, h // G], dtype)
            assert np.array_equal(out[b, h], want)


def test_uniform_scores_give_mean_of_v():
    """Q4: q = 0 or identical keys make the softmax uniform: o = mean of V rows."""
    w = build_decode_workload("u", 11, [3, 16, 17, 40], 2, 2, 8, 4, "f32")
    a = _appended(w)
    zero_q = np.zeros_like(w.q)
    out = _decode(w, pool=a, q=zero_q)
    for b in range(w.num_seqs):
        n = int(w.context_lens[b])
        for h in range(2):
            _, V = oracle.gather(a, "f32", w.block_tables[b], n, h, 2, 4, 8)
            want = [math.fsum(V[:, i]) / n for i in range(8)]
            assert np.allclose(out[b, h], want, rtol=1e-15, atol=1e-15)
    # identical keys: a contiguous pool whose K rows are all equal
    rng = np.random.default_rng(3)
    n, d = 23, 8
    K = [np.repeat(rng.standard_normal((1, 1, d)), n, axis=0)]
    V = [rng.standard_normal((n, 1, d))]
    pool, tables = contiguous_pool(K, V, 4)
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    out = oracle.decode(q, pool, tables, np.array([n]), 1, 4, 0.3, "f32")
    want = [math.fsum(np.float32(V[0][:, 0, i]).astype(np.float64)) / n for i in range(d)]
    assert np.allclose(out[0, 0], want, rtol=1e-14, atol=1e-15)


# -- Q5, Q6: placement invariants -------------------------------------------------

def test_physical_block_permutation_invariance():
    """Q5: relabelling physical blocks (and the tables) leaves the output unchanged."""
    w = make_workload("mha", num_seqs=6, min_len=5, max_len=70, num_heads=2, head_dim=16)
    a = _appended(w)
    base = _decode(w, pool=a)
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    new_pool = np.empty_like(a)
    new_pool[perm] = a
    new_tables = perm[w.block_tables].astype(np.int32)
    out = _decode(w, pool=new_pool, tables=new_tables)
    assert np.array_equal(out, base)


def test_shared_prefix_equals_duplicated_prefix():
    """Q6: sequences pointing at one shared block == each owning a byte-equal copy."""
    w = make_workload("prefix", num_prompts=2, samples=4, prefix_len=21, max_suffix=11,
                      num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4)
    assert w.copy_pairs.shape[0] == 2 * 3
    p = oracle.copy_blocks(w.pool, w.copy_pairs)
    p = oracle.append(p, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads, w.block_size,
                      w.head_dim)
    shared = _decode(w, pool=p)
    p2, t2 = unshare_blocks(p, w.block_tables, w.context_lens, w.block_size, w.poison_block)
    assert p2.shape[0] > p.shape[0]  # the prefix really was shared
    dup = _decode(w, pool=p2, tables=t2)
    assert np.array_equal(shared, dup)


# -- Q7: library special case ---------------------------------------------------

def _sdpa(q, k, v, scale, causal=False):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale,
        is_causal=causal).numpy()


def test_contiguous_table_matches_library_attention():
    """Q7: identity tables reduce the oracle to torch SDPA (float64, CPU)."""
    rng = np.random.default_rng(9)
    lens = [1, 7, 16, 33, 50]
    Hkv, G, d, bs = 2, 3, 16, 8
    K = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in lens]
    V = [rng.standard_normal((n, Hkv, d)).astype(np.float32) for n in lens]
    q = rng.standard_normal((len(lens), Hkv * G, d)).astype(np.float32)
    pool, tables = contiguous_pool(K, V, bs)
    scale = float(np.float32(1 / math.sqrt(d)))
    out = oracle.decode(q, pool, tables, np.array(lens), Hkv, bs, scale, "f32")
    for b, n in enumerate(lens):
        kk = np.repeat(K[b].astype(np.float64).transpose(1, 0, 2), G, axis=0)  # [Hq][n][d]
        vv = np.repeat(V[b].astype(np.float64).transpose(1, 0, 2), G, axis=0)
        qq = q[b].astype(np.float64)[:, None, :]                               # [Hq][1][d]
        ref = _sdpa(qq, kk, vv, scale)[:, 0, :]
        assert np.abs(out[b] - ref).max() < 1e-13


def test_prefill_prior0_matches_causal_library_attention():
    """Q11 (second half): a chunk with no cached prefix is causal SDPA."""
    rng = np.random.default_rng(10)
    L, Hkv, G, d, bs = 19, 2, 2, 8, 4
    K = [rng.standard_normal((L, Hkv, d)).astype(np.float32)]
    V = [rng.standard_normal((L, Hkv, d)).astype(np.float32)]
    pool, tables = contiguous_pool(K, V, bs)
    q = rng.standard_normal((L, Hkv * G, d)).astype(np.float32)
    out = oracle.prefill(q, pool, tables, np.array([L]), np.array([0, L]), Hkv, bs, 0.3, "f32")
    kk = np.repeat(K[0].astype(np.float64).transpose(1, 0, 2), G, axis=0)
    vv = np.repeat(V[0].astype(np.float64).transpose(1, 0, 2), G, axis=0)
    qq = q.astype(np.float64).transpose(1, 0, 2)
    ref = _sdpa(qq, kk, vv, float(np.float32(0.3)), causal=True).transpose(1, 0, 2)
    assert np.abs(out - ref).max() < 1e-13


def test_prefill_chunk_of_one_equals_decode():
    """Q11 (first half): a one-query chunk is a decode step at the last position."""
    w = make_workload("mixed", num_decode=3, dec_min=5, dec_max=40, num_chunks=3, chunk_len=1,
                      max_prior=30, num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4)
    a = _appended(w)
    pre = oracle.prefill(w.prefill_q, a, w.prefill_block_tables, w.prefill_context_lens,
                         w.query_start_loc, w.num_kv_heads, w.block_size, w.scale, w.dtype)
    dec = oracle.decode(w.prefill_q, a, w.prefill_block_tables, w.prefill_context_lens,
                        w.num_kv_heads, w.block_size, w.scale, w.dtype)
    assert np.array_equal(pre, dec)


# -- Q8: GQA = MHA with repeated heads ---------------------------------------------

def test_gqa_equals_mha_with_repeated_kv_heads():
    w = make_workload("gqa", num_seqs=5, median=30, hi=90, num_q_heads=8, num_kv_heads=2,
                      head_dim=8, dtype="f32")
    a = _appended(w)
    out = _decode(w, pool=a)
    G = 4
    nb = a.shape[0]
    halves = a.reshape(nb, 2, w.num_kv_heads, w.block_size * w.head_dim)
    rep = np.repeat(halves, G, axis=2).reshape(nb, -1)  # kv head h // G -> head h
    mha = oracle.decode(w.q, rep, w.block_tables, w.context_lens, 8, w.block_size, w.scale, "f32")
    assert np.array_equal(out, mha)


# -- Q9: batch invariance ----------------------------------------------------------

def test_batch_composition_does_not_change_a_sequence():
    w = make_workload("mha", num_seqs=6, min_len=5, max_len=70, num_heads=2, head_dim=16)
    a = _appended(w)
    full = _decode(w, pool=a)
    order = [4, 1, 5]
    sub = _decode(w, pool=a, q=w.q[order], tables=w.block_tables[order],
                  lens=w.context_lens[order])
    assert np.array_equal(sub, full[order])


# -- Q10: split-K identity -----------------------------------------------------------

@pytest.mark.parametrize("cuts_kind", ["even", "ragged", "with_empty", "single"])
def test_split_k_merge_identity(cuts_kind):
    rng = np.random.default_rng(12)
    n, d = 300, 16
    K = rng.standard_normal((n, d)) * 3
    V = rng.standard_normal((n, d))
    q = rng.standard_normal(d)
    cuts = {"even": [0, 100, 200, 300], "ragged": [0, 7, 8, 150, 299, 300],
            "with_empty": [0, 50, 50, 300, 300], "single": [0, 300]}[cuts_kind]
    whole = oracle.attend(q, K, V, 0.7)
    merged = oracle.merge_partials(oracle.attend_partitioned(q, K, V, 0.7, cuts))
    assert np.abs(whole - merged).max() <= 1e-12 * max(1.0, np.abs(whole).max())


def test_merge_of_all_empty_parts_is_zero():
    parts = [(-np.inf, 0.0, np.zeros(4)), (-np.inf, 0.0, np.zeros(4))]
    assert np.array_equal(oracle.merge_partials(parts), np.zeros(4))


# -- Q12: brute force ---------------------------------------------------------------

@pytest.mark.parametrize("seed", range(6))
def test_decode_matches_brute_force_on_tiny_random(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 5))
    bs = int(rng.choice([4, 8, 16]))
    d = int(rng.choice([8, 16]))
    Hkv = int(rng.choice([1, 2]))
    G = int(rng.choice([1, 2]))
    lens = rng.integers(1, 41, size=B)
    dtype = "bf16" if seed % 2 else "f32"
    w = build_decode_workload("r", 200 + seed, lens, Hkv * G, Hkv, d, bs, dtype,
                              scale=float(rng.uniform(0.1, 1.0)))
    a = _appended(w)
    o = _decode(w, pool=a)
    ob = np.array(brute.decode(w.q, a, w.block_tables, w.context_lens, Hkv, bs, w.scale, dtype))
    assert np.abs(o - ob).max() <= 1e-12


def test_decode_matches_brute_force_on_tiny_config():
    w = make_workload("tiny")
    a = _appended(w)
    o = _decode(w, pool=a)
    ob = np.array(brute.decode(w.q, a, w.block_tables, w.context_lens, w.num_kv_heads,
                               w.block_size, w.scale, w.dtype))
    assert np.abs(o - ob).max() <= 1e-12
    assert not np.isnan(o).any()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_matches_brute_force(dtype):
    w = make_workload("mixed", num_decode=2, dec_min=3, dec_max=20, num_chunks=3, chunk_len=5,
                      max_prior=11, num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=4,
                      dtype=dtype)
    a = _appended(w)
    o = oracle.prefill(w.prefill_q, a, w.prefill_block_tables, w.prefill_context_lens,
                       w.query_start_loc, 2, 4, w.scale, dtype)
    ob = np.array(brute.prefill(w.prefill_q, a, w.prefill_block_tables, w.prefill_context_lens,
                                w.query_start_loc, 2, 4, w.scale, dtype))
    assert np.abs(o - ob).max() <= 1e-12
    assert not np.isnan(o).any()


# -- Q13, Q14 ----------------------------------------------------------------------

def test_output_is_a_convex_combination_of_v():
    w = make_workload("gqa", num_seqs=6, median=40, hi=120, num_q_heads=4, num_kv_heads=2,
                      head_dim=8)
    a = _appended(w)
    out = _decode(w, pool=a)
    for b in range(w.num_seqs):
        for h in range(4):
            _, V = oracle.gather(a, w.dtype, w.block_tables[b], int(w.context_lens[b]), h // 2,
                                 2, w.block_size, 8)
            assert (out[b, h] >= V.min(0) - 1e-12).all() and (out[b, h] <= V.max(0) + 1e-12).all()


def test_scale_equivariance():
    w = build_decode_workload("s", 21, [9, 30, 64], 2, 1, 8, 4, "f32", scale=0.5)
    a = _appended(w)
    base = _decode(w, pool=a)
    q3 = (w.q.astype(np.float64) * 3).astype(np.float32)  # exact: small ints * 3 may round
    exact = np.array_equal(q3.astype(np.float64), w.q.astype(np.float64) * 3)
    out = _decode(w, pool=a, q=q3, scale=float(np.float32(0.5 / 3)))
    tol = 1e-12 if exact else 1e-6
    assert np.abs(out - base).max() <= tol


def test_decode_of_empty_context_is_zero():
    w = build_decode_workload("z", 1, [4, 9], 2, 2, 8, 4, "f32")
    a = _appended(w)
    out = _decode(w, pool=a, lens=np.array([0, 9], np.int32))
    assert np.array_equal(out[0], np.zeros((2, 8)))
    assert not np.isnan(out[1]).any()


# -- weight moments (they size the bf16 error bound of the GPU tests) -------------

def test_moments_of_one_key_are_v_and_zero():
    """softmax_moments: a single key has weight exactly 1, so E|V| = |V0| and
    E|V - o| = 0 (closed form)."""
    V = np.array([[-1.5, 0.25, 3.0]])
    K = np.array([[0.3, -0.2, 0.9]])
    o, ma, md = oracle.softmax_moments(np.array([1.0, 2.0, -1.0]), K, V, 0.7)
    assert np.array_equal(o, V[0]) and np.array_equal(ma, np.abs(V[0]))
    assert np.array_equal(md, np.zeros(3))


def test_moments_of_uniform_weights_are_plain_means():
    """softmax_moments: q = 0 makes every weight 1/n, so the moments are the
    plain means of |V| and of |V - mean V| (math.fsum, per dimension)."""
    rng = np.random.default_rng(17)
    n, d = 13, 5
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    o, ma, md = oracle.softmax_moments(np.zeros(d), K, V, 0.5)
    for i in range(d):
        mean = math.fsum(V[:, i]) / n
        assert math.isclose(o[i], mean, rel_tol=1e-14, abs_tol=1e-15)
        assert math.isclose(ma[i], math.fsum(abs(x) for x in V[:, i]) / n, rel_tol=1e-14)
        assert math.isclose(md[i], math.fsum(abs(x - mean) for x in V[:, i]) / n,
                            rel_tol=1e-12, abs_tol=1e-15)


def test_moments_of_two_keys_follow_the_logistic_weight():
    """softmax_moments: with two keys whose scores differ by D the weights are
    1/(1 + e^-D) and 1/(1 + e^D) (closed form), so with V = (a, b) in one
    dimension E|V| = w0|a| + w1|b| and E|V - o| = 2 w0 w1 |a - b|."""
    a, b, D = 2.0, -3.0, 1.3
    K = np.array([[D], [0.0]])
    V = np.array([[a], [b]])
    o, ma, md = oracle.softmax_moments(np.array([1.0]), K, V, 1.0)
    w0 = 1.0 / (1.0 + math.exp(-D))
    w1 = 1.0 - w0
    assert math.isclose(o[0], w0 * a + w1 * b, rel_tol=1e-14)
    assert math.isclose(ma[0], w0 * abs(a) + w1 * abs(b), rel_tol=1e-14)
    assert math.isclose(md[0], 2 * w0 * w1 * abs(a - b), rel_tol=1e-13)


def test_decode_and_prefill_moments_carry_the_oracle_outputs():
    """decode_moments / prefill_moments gather exactly like decode / prefill:
    their o equals the oracle's outputs (up to summation order), and the
    moments satisfy
    |o| <= E|V| and E|V - o| <= E|V| + |o| (triangle inequality)."""
    w = make_workload("mixed", num_decode=3, dec_min=1, dec_max=200, num_chunks=2, chunk_len=20,
                      max_prior=60, num_q_heads=4, num_kv_heads=2, head_dim=16, dtype="f32")
    p = oracle.append(w.pool, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads, w.block_size,
                      w.head_dim)
    o, ma, md = oracle.decode_moments(w.q, p, w.block_tables, w.context_lens, w.num_kv_heads,
                                      w.block_size, w.scale, w.dtype)
    want = oracle.decode(w.q, p, w.block_tables, w.context_lens, w.num_kv_heads, w.block_size,
                         w.scale, w.dtype)
    assert np.allclose(o, want, rtol=1e-13, atol=1e-15)
    assert (np.abs(o) <= ma + 1e-12).all() and (md <= ma + np.abs(o) + 1e-12).all()
    o2, ma2, md2 = oracle.prefill_moments(w.prefill_q, p, w.prefill_block_tables,
                                          w.prefill_context_lens, w.query_start_loc,
                                          w.num_kv_heads, w.block_size, w.scale, w.dtype)
    want = oracle.prefill(w.prefill_q, p, w.prefill_block_tables, w.prefill_context_lens,
                          w.query_start_loc, w.num_kv_heads, w.block_size, w.scale, w.dtype)
    assert np.allclose(o2, want, rtol=1e-13, atol=1e-15)
    assert (np.abs(o2) <= ma2 + 1e-12).all() and (md2 <= ma2 + np.abs(o2) + 1e-12).all()
