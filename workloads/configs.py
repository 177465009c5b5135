"""The five synthetic workloads, as seeded recipes.

Shapes and value distributions follow the workload descriptions of the
paged-decode benchmark this library is measured on (tiny decode, MHA decode,
GQA long-tail decode, shared-prefix parallel sampling, mixed continuous-batching
iteration). Ragged, long-tailed lengths and shared prompt prefixes stand in for
the serving traces the pages describe ("Paging the KV Cache", section "The waste
hiding inside memory"; the continuous-batching post, section "What this is
worth, measured": output lengths that spread widely, capped at 1536 tokens).

Storage format written here (the library's documented pool layout): the pool is
``num_blocks`` blocks; block ``j`` holds ``2 * Hkv * bs * d`` elements, first the
K half laid out ``[Hkv][d/8][bs][8]`` (8-element slices of a token's vector),
then the V half laid out ``[Hkv][bs/4][d][4]`` (4-token slices of each
dimension). Block ``num_blocks - 1`` is a poison block filled with NaN; every
table entry past a sequence's last block points at it, and every slot that
holds no cached token is NaN too, so a read outside a context is visible.

Draw order: ``SeedSequence(seed).spawn(8)`` gives independent streams for
[0] lengths and structure, [1] the free-list permutation, [2] pool values,
[3] decode queries, [4] appended K, [5] appended V, [6] prefill queries.
All values are N(0, 1) drawn in float32; bf16 storage rounds each draw once
(nearest, ties to even).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .block_manager import BlockManager
from .rng import element_bytes, nan_value, normal_values, storage_dtype

CONFIG_NAMES = ("tiny", "mha", "gqa", "prefix", "mixed")


@dataclass
class Workload:
    name: str
    dtype: str                   # "f32" or "bf16"
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int              # including the poison block (the last id)
    pool: np.ndarray             # [num_blocks, 2*Hkv*bs*d] storage elements
    scale: float                 # a float32 value, passed as float
    # step phase 1: copy-on-write block copies
    copy_pairs: np.ndarray       # [P, 2] int32 (src, dst)
    # step phase 2: KV append
    slot_mapping: np.ndarray     # [T] int32
    k_new: np.ndarray            # [T, Hkv, d]
    v_new: np.ndarray            # [T, Hkv, d]
    append_owner: np.ndarray     # [T, 3] int32: (0 decode / 1 prefill, table row, position)
    # step phase 3: decode
    q: np.ndarray                # [B, Hq, d]
    block_tables: np.ndarray     # [B, MB] int32
    context_lens: np.ndarray     # [B] int32 (includes the appended token)
    # step phase 4 (mixed iteration only): chunked prefill
    prefill_q: np.ndarray | None = None            # [sum L, Hq, d]
    prefill_block_tables: np.ndarray | None = None  # [C, MBp] int32
    prefill_context_lens: np.ndarray | None = None  # [C] int32 (prior + chunk)
    query_start_loc: np.ndarray | None = None       # [C+1] int32
    meta: dict = field(default_factory=dict)

    @property
    def poison_block(self) -> int:
        return self.num_blocks - 1

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def elem_bytes(self) -> int:
        return element_bytes(self.dtype)

    @property
    def block_elems(self) -> int:
        return 2 * self.num_kv_heads * self.block_size * self.head_dim

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


def _split_seeds(seed: int):
    return np.random.SeedSequence(seed).spawn(8)


def _make_pool(ss, nb_total: int, hkv: int, bs: int, d: int, dtype: str,
               valid: np.ndarray) -> np.ndarray:
    """Draw every element, then overwrite non-cached slots with NaN.

    ``valid[j, s]`` says whether slot ``s`` of block ``j`` holds a cached token.
    """
    per_block = 2 * hkv * bs * d
    pool = normal_values(ss, nb_total * per_block, dtype).reshape(nb_total, per_block)
    halves = pool.reshape(nb_total, 2, hkv * bs * d)
    # K: [j][h][i/8][s][i%8] -> [j][s][h][i/8][i%8]
    k_view = halves[:, 0].reshape(nb_total, hkv, d // 8, bs, 8).transpose(0, 3, 1, 2, 4)
    # V: [j][h][s/4][i][s%4] -> [j][s/4][s%4][h][i]
    v_view = halves[:, 1].reshape(nb_total, hkv, bs // 4, d, 4).transpose(0, 2, 4, 1, 3)
    bad = ~valid
    k_view[bad] = nan_value(dtype)
    v_view[bad.reshape(nb_total, bs // 4, 4)] = nan_value(dtype)
    return pool


def _valid_mask(bm: BlockManager, nb_total: int) -> np.ndarray:
    valid = np.zeros((nb_total, bm.block_size), bool)
    for seq, table in bm.tables.items():
        n = bm.lens[seq]
        for t in range(0, n, bm.block_size):
            blk = table[t // bm.block_size]
            valid[blk, : min(bm.block_size, n - t)] = True
    return valid


def _blocks_for(n: int, bs: int) -> int:
    return -(-int(n) // bs)


def _pool_blocks(needed: int, factor: float = 1.25) -> int:
    return max(1, math.ceil(factor * needed))


def build_decode_workload(name: str, seed: int, lens_post, num_q_heads: int,
                          num_kv_heads: int, head_dim: int, block_size: int,
                          dtype: str, num_blocks: int | None = None,
                          pool_factor: float = 1.25, scale: float | None = None,
                          meta: dict | None = None) -> Workload:
    """A decode iteration: each sequence caches ``n - 1`` tokens, appends one, attends to ``n``.

    ``lens_post`` are the context lengths the decode attends to (>= 1), i.e.
    after the append. ``num_blocks`` (excluding the poison block) defaults to
    ``ceil(pool_factor * blocks needed after the append)``.
    """
    ss = _split_seeds(seed)
    lens_post = np.asarray(lens_post, np.int64)
    if lens_post.ndim != 1 or (lens_post < 1).any():
        raise ValueError("decode context lengths must be >= 1")
    B = lens_post.size
    needed = int(sum(_blocks_for(n, block_size) for n in lens_post))
    nb = _pool_blocks(needed, pool_factor) if num_blocks is None else int(num_blocks)
    bm = BlockManager(nb, block_size, np.random.default_rng(ss[1]))
    for b in range(B):
        bm.add_sequence(b, int(lens_post[b]) - 1)
    nb_total = nb + 1
    poison = nb
    pool = _make_pool(ss[2], nb_total, num_kv_heads, block_size, head_dim, dtype,
                      _valid_mask(bm, nb_total))
    slots = np.array([bm.append_slot(b) for b in range(B)], np.int32)
    owner = np.stack([np.zeros(B, np.int64), np.arange(B), lens_post - 1], 1).astype(np.int32)
    pairs = bm.take_copy_pairs()
    assert pairs.shape[0] == 0
    bm.check()
    tables = bm.table_array(range(B), poison)
    q = normal_values(ss[3], B * num_q_heads * head_dim, dtype).reshape(B, num_q_heads, head_dim)
    kn = normal_values(ss[4], B * num_kv_heads * head_dim, dtype).reshape(B, num_kv_heads, head_dim)
    vn = normal_values(ss[5], B * num_kv_heads * head_dim, dtype).reshape(B, num_kv_heads, head_dim)
    sc = float(np.float32(1.0 / math.sqrt(head_dim))) if scale is None else float(np.float32(scale))
    return Workload(name=name, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size, num_blocks=nb_total, pool=pool,
                    scale=sc, copy_pairs=pairs, slot_mapping=slots, k_new=kn, v_new=vn,
                    append_owner=owner, q=q, block_tables=tables,
                    context_lens=lens_post.astype(np.int32), meta=dict(meta or {}))


# -- the five recipes ---------------------------------------------------------

def tiny(seed: int = 0, dtype: str = "f32") -> Workload:
    """4 sequences caching {5, 17, 33, 64} tokens, one appended token each.

    Heads 2/2, head_dim 64, block_size 16, a 32-block pool placed by a seeded
    permutation; after the append the contexts are {6, 18, 34, 65} and the last
    sequence takes a fifth block.
    """
    return build_decode_workload("tiny", seed, [6, 18, 34, 65], 2, 2, 64, 16, dtype,
                                 num_blocks=32)


def mha(seed: int = 1, dtype: str = "bf16", num_seqs: int = 64, min_len: int = 128,
        max_len: int = 2048, num_heads: int = 32, head_dim: int = 128) -> Workload:
    """MHA decode batch (7B-like layer): context lengths uniform in [min_len, max_len]."""
    g = np.random.default_rng(_split_seeds(seed)[0])
    lens = g.integers(min_len, max_len, size=num_seqs, endpoint=True)
    return build_decode_workload("mha", seed, lens, num_heads, num_heads, head_dim, 16, dtype,
                                 meta={"len_dist": f"uniform[{min_len},{max_len}]"})


def gqa_lengths(g: np.random.Generator, num_seqs: int, median: float = 800.0,
                sigma: float = 1.0, lo: int = 16, hi: int = 8192) -> np.ndarray:
    z = g.standard_normal(num_seqs)
    return np.clip(np.rint(np.exp(math.log(median) + sigma * z)), lo, hi).astype(np.int64)


def gqa(seed: int = 2, dtype: str = "bf16", num_seqs: int = 256, median: float = 800.0,
        sigma: float = 1.0, lo: int = 16, hi: int = 8192, num_q_heads: int = 64,
        num_kv_heads: int = 8, head_dim: int = 128) -> Workload:
    """GQA long-tail decode: lognormal context lengths (median 800, ln-sigma 1), clipped."""
    g = np.random.default_rng(_split_seeds(seed)[0])
    lens = gqa_lengths(g, num_seqs, median, sigma, lo, hi)
    return build_decode_workload("gqa", seed, lens, num_q_heads, num_kv_heads, head_dim, 16,
                                 dtype, meta={"len_dist": f"lognormal(median={median},sigma={sigma})"
                                              f" clipped [{lo},{hi}]"})


def prefix(seed: int = 3, dtype: str = "bf16", num_prompts: int = 32, samples: int = 8,
           prefix_len: int = 1032, max_suffix: int = 512, num_q_heads: int = 32,
           num_kv_heads: int = 8, head_dim: int = 128, block_size: int = 16) -> Workload:
    """Shared-prefix parallel sampling.

    Each prompt's ``prefix_len`` tokens are cached once and its ``samples``
    sequences point at the same physical blocks (refcount = samples). The step
    appends every sample's divergent suffix (length uniform in [1, max_suffix]);
    the first divergent write into a shared partial block copies it (all but the
    last sharer copy; the last writes in place). With ``share=False`` every
    sample starts from its own copy of identical prefix bytes instead.
    """
    ss = _split_seeds(seed)
    g = np.random.default_rng(ss[0])
    B = num_prompts * samples
    suffix = g.integers(1, max_suffix, size=B, endpoint=True)
    bs = block_size
    pblk = _blocks_for(prefix_len, bs)
    shared_partial = prefix_len % bs != 0
    needed = 0
    for b in range(B):
        needed += _blocks_for(prefix_len + suffix[b], bs) - pblk
        if shared_partial:
            needed += 1  # the copied partial block
    needed += num_prompts * pblk
    nb = _pool_blocks(needed)
    bm = BlockManager(nb, bs, np.random.default_rng(ss[1]))
    nb_total = nb + 1
    for p in range(num_prompts):
        bm.add_sequence(("prompt", p), prefix_len)
        for s in range(samples):
            bm.fork(("prompt", p), p * samples + s)
        bm.free_sequence(("prompt", p))  # the prompt itself no longer holds blocks
    valid = _valid_mask(bm, nb_total)
    pool = _make_pool(ss[2], nb_total, num_kv_heads, bs, head_dim, dtype, valid)
    slots, owner = [], []
    for b in range(B):
        for t in range(int(suffix[b])):
            owner.append((0, b, bm.lens[b]))
            slots.append(bm.append_slot(b))
    pairs = bm.take_copy_pairs()
    bm.check()
    T = len(slots)
    tables = bm.table_array(range(B), nb)
    lens = (prefix_len + suffix).astype(np.int32)
    q = normal_values(ss[3], B * num_q_heads * head_dim, dtype).reshape(B, num_q_heads, head_dim)
    kn = normal_values(ss[4], T * num_kv_heads * head_dim, dtype).reshape(T, num_kv_heads, head_dim)
    vn = normal_values(ss[5], T * num_kv_heads * head_dim, dtype).reshape(T, num_kv_heads, head_dim)
    sc = float(np.float32(1.0 / math.sqrt(head_dim)))
    return Workload(name="prefix", dtype=dtype, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs,
                    num_blocks=nb_total, pool=pool, scale=sc, copy_pairs=pairs,
                    slot_mapping=np.asarray(slots, np.int32), k_new=kn, v_new=vn,
                    append_owner=np.asarray(owner, np.int32).reshape(-1, 3), q=q,
                    block_tables=tables, context_lens=lens,
                    meta={"prefix_len": prefix_len, "samples": samples,
                          "num_prompts": num_prompts})


def mixed(seed: int = 4, dtype: str = "bf16", num_decode: int = 240, dec_min: int = 256,
          dec_max: int = 4096, num_chunks: int = 16, chunk_len: int = 512,
          max_prior: int = 2048, num_q_heads: int = 32, num_kv_heads: int = 8,
          head_dim: int = 128, block_size: int = 32) -> Workload:
    """Mixed continuous-batching iteration: prefill chunks plus decode sequences.

    Chunk ``c`` has ``prior_c`` cached tokens (uniform in [0, max_prior]; chunk 0
    forced to 0 and chunk 1 to max_prior) and appends ``chunk_len`` new tokens
    that attend causally to all cached tokens and to earlier tokens of the
    chunk. Decode sequences attend to contexts uniform in [dec_min, dec_max]
    (after their one appended token). Every new token's K/V is appended, chunk
    tokens first, before attention.
    """
    ss = _split_seeds(seed)
    g = np.random.default_rng(ss[0])
    dec_lens = g.integers(dec_min, dec_max, size=num_decode, endpoint=True)
    prior = g.integers(0, max_prior, size=num_chunks, endpoint=True)
    if num_chunks > 0:
        prior[0] = 0
    if num_chunks > 1:
        prior[1] = max_prior
    bs = block_size
    needed = sum(_blocks_for(n, bs) for n in dec_lens) + \
        sum(_blocks_for(p + chunk_len, bs) for p in prior)
    nb = _pool_blocks(needed)
    bm = BlockManager(nb, bs, np.random.default_rng(ss[1]))
    nb_total = nb + 1
    for c in range(num_chunks):
        bm.add_sequence(("chunk", c), int(prior[c]))
    for b in range(num_decode):
        bm.add_sequence(b, int(dec_lens[b]) - 1)
    pool = _make_pool(ss[2], nb_total, num_kv_heads, bs, head_dim, dtype, _valid_mask(bm, nb_total))
    slots, owner = [], []
    for c in range(num_chunks):
        for i in range(chunk_len):
            owner.append((1, c, bm.lens[("chunk", c)]))
            slots.append(bm.append_slot(("chunk", c)))
    for b in range(num_decode):
        owner.append((0, b, bm.lens[b]))
        slots.append(bm.append_slot(b))
    pairs = bm.take_copy_pairs()
    assert pairs.shape[0] == 0
    bm.check()
    T = len(slots)
    dec_tables = bm.table_array(range(num_decode), nb)
    pre_tables = bm.table_array([("chunk", c) for c in range(num_chunks)], nb)
    q = normal_values(ss[3], num_decode * num_q_heads * head_dim, dtype).reshape(
        num_decode, num_q_heads, head_dim)
    kn = normal_values(ss[4], T * num_kv_heads * head_dim, dtype).reshape(T, num_kv_heads, head_dim)
    vn = normal_values(ss[5], T * num_kv_heads * head_dim, dtype).reshape(T, num_kv_heads, head_dim)
    nq = num_chunks * chunk_len
    pq = normal_values(ss[6], nq * num_q_heads * head_dim, dtype).reshape(nq, num_q_heads, head_dim)
    qsl = (np.arange(num_chunks + 1) * chunk_len).astype(np.int32)
    sc = float(np.float32(1.0 / math.sqrt(head_dim)))
    return Workload(name="mixed", dtype=dtype, num_q_heads=num_q_heads,
                    num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs,
                    num_blocks=nb_total, pool=pool, scale=sc, copy_pairs=pairs,
                    slot_mapping=np.asarray(slots, np.int32), k_new=kn, v_new=vn,
                    append_owner=np.asarray(owner, np.int32).reshape(-1, 3), q=q,
                    block_tables=dec_tables, context_lens=dec_lens.astype(np.int32),
                    prefill_q=pq, prefill_block_tables=pre_tables,
                    prefill_context_lens=(prior + chunk_len).astype(np.int32),
                    query_start_loc=qsl, meta={"prior": prior.tolist(), "chunk_len": chunk_len})


RECIPES = {"tiny": tiny, "mha": mha, "gqa": gqa, "prefix": prefix, "mixed": mixed}


def make_workload(name: str, **kw) -> Workload:
    if name not in RECIPES:
        raise KeyError(f"unknown workload {name!r}; choose from {CONFIG_NAMES}")
    return RECIPES[name](**kw)
