"""fp64 NumPy oracle for paged decode / chunked-prefill attention, KV append and block copy.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pool format (the library's documented layout): ``pool`` is ``[num_blocks,
2*Hkv*bs*d]`` storage elements. Block ``j`` holds its K half then its V half.
Per kv head, the K half is ``[d/8][bs][8]`` (dimension i of slot s at
``((i // 8) * bs + s) * 8 + i % 8``) and the V half is ``[bs/4][d][4]``
(dimension i of slot s at ``((s // 4) * d + i) * 4 + s % 4``). Elements are
float32 values or bfloat16 bit patterns (uint16); both decode exactly to
float64.
"""
from __future__ import annotations

import numpy as np


# -- element decoding -----------------------------------------------------------

def decode_elements(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (float32 values or bfloat16 bits).

    A bfloat16 is the upper 16 bits of a float32, so its value is that float32
    with the low 16 bits zero.
    """
    if dtype == "f32":
        return np.asarray(raw, np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(raw, np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def pool_views(pool: np.ndarray, num_kv_heads: int, block_size: int, head_dim: int):
    """Views of the raw pool: K as [blk][head][d/8][slot][8], V as [blk][head][slot/4][d][4]."""
    nb = pool.shape[0]
    halves = pool.reshape(nb, 2, num_kv_heads * block_size * head_dim)
    k = halves[:, 0].reshape(nb, num_kv_heads, head_dim // 8, block_size, 8)
    v = halves[:, 1].reshape(nb, num_kv_heads, block_size // 4, head_dim, 4)
    return k, v


# -- O1: gather through the block table -------------------------------------------

def gather(pool, dtype, table_row, n, g, num_kv_heads, block_size, head_dim):
    """K, V (float64, [n][d]) of logical tokens 0..n-1 of one sequence, kv head ``g``.

    Logical token t lives in physical block ``table_row[t // bs]`` at slot
    ``t % bs`` ("Module 4", section "PagedAttention": a per-sequence block
    table maps logical blocks to physical ones; attention gathers K and V
    through that indirection).
    """
    kview, vview = pool_views(pool, num_kv_heads, block_size, head_dim)
    t = np.arange(n)
    blk = np.asarray(table_row)[t // block_size]
    off = t % block_size
    k = kview[blk, g, :, off, :].reshape(n, head_dim)     # [n][d/8][8] -> [n][d]
    v = vview[blk, g, off // 4, :, off % 4]                # [n][d]
    return decode_elements(k, dtype), decode_elements(v, dtype)


# -- O2: textbook attention of one query -------------------------------------------

def attend(qv: np.ndarray, K: np.ndarray, V: np.ndarray, sigma: float) -> np.ndarray:
    """softmax(sigma * q K^T) V for one query over its own keys (float64).

    worksonmygpu.com continuous-batching post, section "Selective batching":
    softmax(Q K^T / sqrt(d_k)) V, each request over its own prior tokens; the
    caller passes sigma (1/sqrt(d_k) in every workload). Zero keys give zeros.
    """
    n = K.shape[0]
    if n == 0:
        return np.zeros(V.shape[1], np.float64)
    s = sigma * (K @ qv)
    m = s.max()
    w = np.exp(s - m)
    return (w @ V) / w.sum()


def decode(q, pool, block_tables, context_lens, num_kv_heads, block_size, scale, dtype):
    """Decode attention for every (sequence, query head): float64 [B][Hq][d].

    Query head h reads kv head ``h // (Hq / Hkv)`` (contiguous groups). The
    context of sequence b is its first ``context_lens[b]`` logical tokens,
    which include the token appended this step. ``scale`` is used as the
    float32 value the library receives.
    """
    q64 = decode_elements(q, dtype)
    B, Hq, d = q64.shape
    G = Hq // num_kv_heads
    sigma = float(np.float32(scale))
    out = np.zeros((B, Hq, d), np.float64)
    for b in range(B):
        n = int(context_lens[b])
        for g in range(num_kv_heads):
            K, V = gather(pool, dtype, block_tables[b], n, g, num_kv_heads, block_size, d)
            for h in range(g * G, (g + 1) * G):
                out[b, h] = attend(q64[b, h], K, V, sigma)
    return out


# -- O3: chunked prefill ------------------------------------------------------------

def prefill(q, pool, block_tables, context_lens, query_start_loc, num_kv_heads, block_size,
            scale, dtype):
    """Chunked-prefill attention: float64 [sum L][Hq][d].

    Chunk c has ``L = qsl[c+1] - qsl[c]`` queries, the last L of its
    ``context_lens[c]`` tokens (already appended to the cache). Query i sits at
    position ``a = context_lens[c] - L + i`` and attends to keys 0..a: causal
    within the chunk, full over the earlier cached tokens (the continuous-
    batching post, section "The prefill/decode mix").
    """
    q64 = decode_elements(q, dtype)
    T, Hq, d = q64.shape
    G = Hq // num_kv_heads
    sigma = float(np.float32(scale))
    out = np.zeros((T, Hq, d), np.float64)
    C = len(context_lens)
    for c in range(C):
        lo, hi = int(query_start_loc[c]), int(query_start_loc[c + 1])
        L, n = hi - lo, int(context_lens[c])
        for g in range(num_kv_heads):
            K, V = gather(pool, dtype, block_tables[c], n, g, num_kv_heads, block_size, d)
            for i in range(L):
                a = n - L + i
                for h in range(g * G, (g + 1) * G):
                    out[lo + i, h] = attend(q64[lo + i, h], K[: a + 1], V[: a + 1], sigma)
    return out


# -- O4: append, O5: copy --------------------------------------------------------

def append(pool, k_new, v_new, slot_mapping, num_kv_heads, block_size, head_dim):
    """New pool with token i's K/V rows written, bit for bit, at ``slot_mapping[i]``.

    Slot s is block ``s // bs``, offset ``s % bs``; negative slots are skipped.
    The cache grows one token at a time ("Paging the KV Cache", section "The
    waste hiding inside memory").
    """
    out = pool.copy()
    kview, vview = pool_views(out, num_kv_heads, block_size, head_dim)
    for i, s in enumerate(np.asarray(slot_mapping)):
        if s < 0:
            continue
        blk, off = divmod(int(s), block_size)
        kview[blk, :, :, off, :] = k_new[i].reshape(num_kv_heads, head_dim // 8, 8)
        vview[blk, :, off // 4, :, off % 4] = v_new[i]
    return out


def copy_blocks(pool, pairs):
    """New pool with ``pool[dst] = pool_before[src]`` for every (src, dst) pair.

    Copy-on-write of a shared block ("Module 4", section "Block sharing"). All
    copies read the state before the call.
    """
    snap = pool.copy()
    out = pool.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        out[int(dst)] = snap[int(src)]
    return out


def swap_blocks(pool, host, pairs, direction):
    """New (pool, host) after moving whole blocks between them.

    direction 0 (out): host[dst] = pool[src]; 1 (in): pool[dst] = host[src].
    An evicted request's blocks go to CPU memory and come back later
    ("Module 4", section "PagedAttention"). Reads see the state before the
    call.
    """
    new_pool, new_host = pool.copy(), host.copy()
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        if direction == 0:
            new_host[int(dst)] = pool[int(src)]
        else:
            new_pool[int(dst)] = host[int(src)]
    return new_pool, new_host


def check_slots(slot_mapping, append_owner, block_tables, block_size,
                prefill_block_tables=None) -> None:
    """Assert each slot equals the one its (table, row, position) implies.

    ``append_owner[i] = (kind, row, pos)``; kind 0 reads ``block_tables``, kind
    1 reads ``prefill_block_tables``. The slot of position p is
    ``table[p // bs] * bs + p % bs``.
    """
    for i, (kind, row, pos) in enumerate(np.asarray(append_owner)):
        tables = block_tables if kind == 0 else prefill_block_tables
        want = int(tables[row][pos // block_size]) * block_size + int(pos) % block_size
        if int(slot_mapping[i]) != want:
            raise AssertionError(f"token {i}: slot {int(slot_mapping[i])} != {want}")


# -- split-K merge (log-sum-exp identity) --------------------------------------------

def attend_partitioned(qv, K, V, sigma, cuts):
    """Per-piece (m, l, unnormalised o) of attention with keys cut at ``cuts``.

    Piece j covers keys [cuts[j], cuts[j+1]); for it m = max s, l = sum
    exp(s - m), o = sum exp(s - m) V. An empty piece gives (-inf, 0, 0).
    """
    parts = []
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        if hi <= lo:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[1])))
            continue
        s = sigma * (K[lo:hi] @ qv)
        m = s.max()
        w = np.exp(s - m)
        parts.append((m, w.sum(), w @ V[lo:hi]))
    return parts


def merge_partials(parts):
    """Normalised output from pieces (m_j, l_j, o_j).

    M = max m_j, l = sum l_j e^(m_j - M), o = sum o_j e^(m_j - M) / l: the
    softmax of a union of key sets from the softmaxes of its pieces.
    """
    finite = [p for p in parts if np.isfinite(p[0])]
    if not finite:
        return np.zeros_like(parts[0][2], dtype=np.float64)
    M = max(p[0] for p in finite)
    l = sum(p[1] * np.exp(p[0] - M) for p in finite)
    o = sum(p[2] * np.exp(p[0] - M) for p in finite)
    return o / l


# -- weight moments: what a rounding of the weights or of a partial can move ------

def softmax_moments(qv, K, V, sigma):
    """(o, E_w|V|, E_w|V - o|) of one query, all float64 [d].

    w are the softmax weights of ``sigma * K qv`` (the same definition as
    ``attend``), o = sum_t w_t V_t, and the two moments are the w-weighted
    means of |V_t| and of |V_t - o| per dimension. They size the error of an
    implementation that perturbs each weight by a relative amount (rounding
    the weights, or inexact scores: at most its bound times E_w|V - o|, since
    the perturbed weights are renormalised) or rounds partial outputs that
    are themselves convex combinations of V (at most the rounding unit times
    E_w|V|). An empty context gives three zero vectors.
    """
    n, d = V.shape
    if n == 0:
        z = np.zeros(d, np.float64)
        return z, z.copy(), z.copy()
    s = sigma * (K @ qv)
    w = np.exp(s - s.max())
    w = w / w.sum()
    o = w @ V
    return o, w @ np.abs(V), w @ np.abs(V - o)


def decode_moments(q, pool, block_tables, context_lens, num_kv_heads, block_size, scale, dtype):
    """``softmax_moments`` of every (sequence, query head) of a decode batch:
    three float64 arrays [B][Hq][d] (o, E_w|V|, E_w|V - o|)."""
    q64 = decode_elements(q, dtype)
    B, Hq, d = q64.shape
    G = Hq // num_kv_heads
    sigma = float(np.float32(scale))
    res = np.zeros((3, B, Hq, d), np.float64)
    for b in range(B):
        n = int(context_lens[b])
        for g in range(num_kv_heads):
            K, V = gather(pool, dtype, block_tables[b], n, g, num_kv_heads, block_size, d)
            for h in range(g * G, (g + 1) * G):
                res[:, b, h] = softmax_moments(q64[b, h], K, V, sigma)
    return res[0], res[1], res[2]


def prefill_moments(q, pool, block_tables, context_lens, query_start_loc, num_kv_heads,
                    block_size, scale, dtype):
    """``softmax_moments`` of every (query, head) of a chunked prefill (the
    causal key ranges of ``prefill``): three float64 arrays [sum L][Hq][d]."""
    q64 = decode_elements(q, dtype)
    T, Hq, d = q64.shape
    G = Hq // num_kv_heads
    sigma = float(np.float32(scale))
    res = np.zeros((3, T, Hq, d), np.float64)
    for c in range(len(context_lens)):
        lo, hi = int(query_start_loc[c]), int(query_start_loc[c + 1])
        L, n = hi - lo, int(context_lens[c])
        for g in range(num_kv_heads):
            K, V = gather(pool, dtype, block_tables[c], n, g, num_kv_heads, block_size, d)
            for i in range(L):
                a = n - L + i
                for h in range(g * G, (g + 1) * G):
                    res[:, lo + i, h] = softmax_moments(q64[lo + i, h], K[: a + 1], V[: a + 1],
                                                        sigma)
    return res[0], res[1], res[2]
