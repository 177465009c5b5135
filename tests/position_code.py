"""Position-coded inputs whose attention output is known exactly (test input
construction only: no attention arithmetic).

Every cached or appended token t of kv head g gets
  V[t, g] = a vector of small integers that encodes t (dims 0 and 1 hold
            1 + t % 128 and 1 + t // 128, dim 2 holds 1 + g, the rest are
            1 + (31 t + 7 i + 3 g) % 97), exact in bfloat16 and float32;
  K[t, g] = 0, except at a few marked positions, where K[t, g] = SPIKE * e_j
            for a dimension j that no other marked token of the same context
            and head uses.
A query q = e_j (1.0 at dimension j) of a head of kv head g then scores
SPIKE * scale on the marked token with dimension j and exactly 0 on every
other token. With SPIKE * scale * log2(e) > 64 every other weight is below
2^-64 of the target's, far below the bfloat16 and float32 resolution of the
sums, so an implementation that reads every token from the right block and
slot returns exactly V of the target; a wrong block or slot for the target
gives another token's V or the mean over the context instead.

Marks include the first token, the last (the one appended this step), block
and 32-token step edges, the split-K partition edges and random positions.
Prompt-prefix positions that several samples share carry marks chosen once
per prompt (dimensions 0..7), so a shared slot holds the same bytes for every
sequence that reads it; positions private to a sample use dimensions 8 and up.
"""
from __future__ import annotations

import numpy as np

from workloads import f32_to_bf16_bits

SPIKE = 512.0  # 2^9: exact in bfloat16


def v_code(pos: np.ndarray, g: int, d: int) -> np.ndarray:
    """float32 [len(pos)][d]: the value rows of positions ``pos`` of kv head g."""
    pos = np.asarray(pos, np.int64)
    out = np.empty((len(pos), d), np.float32)
    out[:, 0] = 1 + pos % 128
    out[:, 1] = 1 + pos // 128
    out[:, 2] = 1 + g
    i = np.arange(3, d)
    out[:, 3:] = 1 + (pos[:, None] * 31 + i[None, :] * 7 + g * 3) % 97
    return out


def _enc(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == "bf16" else np.asarray(x, np.float32)


def _write(pool, table_row, pos, K, V, Hkv, bs, d):
    """Write K/V rows ([n][Hkv][d] stored elements) of positions ``pos`` at
    their slots (block table_row[t // bs], slot t % bs) in the documented pool
    layout."""
    nb = pool.shape[0]
    halves = pool.reshape(nb, 2, Hkv * bs * d)
    kview = halves[:, 0].reshape(nb, Hkv, d // 8, bs, 8)
    vview = halves[:, 1].reshape(nb, Hkv, bs // 4, d, 4)
    blk = np.asarray(table_row)[pos // bs]
    slot = pos % bs
    kview[blk, :, :, slot, :] = K.reshape(len(pos), Hkv, d // 8, 8)
    vview[blk, :, slot // 4, :, slot % 4] = V


class PositionCoded:
    """Rewrites a workload's pool, appended rows and queries in place; holds
    the exact expected outputs (float32 values) of its decode and prefill."""

    DECODE_EDGES = (0, 1, 15, 16, 17, 31, 32, 33, 1023, 1024, 1025, 2047, 2048, 4095, 4096)
    PREFILL_EDGES = (0, 31, 32, 1023, 1024, 2047, 2048)

    def __init__(self, w, seed: int, prefix_len: int = 0, samples: int = 1):
        self.w = w
        rng = np.random.default_rng(seed)
        Hkv, d, bs, dtype = w.num_kv_heads, w.head_dim, w.block_size, w.dtype
        G = w.num_q_heads // Hkv
        assert d >= 16
        # marks[(kind, row)][g] = {position: dimension}
        self.marks = {}
        shared = {}  # (prompt, g) -> {position: dimension} for shared prefix positions
        B = w.num_seqs
        for b in range(B):
            n = int(w.context_lens[b])
            per_g = []
            for g in range(Hkv):
                m = {}
                lo = 0
                if prefix_len:
                    p = b // samples
                    if (p, g) not in shared:
                        cand = {0, 15, 16, 1023, 1024, prefix_len - 1}
                        cand |= set(int(x) for x in rng.integers(0, prefix_len, 2))
                        cand = sorted(c for c in cand if c < prefix_len)
                        dims = rng.permutation(8)[: len(cand)]
                        shared[(p, g)] = dict(zip(cand, (int(x) for x in dims)))
                    m.update(shared[(p, g)])
                    lo = prefix_len
                cand = {n - 1, n - 2, n // 2, lo} | {e for e in self.DECODE_EDGES}
                cand |= set(int(x) for x in rng.integers(lo, max(lo + 1, n), 4))
                cand = sorted(c for c in cand if lo <= c < n)
                first = 8 if prefix_len else 0
                dims = first + rng.permutation(d - first)[: len(cand)]
                m.update(zip(cand, (int(x) for x in dims)))
                per_g.append(m)
            self.marks[(0, b)] = per_g
        C = 0 if w.prefill_q is None else len(w.prefill_context_lens)
        for c in range(C):
            n = int(w.prefill_context_lens[c])
            L = int(w.query_start_loc[c + 1] - w.query_start_loc[c])
            prior = n - L
            per_g = []
            for g in range(Hkv):
                cand = {0, prior - 1, prior, prior + 1, n - 1, n - 2} | set(self.PREFILL_EDGES)
                cand |= set(int(x) for x in rng.integers(0, n, 12))
                cand = sorted(x for x in cand if 0 <= x < n)
                dims = rng.permutation(d)[: len(cand)]
                per_g.append(dict(zip(cand, (int(x) for x in dims))))
            self.marks[(1, c)] = per_g

        # the pool: every position of every context, at its final slot (slots
        # that this step appends or copies are rewritten with the same bytes)
        top = max([int(w.context_lens.max()) if B else 0] +
                  [int(w.prefill_context_lens.max()) if C else 0])
        # [top][Hkv][d] stored elements
        vall = _enc(np.stack([v_code(np.arange(top), g, d) for g in range(Hkv)], 1), dtype)
        spike = _enc(np.array([SPIKE], np.float32), dtype)[0]

        def rows_of(kind, row, pos):
            """Stored K and V rows of positions ``pos`` (sorted) of one context."""
            K = np.zeros((len(pos), Hkv, d), vall.dtype)
            V = vall[pos]
            for g in range(Hkv):
                for t, j in self.marks[(kind, row)][g].items():
                    k = int(np.searchsorted(pos, t))
                    if k < len(pos) and pos[k] == t:
                        K[k, g, j] = spike
            return K, V

        for b in range(B):
            pos = np.arange(int(w.context_lens[b]))
            K, V = rows_of(0, b, pos)
            _write(w.pool, w.block_tables[b], pos, K, V, Hkv, bs, d)
        for c in range(C):
            pos = np.arange(int(w.prefill_context_lens[c]))
            K, V = rows_of(1, c, pos)
            _write(w.pool, w.prefill_block_tables[c], pos, K, V, Hkv, bs, d)
        # the rows this step appends (positions past a shortened context keep
        # their drawn values: no attention reads them)
        for i, (kind, row, pos) in enumerate(np.asarray(w.append_owner)):
            if pos < top:
                K, V = rows_of(int(kind), int(row), np.array([int(pos)]))
                w.k_new[i], w.v_new[i] = K[0], V[0]

        # decode queries: head j of kv head g targets the last token, the first
        # token or one of the marks, in rotation over (sequence, head)
        q = np.zeros(w.q.shape, np.float32)
        want = np.empty(w.q.shape, np.float32)
        self.decode_targets = np.empty(w.q.shape[:2], np.int64)
        for b in range(B):
            n = int(w.context_lens[b])
            for g in range(Hkv):
                mk = self.marks[(0, b)][g]
                order = sorted(mk)
                for j in range(G):
                    h = g * G + j
                    k = (7 * b + 3 * g + 5 * j) % (len(order) + 2)
                    t = n - 1 if k == 0 else (0 if k == 1 else order[k - 2])
                    q[b, h, mk[t]] = 1.0
                    want[b, h] = v_code(np.array([t]), g, d)[0]
                    self.decode_targets[b, h] = t
        w.q[...] = _enc(q, dtype)
        self.decode_want = want
        # prefill queries: query i (position a) of head j targets the k-th
        # latest mark at or before a
        self.prefill_want = None
        if C:
            pq = np.zeros(w.prefill_q.shape, np.float32)
            pw = np.empty(w.prefill_q.shape, np.float32)
            for c in range(C):
                lo, hi = int(w.query_start_loc[c]), int(w.query_start_loc[c + 1])
                n = int(w.prefill_context_lens[c])
                L = hi - lo
                for g in range(Hkv):
                    mk = self.marks[(1, c)][g]
                    order = np.array(sorted(mk))
                    vals = v_code(order, g, d)
                    for i in range(L):
                        a = n - L + i
                        upto = int(np.searchsorted(order, a, side="right"))
                        for j in range(G):
                            k = upto - 1 - (i + j) % upto
                            t = int(order[k])
                            pq[lo + i, g * G + j, mk[t]] = 1.0
                            pw[lo + i, g * G + j] = vals[k]
            w.prefill_q[...] = _enc(pq, dtype)
            self.prefill_want = pw

    def want_bits(self, which: str) -> np.ndarray:
        """Expected outputs as stored elements (bfloat16 bits or float32)."""
        x = self.decode_want if which == "decode" else self.prefill_want
        return _enc(x, self.w.dtype)
