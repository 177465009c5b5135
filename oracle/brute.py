"""Pure-Python scalar brute force of the same operations — TEST INFRASTRUCTURE ONLY.

Independent of ``oracle.paged_attention``: it reads the pool as a flat list
with its own index arithmetic (K element (blk, head, slot, dim) at
``blk*E + head*bs*d + ((dim // 8)*bs + slot)*8 + dim % 8``; V element at
``blk*E + Hkv*bs*d + head*bs*d + ((slot // 4)*d + dim)*4 + slot % 4`` with
``E = 2*Hkv*bs*d``),
decodes bfloat16 through ``struct``, and uses explicit loops, ``math.exp`` and
``math.fsum``. Only for tiny inputs.
"""
from __future__ import annotations

import math
import struct


def _value(word, dtype):
    if dtype == "f32":
        return float(word)
    return struct.unpack("<f", struct.pack("<I", (int(word) & 0xFFFF) << 16))[0]


def _k_index(blk, head, slot, dim, Hkv, bs, d):
    return blk * (2 * Hkv * bs * d) + head * bs * d + ((dim // 8) * bs + slot) * 8 + dim % 8


def _v_index(blk, head, slot, dim, Hkv, bs, d):
    return (blk * (2 * Hkv * bs * d) + Hkv * bs * d + head * bs * d
            + ((slot // 4) * d + dim) * 4 + slot % 4)


def _attend_one(qv, keys, vals, sigma):
    if not keys:
        return [0.0] * len(qv)
    scores = [sigma * math.fsum(a * b for a, b in zip(qv, k)) for k in keys]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    z = math.fsum(w)
    d = len(vals[0])
    return [math.fsum(w[t] * vals[t][i] for t in range(len(w))) / z for i in range(d)]


def _tokens(flat, dtype, table_row, n, g, Hkv, bs, d):
    keys, vals = [], []
    for t in range(n):
        blk = int(table_row[t // bs])
        slot = t - (t // bs) * bs
        keys.append([_value(flat[_k_index(blk, g, slot, i, Hkv, bs, d)], dtype) for i in range(d)])
        vals.append([_value(flat[_v_index(blk, g, slot, i, Hkv, bs, d)], dtype) for i in range(d)])
    return keys, vals


def decode(q, pool, block_tables, context_lens, Hkv, bs, scale, dtype):
    flat = list(pool.reshape(-1))
    B, Hq, d = q.shape
    group = Hq // Hkv
    sigma = float(struct.unpack("<f", struct.pack("<f", scale))[0])
    out = []
    for b in range(B):
        rows = []
        for h in range(Hq):
            g = h // group
            keys, vals = _tokens(flat, dtype, block_tables[b], int(context_lens[b]), g, Hkv, bs, d)
            qv = [_value(x, dtype) for x in q[b, h]]
            rows.append(_attend_one(qv, keys, vals, sigma))
        out.append(rows)
    return out


def prefill(q, pool, block_tables, context_lens, query_start_loc, Hkv, bs, scale, dtype):
    flat = list(pool.reshape(-1))
    T, Hq, d = q.shape
    group = Hq // Hkv
    sigma = float(struct.unpack("<f", struct.pack("<f", scale))[0])
    out = [None] * T
    for c in range(len(context_lens)):
        lo, hi = int(query_start_loc[c]), int(query_start_loc[c + 1])
        n = int(context_lens[c])
        for i in range(hi - lo):
            pos = n - (hi - lo) + i
            rows = []
            for h in range(Hq):
                keys, vals = _tokens(flat, dtype, block_tables[c], pos + 1, h // group, Hkv, bs, d)
                qv = [_value(x, dtype) for x in q[lo + i, h]]
                rows.append(_attend_one(qv, keys, vals, sigma))
            out[lo + i] = rows
    return out


def append(pool, k_new, v_new, slot_mapping, Hkv, bs, d):
    flat = pool.reshape(-1).copy()
    for i in range(len(slot_mapping)):
        s = int(slot_mapping[i])
        if s < 0:
            continue
        blk, slot = s // bs, s - (s // bs) * bs
        for g in range(Hkv):
            for x in range(d):
                flat[_k_index(blk, g, slot, x, Hkv, bs, d)] = k_new[i, g, x]
                flat[_v_index(blk, g, slot, x, Hkv, bs, d)] = v_new[i, g, x]
    return flat.reshape(pool.shape)


def copy_blocks(pool, pairs):
    E = pool.shape[1]
    before = list(pool.reshape(-1))
    flat = pool.reshape(-1).copy()
    for src, dst in pairs:
        for e in range(E):
            flat[int(dst) * E + e] = before[int(src) * E + e]
    return flat.reshape(pool.shape)
