"""Test-side writer of the pool layout, independent of the oracle and the library.

Writes logical tokens of contiguous per-sequence K/V into a pool of the
documented layout: block j = K half [Hkv][d/8][bs][8] then V half
[Hkv][bs/4][d][4].
"""
from __future__ import annotations

import numpy as np


def empty_pool(num_blocks, Hkv, bs, d, dtype=np.float64):
    return np.full((num_blocks, 2 * Hkv * bs * d), np.nan, dtype)


def put_token(pool, blk, slot, k_heads, v_heads, Hkv, bs, d):
    """k_heads, v_heads: [Hkv][d] values of one token."""
    for g in range(Hkv):
        for i in range(d):
            pool[blk, g * bs * d + ((i // 8) * bs + slot) * 8 + i % 8] = k_heads[g][i]
            pool[blk, Hkv * bs * d + g * bs * d + ((slot // 4) * d + i) * 4 + slot % 4] = \
                v_heads[g][i]


def contiguous_pool(K, V, bs, dtype=np.float32):
    """Pool + identity tables for per-sequence contiguous K, V.

    K[b], V[b]: arrays [n_b][Hkv][d]. Sequence b owns consecutive blocks; one
    trailing NaN block serves as padding for table rows.
    """
    Hkv, d = K[0].shape[1], K[0].shape[2]
    nblk = [-(-k.shape[0] // bs) for k in K]
    total = sum(nblk)
    pool = empty_pool(total + 1, Hkv, bs, d, dtype)
    width = max(max(nblk), 1)
    tables = np.full((len(K), width), total, np.int32)
    base = 0
    for b, (k, v) in enumerate(zip(K, V)):
        for j in range(nblk[b]):
            tables[b, j] = base + j
        for t in range(k.shape[0]):
            put_token(pool, base + t // bs, t % bs, k[t], v[t], Hkv, bs, d)
        base += nblk[b]
    return pool, tables


def unshare_blocks(pool, tables, lens, block_size, pad):
    """Give every table row private copies of the blocks it shares with earlier rows.

    Returns (new_pool, new_tables): the new pool appends one byte-equal copy per
    extra reference (the pad block stays last); rows keep the same logical
    contents, now in unshared physical blocks.
    """
    nb = pool.shape[0]
    seen = set()
    extra = []
    new_tables = np.array(tables, copy=True)
    for r in range(tables.shape[0]):
        used = -(-int(lens[r]) // block_size)
        for j in range(used):
            blk = int(tables[r, j])
            if blk in seen:
                extra.append(blk)
                new_tables[r, j] = -len(extra)  # placeholder, fixed below
            else:
                seen.add(blk)
    # layout: old blocks 0..nb-2, copies, then the pad block last
    new_pad = nb - 1 + len(extra)
    out = np.empty((nb + len(extra),) + pool.shape[1:], pool.dtype)
    out[: nb - 1] = np.delete(pool, pad, axis=0) if pad != nb - 1 else pool[: nb - 1]
    assert pad == nb - 1, "pad block must be the last block"
    for i, blk in enumerate(extra):
        out[nb - 1 + i] = pool[blk]
    out[new_pad] = pool[pad]
    new_tables[new_tables == pad] = new_pad
    neg = new_tables < 0
    new_tables[neg] = nb - 1 + (-new_tables[neg] - 1)
    return out, new_tables.astype(np.int32)
