"""The sharing hint pa_decode_shared takes, derived from block tables.

A caller that forks sequences knows which ones share blocks; one that only has
the tables can read it off them, as here: sequence b shares with b-1 the
tokens of the leading table entries the two rows have in common, up to either
context's length ("Module 4 · Batching, Scheduling, and Paging", section
"Block sharing": the samples of a prompt point at the same physical blocks).
"""
from __future__ import annotations

import numpy as np


def share_prev_hint(block_tables: np.ndarray, context_lens: np.ndarray,
                    block_size: int) -> np.ndarray:
    """int32 [B]: leading tokens of sequence b held in the same blocks as b-1's (0 for b = 0)."""
    tables = np.asarray(block_tables)
    lens = np.asarray(context_lens, np.int64)
    B = lens.size
    out = np.zeros(B, np.int32)
    for b in range(1, B):
        n = min(int(lens[b]), int(lens[b - 1]))
        if n <= 0:
            continue
        nblk = -(-n // block_size)
        same = tables[b, :nblk] == tables[b - 1, :nblk]
        k = nblk if same.all() else int(np.argmin(same))
        out[b] = min(k * block_size, n)
    return out
