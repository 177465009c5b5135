"""Minimal host-side KV block manager used to build inputs.

Behaviour taken from "Module 4 · Batching, Scheduling, and Paging", section
"PagedAttention" (the host owns each sequence's table of physical blocks; a
sequence gets a fresh block at the moment its current last block is full, and
all of its blocks return to the free list when it ends), section "Block
sharing" (samples of one prompt share its physical blocks, a shared block is
duplicated before the first write that would make the samples differ, and a
per-block count of sharers decides when a block is free again), and "Paging
the KV Cache", section "The waste hiding inside memory" (a request's cache is
a list of pages, and a finished request's pages are reused by later ones).

Physical placement: the free list is a seeded random permutation of the block
ids, consumed from the front; freed blocks go to the back.

Copy-on-write reading: a writer whose target block has refcount > 1 takes a
fresh block, records a (src, dst) copy pair and decrements the shared block;
the last sharer (refcount 1) writes in place. Sequences are processed in the
order the caller appends to them.
"""
from __future__ import annotations

from collections import deque

import numpy as np


class PoolExhausted(RuntimeError):
    """Raised when an allocation finds no free block (the manager refuses)."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int, rng: np.random.Generator):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        self.free = deque(int(b) for b in rng.permutation(num_blocks))
        self.refcount = np.zeros(num_blocks, np.int64)
        self.tables: dict[object, list[int]] = {}
        self.lens: dict[object, int] = {}
        self.copy_pairs: list[tuple[int, int]] = []

    # -- allocation -------------------------------------------------------
    def _alloc(self) -> int:
        if not self.free:
            raise PoolExhausted("no free KV block")
        b = self.free.popleft()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        assert self.refcount[b] >= 0
        if self.refcount[b] == 0:
            self.free.append(b)

    def num_free(self) -> int:
        return len(self.free)

    def add_sequence(self, seq, num_tokens: int) -> list[int]:
        """Register a sequence whose first ``num_tokens`` tokens are already cached."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq!r} exists")
        nblk = -(-num_tokens // self.block_size)
        if nblk > len(self.free):
            raise PoolExhausted(f"need {nblk} blocks, {len(self.free)} free")
        self.tables[seq] = [self._alloc() for _ in range(nblk)]
        self.lens[seq] = int(num_tokens)
        return self.tables[seq]

    def fork(self, parent, child) -> None:
        """``child`` shares every block of ``parent`` (refcounts go up)."""
        if child in self.tables:
            raise KeyError(f"sequence {child!r} exists")
        blocks = list(self.tables[parent])
        for b in blocks:
            self.refcount[b] += 1
        self.tables[child] = blocks
        self.lens[child] = self.lens[parent]

    def append_slot(self, seq) -> int:
        """Reserve the slot for the next token of ``seq`` and return it.

        Allocates a block when the last one is full; copies-on-write when the
        last block is shared. The copy pair, if any, is appended to
        ``self.copy_pairs``.
        """
        pos = self.lens[seq]
        table = self.tables[seq]
        idx, off = divmod(pos, self.block_size)
        if idx == len(table):
            table.append(self._alloc())
        elif self.refcount[table[idx]] > 1:
            src = table[idx]
            dst = self._alloc()
            self.copy_pairs.append((src, dst))
            self.refcount[src] -= 1
            table[idx] = dst
        self.lens[seq] = pos + 1
        return table[idx] * self.block_size + off

    def free_sequence(self, seq) -> None:
        for b in self.tables.pop(seq):
            self._release(b)
        del self.lens[seq]

    def take_copy_pairs(self) -> np.ndarray:
        pairs = np.asarray(self.copy_pairs, np.int32).reshape(-1, 2)
        self.copy_pairs = []
        return pairs

    # -- export -----------------------------------------------------------
    def table_array(self, seqs, pad: int, width: int | None = None) -> np.ndarray:
        rows = [self.tables[s] for s in seqs]
        w = max((len(r) for r in rows), default=0) if width is None else width
        w = max(w, 1)
        out = np.full((len(rows), w), pad, np.int32)
        for i, r in enumerate(rows):
            out[i, : len(r)] = r
        return out

    def check(self) -> None:
        """Refcounts equal the number of table references; free list is disjoint."""
        counts = np.zeros(self.num_blocks, np.int64)
        for t in self.tables.values():
            for b in t:
                counts[b] += 1
        if not np.array_equal(counts, self.refcount):
            raise AssertionError("refcount does not match table references")
        free = list(self.free)
        if len(set(free)) != len(free) or any(counts[b] for b in free):
            raise AssertionError("free list holds a referenced or duplicate block")
        if len(free) + int((counts > 0).sum()) != self.num_blocks:
            raise AssertionError("a block is neither free nor referenced")
