"""Seeded value sources shared by the tests, the bench and the oracle's tests.

Only input *formatting* lives here: standard-normal draws and the fp32 -> bf16
round-to-nearest-even encoding used to store them. Nothing here computes
attention, gathers through a block table or merges partial results.

Draws are split into fixed-size chunks, each with its own child of one
``numpy.random.SeedSequence``; the chunk -> child assignment is fixed, so the
values depend only on the seed and the count, never on the thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22  # values per child generator

BF16_NAN_BITS = np.uint16(0x7FC0)
F32_NAN = np.float32(np.nan)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    NaN inputs map to the canonical quiet NaN 0x7FC0.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint32, copy=True)
    nan = np.isnan(x)
    b += ((b >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    out = (b >> 16).astype(np.uint16)
    out[nan] = BF16_NAN_BITS
    return out


def normal_values(seed_seq: np.random.SeedSequence, count: int, dtype: str,
                  scale: float = 1.0) -> np.ndarray:
    """``count`` i.i.d. N(0, scale^2) values drawn in float32, stored as ``dtype``.

    dtype "f32" returns float32; "bf16" returns uint16 bfloat16 bits (each fp32
    draw rounded once, to nearest even).
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError(f"unknown dtype {dtype!r}")
    out = np.empty(count, np.float32 if dtype == "f32" else np.uint16)
    if count == 0:
        return out
    nchunks = (count + CHUNK - 1) // CHUNK
    kids = seed_seq.spawn(nchunks)

    def work(i: int) -> None:
        lo = i * CHUNK
        hi = min(count, lo + CHUNK)
        g = np.random.default_rng(kids[i])
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        if dtype == "f32":
            out[lo:hi] = x
        else:
            b = x.view(np.uint32)
            b += ((b >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
            out[lo:hi] = b >> 16

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def nan_value(dtype: str):
    return F32_NAN if dtype == "f32" else BF16_NAN_BITS


def storage_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def element_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2
