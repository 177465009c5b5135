"""Discriminating parity for every attention kernel path.

1. Position-coded inputs (tests/position_code.py): every query's softmax is a
   spike on one marked token, and V encodes the token's position, so a kernel
   that reads every token through the right block and slot must return that
   token's V exactly; a wrong block, slot, step or partition edge for the
   target returns another token's V or the context's mean. Outputs are
   compared bit for bit with the expected rows (and the oracle is checked to
   agree with them on sampled rows).
2. Sharpened random inputs (q x 8, a peaked softmax on N(0,1) keys and
   values) against the fp64 oracle, element by element, under the bound the
   bfloat16 path's roundings allow:
     |o - o*| <= 2^-8 |o*| + (2^-8 + 2^-10) E_w|V| + (2^-7 + 2^-10) E_w|V - o*|
   where o* is the oracle's output and E_w the mean under its softmax
   weights: the final rounding of o to bfloat16 (half an ulp, at most 2^-8
   relative); the rounding of each split-K partition's normalised output to
   bfloat16 (each partial is a convex combination of V, so at most 2^-8
   E_w|V| after the merge); the rounding of each weight p to bfloat16, which
   the row sum shares, so the perturbed weights stay normalised (each relative
   weight changes by at most about 2^-7, which moves o by at most 2^-7
   E_w|V - o*|); and float32 accumulation of scores and sums (2^-10 terms).
   The worst error is also reported in units of the output's bfloat16 ulp.

Kernel paths: persistent decode at block sizes 16 and 32, with cached and
with nontemporal loads (batches under and over 256 MiB of K+V), with shared
prefix blocks, at G = 1, 2, 4, 8; the one-workgroup-per-item decode (over
2048 sequences); the longest-first prefill and the one-workgroup-per-tile
prefill (over 1024 tiles); the single-launch mixed batch; and the float32
kernels.
"""
import numpy as np
import pytest
import torch

import oracle

from tests.gpu_helpers import (DeviceStep, bits, oracle_decode, oracle_pool_after,
                               oracle_prefill, values)
from tests.position_code import PositionCoded
from workloads import build_decode_workload, make_workload

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _long_lens(seed, n=1024, lo=1100, hi=2100):
    return np.random.default_rng(seed).integers(lo, hi + 1, n)


def _many_tile_workload(dtype="bf16"):
    w = make_workload("mixed", dtype=dtype, seed=4243, num_decode=1, num_chunks=33,
                      chunk_len=512, max_prior=64, num_q_heads=16, num_kv_heads=2, head_dim=64,
                      dec_min=1, dec_max=100)
    rng = np.random.default_rng(6)
    lens = [512] + [int(x) for x in rng.integers(1, 41, 32)]
    q, qsl, ctx = [], [0], []
    for c, L in enumerate(lens):
        lo = int(w.query_start_loc[c])
        q.append(w.prefill_q[lo:lo + L])
        qsl.append(qsl[-1] + L)
        ctx.append(int(w.prefill_context_lens[c]) - 512 + L)
    # (the appended rows past a shortened context stay in the step: they land
    # in slots past the context, which no attention reads)
    w.prefill_q = np.concatenate(q)
    w.query_start_loc = np.array(qsl, np.int32)
    w.prefill_context_lens = np.array(ctx, np.int32)
    return w


# name -> (builder, PositionCoded kwargs)
CASES = {
    "gqa_bs16_cached_G8": (lambda dt: make_workload(
        "gqa", dtype=dt, num_seqs=24, median=300, hi=2100, num_q_heads=16, num_kv_heads=2), {}),
    "gqa_full_bs16_nt_G8": (lambda dt: make_workload("gqa", dtype=dt), {}),
    "mha_full_nt_G1": (lambda dt: make_workload("mha", dtype=dt), {}),
    "long_bs32_nt_G4": (lambda dt: build_decode_workload(
        "long32", 7301, _long_lens(7300), 8, 2, 128, 32, dt), {}),
    "long_bs16_d64_nt_G2": (lambda dt: build_decode_workload(
        "long16", 7303, _long_lens(7302), 4, 2, 64, 16, dt), {}),
    "bs32_d64_cached_G4": (lambda dt: build_decode_workload(
        "small32", 7305, np.random.default_rng(7304).integers(1, 3500, 40), 8, 2, 64, 32, dt),
        {}),
    "over2048_G2": (lambda dt: build_decode_workload(
        "over2048", 9102, np.random.default_rng(9103).integers(1, 1301, 2100), 4, 2, 64, 16,
        dt), {}),
    "prefix_full_shared": (lambda dt: make_workload("prefix", dtype=dt),
                           dict(prefix_len=1032, samples=8)),
    "mixed_full": (lambda dt: make_workload("mixed", dtype=dt), {}),
    "prefill_many_tiles": (lambda dt: _many_tile_workload(dt), {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_position_coded_outputs_are_exact(name):
    builder, kw = CASES[name]
    w = builder("bf16")
    _say(f"[case] position-coded {name}: B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads}"
         f" d={w.head_dim} bs={w.block_size} max_ctx={w.max_context_len}")
    pc = PositionCoded(w, 100 + len(name), **kw)
    st = DeviceStep(w)
    st.run()
    got = bits(st.out)
    want = pc.want_bits("decode")
    bad = np.argwhere((got != want).any(axis=2))
    _say(f"  decode: {len(bad)} of {got.shape[0] * got.shape[1]} rows differ")
    assert len(bad) == 0, f"first rows that differ (seq, head): {bad[:5].tolist()}, targets " \
                          f"{[int(pc.decode_targets[b, h]) for b, h in bad[:5]]}"
    if w.prefill_q is not None:
        pgot, pwant = bits(st.pout), pc.want_bits("prefill")
        pbad = np.argwhere((pgot != pwant).any(axis=2))
        _say(f"  prefill: {len(pbad)} of {pgot.shape[0] * pgot.shape[1]} rows differ")
        assert len(pbad) == 0, f"first rows that differ (query, head): {pbad[:5].tolist()}"
        # the same step in one pa_mixed_attention call
        out2, pout2 = torch.empty_like(st.out), torch.empty_like(st.pout)
        st.mixed(out2, pout2)
        torch.cuda.synchronize()
        assert np.array_equal(bits(out2), want)
        assert np.array_equal(bits(pout2), pwant)
    # the oracle agrees with the constructed answer on sampled rows
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([[0, w.num_seqs - 1], rng.choice(w.num_seqs, 6)]))
    pool_after = oracle_pool_after(w) if w.num_blocks * w.block_elems < 2e9 else None
    if pool_after is not None:
        o = oracle_decode(w, pool_after, idx)
        assert np.abs(o - pc.decode_want[idx]).max() < 1e-9


@pytest.mark.parametrize("name", ["gqa_bs16_cached_G8", "bs32_d64_cached_G4"])
def test_position_coded_float32(name):
    builder, kw = CASES[name]
    w = builder("f32")
    _say(f"[case] position-coded f32 {name}: B={w.num_seqs}")
    pc = PositionCoded(w, 200 + len(name), **kw)
    st = DeviceStep(w)
    st.run()
    assert np.array_equal(bits(st.out), pc.want_bits("decode"))


def _ulp_bf16(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _check_bound(got, o, ma, md, label):
    err = np.abs(got - o)
    bound = 2.0 ** -8 * np.abs(o) + (2.0 ** -8 + 2.0 ** -10) * ma + \
        (2.0 ** -7 + 2.0 ** -10) * md + 1e-6
    ulps = float((err / _ulp_bf16(o)).max())
    ratio = float((err / bound).max())
    _say(f"  {label}: max abs err {err.max():.3e}, max {ulps:.2f} output ulps, "
         f"worst err / bound {ratio:.3f}")
    assert np.isfinite(got).all()
    assert (err <= bound).all(), f"{int((err > bound).sum())} elements exceed the bound"


def _sharpen(w):
    """q x 8 (exact in bfloat16: a power of two)."""
    f = (w.q.astype(np.uint32) << 16).view(np.float32) * 8
    w.q = (f.view(np.uint32) >> 16).astype(np.uint16)
    if w.prefill_q is not None:
        f = (w.prefill_q.astype(np.uint32) << 16).view(np.float32) * 8
        w.prefill_q = (f.view(np.uint32) >> 16).astype(np.uint16)


SHARP = {
    "gqa_bs16_cached_G8": CASES["gqa_bs16_cached_G8"][0],
    "long_bs32_nt_G4": lambda dt: build_decode_workload(
        "long32s", 7311, _long_lens(7310, n=600, lo=2000, hi=3000), 8, 2, 128, 32, dt),
    "bs32_d64_cached_G4": CASES["bs32_d64_cached_G4"][0],
    "mha_G1": lambda dt: make_workload("mha", dtype=dt, num_seqs=12, min_len=1, max_len=3000,
                                       num_heads=4),
    "prefix_shared": lambda dt: make_workload(
        "prefix", dtype=dt, num_prompts=3, samples=4, prefix_len=1032, max_suffix=200,
        num_q_heads=8, num_kv_heads=2),
    "mixed_small": lambda dt: make_workload(
        "mixed", dtype=dt, num_decode=10, dec_min=1, dec_max=2500, num_chunks=4, chunk_len=100,
        max_prior=700, num_q_heads=8, num_kv_heads=2),
}


@pytest.mark.parametrize("name", list(SHARP))
def test_sharpened_within_the_rounding_bound(name):
    w = SHARP[name]("bf16")
    _sharpen(w)
    _say(f"[case] sharpened {name}: B={w.num_seqs} Hq={w.num_q_heads} d={w.head_dim} "
         f"bs={w.block_size} max_ctx={w.max_context_len}")
    st = DeviceStep(w)
    st.run()
    pool = oracle_pool_after(w)
    # long batches: a sample of sequences (every one with several partitions
    # among the first ones)
    idx = np.arange(w.num_seqs) if w.num_seqs <= 64 else \
        np.unique(np.random.default_rng(3).choice(w.num_seqs, 48, replace=False))
    o, ma, md = oracle.decode_moments(w.q[idx], pool, w.block_tables[idx], w.context_lens[idx],
                                      w.num_kv_heads, w.block_size, w.scale, w.dtype)
    _check_bound(values(st.out)[idx], o, ma, md, "decode")
    if w.prefill_q is not None:
        o, ma, md = oracle.prefill_moments(w.prefill_q, pool, w.prefill_block_tables,
                                           w.prefill_context_lens, w.query_start_loc,
                                           w.num_kv_heads, w.block_size, w.scale, w.dtype)
        _check_bound(values(st.pout), o, ma, md, "prefill")
        out2, pout2 = torch.empty_like(st.out), torch.empty_like(st.pout)
        st.mixed(out2, pout2)
        torch.cuda.synchronize()
        _check_bound(values(pout2), o, ma, md, "mixed launch, prefill")
        o, ma, md = oracle.decode_moments(w.q, pool, w.block_tables, w.context_lens,
                                          w.num_kv_heads, w.block_size, w.scale, w.dtype)
        _check_bound(values(out2), o, ma, md, "mixed launch, decode")
