#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Headline workload: the GQA long-tail decode batch -- 256 sequences, 64 query
heads / 8 KV heads, head_dim 128, block_size 16, bfloat16 with float32
accumulation, context lengths lognormal (median 800, ln-sigma 1) clipped to
[16, 8192], blocks placed by a seeded random permutation.

One step = one decode iteration over L layers (default 4, each its own pool so
repeated calls do not hit in the 256 MB last-level cache): per layer, append
every sequence's new token (pa_append_kv) and run paged decode attention
(pa_decode). Inputs are resident in HBM before timing starts. The step is
captured once into a HIP graph and the timed region is K replays of it between
two HIP events on the launch stream.

Reported (one JSON line on stdout):
  value      effective KV bandwidth = algorithmic K+V bytes attended / time, GB/s
             (each attended token's K and V read once per (sequence, kv head))
  roofline   pa_decode on the headline batch: algorithmic bytes per call / its
             mean duration (HIP events on the launch stream around graph
             replays of back-to-back calls over the layer pools; a call is one
             persistent kernel, which folds its split-K partitions itself), against
             8 TB/s and against a measured streaming rate (one pa_copy_blocks
             call of about 1.7 GB read + written); `traffic` is the HBM bytes
             per call measured with rocprofv3 counters for this exact kernel
             source (null otherwise)
  fused_step the same step with each layer's append and decode in one
             pa_decode_append call (bit-identical outputs and pool), timed per
             step against the two-call step in the same run, and one such call
  rows       every step of the hot path on its own workload: append, block copy,
             decode on the other batches, chunked prefill -- median time,
             algorithmic bytes or flops, fraction of the matching roofline, and
             the oracle's rate on a bounded sample of the same inputs; and the
             mixed iteration's decode and prefill in one pa_mixed_attention
             call. Every row cycles through enough copies of its buffers (at
             least 4, covering at least 1 GiB) that no call finds its data in
             the last-level cache from the call before.
  cpu_baseline  the fp64 NumPy oracle on full headline layers (BLAS on the
             process's affinity cores, the per-sequence loop on one)
  engine     the C++ block manager + iteration-level scheduler driving these
             kernels on a long-tail request stream, under paged allocation,
             Orca-style max-length reservation and static batching: output
             tokens/s, host time per iteration, decode KV GB/s of the loop

With --loop decode|prefill|mixed it measures nothing: it runs that call of the
mixed iteration back to back for --loop-seconds, a steady load for sampling
board power and clocks from outside (amd-smi), and prints calls and time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, vendor figure
PCIE_PEAK_GBS = 64.0       # PCIe Gen5 x16, nominal per direction (host link of the swap row)
METRIC = "paged decode attention: effective KV HBM GB/s (% of peak) and seq-layers/s"
WORKLOAD_DESC = {
    "gqa": "GQA long-tail decode: 256 seqs, 64 q / 8 kv heads, head_dim 128, block_size 16, "
           "bf16, context lengths lognormal(median 800, sigma 1) clipped [16, 8192]",
    "mha": "MHA decode (7B-like layer): 64 seqs, 32/32 heads, head_dim 128, block_size 16, "
           "bf16, context lengths uniform [128, 2048]",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pa_decode_gqa_longtail_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "paged_kv_cache_282_amd", "csrc", f)
                  for f in ("pa_kernels.hip", "pa_launch.h", "pa_api.cpp")]


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--workload", default="gqa", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip every oracle timing (headline and rows)")
    ap.add_argument("--rows-only", action="store_true",
                    help="skip the headline: only the rows named by --sections (and the engine "
                         "loop unless --no-engine), for profiling one workload's kernels alone; "
                         "the JSON line then carries no headline value")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the per-row measurements")
    ap.add_argument("--repeats", type=int, default=20, help="timed calls per batch, per row")
    ap.add_argument("--sections", default="prefix,prefix1024,mha,mixed,swap",
                    help="row groups to measure (comma list of prefix, prefix1024, mha, mixed, "
                         "swap)")
    ap.add_argument("--no-engine", action="store_true", help="skip the engine-loop rows")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the headline, copy half of the first layer's pool onto the "
                         "other half with one pa_copy_blocks call (a copy of known size for "
                         "scaling memory-traffic counters)")
    ap.add_argument("--loop", choices=("decode", "prefill", "mixed"),
                    help="instead of measuring, run one call of the mixed iteration (its "
                         "decode, its prefill, or both in one pa_mixed_attention call) back to "
                         "back for --loop-seconds, printing a line a second: a steady load for "
                         "sampling power and clocks from outside")
    ap.add_argument("--loop-seconds", type=float, default=20.0)
    return ap.parse_args()


def loop_calls(pa, torch, make_workload, which: str, seconds: float) -> dict:
    """One call of the mixed iteration back to back (pool after the iteration's append)."""
    w = make_workload("mixed")
    pool = to_dev(w.pool, w.dtype, torch)
    pa.pa_append_kv(pool, to_dev(w.k_new, w.dtype, torch), to_dev(w.v_new, w.dtype, torch),
                    i32(w.slot_mapping, torch), w.block_size)
    q, tables, lens = to_dev(w.q, w.dtype, torch), i32(w.block_tables, torch), \
        i32(w.context_lens, torch)
    out = torch.empty_like(q)
    ws = pa.new_decode_workspace(w.num_seqs, w.num_q_heads, w.head_dim, w.max_context_len)
    pq = to_dev(w.prefill_q, w.dtype, torch)
    pout = torch.empty_like(pq)
    pt, pl = i32(w.prefill_block_tables, torch), i32(w.prefill_context_lens, torch)
    qsl = i32(w.query_start_loc, torch)
    max_chunk = int(np.diff(w.query_start_loc).max())

    def decode():
        pa.pa_decode(out, q, pool, tables, lens, w.max_context_len, w.num_kv_heads,
                     w.block_size, w.scale, ws)

    def prefill():
        pa.pa_prefill_chunk(pout, pq, pool, pt, pl, qsl, max_chunk, w.num_kv_heads,
                            w.block_size, w.scale)

    def mixed():
        pa.pa_mixed_attention(out, q, tables, lens, w.max_context_len, pout, pq, pt, pl, qsl,
                              max_chunk, pool, w.num_kv_heads, w.block_size, w.scale, ws)

    fn = {"decode": decode, "prefill": prefill, "mixed": mixed}[which]
    fn()
    torch.cuda.synchronize()
    log(f"looping {which} for {seconds:.0f} s")
    n, t0, last = 0, time.time(), time.time()
    while time.time() - t0 < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
        n += 20
        if time.time() - last >= 1.0:
            last = time.time()
            log(f"  {which}: {n} calls, {(last - t0) / n * 1e6:.1f} us per call")
    dt = time.time() - t0
    return {"loop": which, "calls": n, "seconds": round(dt, 2),
            "us_per_call": round(dt / n * 1e6, 1),
            "workload": "mixed iteration (240 decode seqs, 16 prefill chunks x 512), "
                        "pool after its append"}


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per pa_decode call on the headline batch, from the committed
    rocprofv3 counter summary, if it was taken on the kernel source built now."""
    try:
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if line.startswith("RESULT "):
                    rec = json.loads(line[len("RESULT "):])
                    if rec.get("kernel_source_sha256") == kernel_source_hash():
                        return rec
    except OSError:
        pass
    return None


def to_dev(arr, dtype, torch):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).cuda()


def i32(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def time_calls(fn, torch, repeats: int, warmup: int = 3, batches: int = 9):
    """Median / p10 / p90 / mean duration (ms) per call of fn(), and how it was timed.

    The calls are captured once into a HIP graph of `repeats` back-to-back
    calls, which is replayed `batches` times between HIP events, so that short
    kernels are not timed together with the host's launch cost. (The library's
    calls enqueue kernels only: no memsets, no host synchronisation.) The
    statistics are over the batches' per-call averages. If capture is not
    available, the calls run back to back from the host instead.
    """
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(warmup):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    how = "hip graph of back-to-back calls"
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(repeats):
                fn()
        run = g.replay
    except Exception as e:  # pragma: no cover - depends on the runtime
        log(f"graph capture unavailable ({e}); timing host-launched calls")
        how = "host-launched back-to-back calls"

        def run():
            for _ in range(repeats):
                fn()
    run()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(batches)]
    for a, b in ev:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) / repeats for a, b in ev])
    return (float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90)), how,
            float(t.mean()))


# Bytes one rotation of a row's buffers must cover: four times the 256 MB
# last-level cache, so that a call never finds its data there from the call
# before.
ROTATE_BYTES = 1 << 30


def rotations(bytes_per_call: float, lo: int = 4, hi: int = 48) -> int:
    """How many copies of a row's buffers to cycle through."""
    return int(min(hi, max(lo, -(-ROTATE_BYTES // max(1, int(bytes_per_call))))))


def kv_bytes(w) -> float:
    return float(w.context_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_dim \
        * w.elem_bytes


def host_cores() -> int:
    """The host cores this process may run on (its CPU affinity)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def cpu_baseline(w, gpu_out0: np.ndarray, min_seconds: float = 10.0, max_reps: int = 24) -> dict:
    """Time the fp64 oracle on full layers (append + decode of every sequence),
    repeated until at least `min_seconds` of CPU work. BLAS may use every core
    of the process's affinity set; the oracle's loop over sequences and heads
    is plain Python on one of them."""
    import oracle
    from threadpoolctl import threadpool_limits

    cores = host_cores()
    reps, dt, ref = 0, 0.0, None
    with threadpool_limits(cores):
        while reps < max_reps and (reps == 0 or dt < min_seconds):
            t0 = time.perf_counter()
            pool_after = oracle.append(w.pool, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads,
                                       w.block_size, w.head_dim)
            ref = oracle.decode(w.q, pool_after, w.block_tables, w.context_lens, w.num_kv_heads,
                                w.block_size, w.scale, w.dtype)
            dt += time.perf_counter() - t0
            reps += 1
    err = float(np.abs(gpu_out0 - ref).max())
    return {"value": round(kv_bytes(w) * reps / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} repetition{'s' if reps != 1 else ''} of one full layer "
                      f"(append of {w.num_seqs} tokens + "
                      f"decode of all {w.num_seqs} sequences), fp64 NumPy, BLAS limited to "
                      f"{cores} threads (the affinity set), Python loop over "
                      f"sequences and heads on one thread",
            "seconds": round(dt, 3), "seq_layers_per_s": round(w.num_seqs * reps / dt, 2),
            "gpu_vs_oracle_max_abs_err": err}


# -- per-row measurements -------------------------------------------------------------

class Rows:
    """Each step of the hot path on its own workload, against its own roofline."""

    def __init__(self, pa, torch, repeats: int, oracle_on: bool, measured_peak=None):
        self.pa, self.torch, self.repeats, self.oracle_on = pa, torch, repeats, oracle_on
        self.measured_peak = measured_peak
        self.cores = host_cores()
        self.out = {}

    def _oracle(self, fn, amount: float, unit: str, sample: str) -> dict | None:
        if not self.oracle_on:
            return None
        from threadpoolctl import threadpool_limits
        with threadpool_limits(self.cores):
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
        return {"value": round(amount / dt, 4), "unit": unit, "cores": self.cores,
                "kind": "oracle", "sample": sample, "seconds": round(dt, 3)}

    def _record(self, key, kernel, workload, ms, amount, unit, peak, bound, oracle=None,
                rotated=None, **extra):
        med, p10, p90, how, mean = ms
        scale = 1e9 if unit == "GB/s" else 1e12
        achieved = amount / (med * 1e-3) / scale
        self.out[key] = {"kernel": kernel, "workload": workload,
                         "us": round(med * 1e3, 2), "us_stat": "median",
                         "us_p10": round(p10 * 1e3, 2), "us_p90": round(p90 * 1e3, 2),
                         "us_mean": round(mean * 1e3, 2), "timing": how,
                         "rotated_pools": rotated,
                         "algorithmic": amount, "achieved": round(achieved, 2), "unit": unit,
                         "peak": peak, "bound": bound, "frac": round(achieved / peak, 4),
                         "cpu_oracle": oracle, **extra}
        if unit == "GB/s" and self.measured_peak:
            self.out[key]["frac_of_measured_copy_peak"] = round(achieved / self.measured_peak, 4)
        log(f"  {key:28s} {med * 1e3:9.1f} us  {achieved:9.1f} {unit}  "
            f"({100 * achieved / peak:.1f}% of {peak:.0f}; {rotated} rotated buffer sets)")

    def device(self, w):
        t, pa = self.torch, self.pa
        d = {"pool": to_dev(w.pool, w.dtype, t), "q": to_dev(w.q, w.dtype, t),
             "k_new": to_dev(w.k_new, w.dtype, t), "v_new": to_dev(w.v_new, w.dtype, t),
             "slots": i32(w.slot_mapping, t), "tables": i32(w.block_tables, t),
             "lens": i32(w.context_lens, t), "pairs": i32(w.copy_pairs.reshape(-1, 2), t)}
        d["out"] = t.empty_like(d["q"])
        d["ws"] = pa.new_decode_workspace(w.num_seqs, w.num_q_heads, w.head_dim,
                                          w.max_context_len)
        d["pools"] = [d["pool"]]
        return d

    def rotate(self, d, n: int) -> int:
        """Give d n device copies of its pool (they stay equal: every timed call
        writes the same bytes to each). Returns n."""
        while len(d["pools"]) < n:
            d["pools"].append(d["pool"].clone())
        return n

    def cycled(self, fn, n: int):
        """fn(i) for i = 0, 1, ... mod n, one step per call (the graph captures
        the calls in order, so its replays cycle through the n buffer sets)."""
        k = [0]

        def call():
            fn(k[0] % n)
            k[0] += 1
        return call

    def reps(self, n: int) -> int:
        return max(self.repeats, n) // n * n  # a whole number of rotations per replay

    def decode_row(self, key, w, d, desc, unique_bytes=None, hint=None):
        """hint: the share_prev array; the row then times pa_decode_shared."""
        pa = self.pa
        n = self.rotate(d, rotations(unique_bytes or kv_bytes(w)))
        outs = [d["out"]] + [self.torch.empty_like(d["out"]) for _ in range(n - 1)]
        share = None if hint is None else i32(hint, self.torch)

        def call(i):
            if share is None:
                pa.pa_decode(outs[i], d["q"], d["pools"][i], d["tables"], d["lens"],
                             w.max_context_len, w.num_kv_heads, w.block_size, w.scale, d["ws"])
            else:
                pa.pa_decode_shared(outs[i], d["q"], d["pools"][i], d["tables"], d["lens"],
                                    share, w.max_context_len, w.num_kv_heads, w.block_size,
                                    w.scale, d["ws"])

        ms = time_calls(self.cycled(call, n), self.torch, self.reps(n))
        ns = min(16, w.num_seqs)
        sample_bytes = float(w.context_lens[:ns].astype(np.int64).sum()) * 2 * w.num_kv_heads \
            * w.head_dim * w.elem_bytes

        def orc():
            import oracle
            oracle.decode(w.q[:ns], w.pool, w.block_tables[:ns], w.context_lens[:ns],
                          w.num_kv_heads, w.block_size, w.scale, w.dtype)

        extra = {}
        if share is not None:
            # the same call without the hint, on the same pool: bit-identical
            plain = self.torch.empty_like(d["out"])
            call(0)
            pa.pa_decode(plain, d["q"], d["pools"][0], d["tables"], d["lens"], w.max_context_len,
                         w.num_kv_heads, w.block_size, w.scale, d["ws"])
            self.torch.cuda.synchronize()
            extra["bit_identical_to_pa_decode"] = bool(self.torch.equal(
                outs[0].view(self.torch.int16), plain.view(self.torch.int16)))
            extra["hint"] = ("share_prev from the tables: leading table entries each sequence "
                             "has in common with the one before it")
        if unique_bytes is not None:
            extra["unique_bytes"] = unique_bytes
            extra["achieved_unique"] = round(unique_bytes / (ms[0] * 1e-3) / 1e9, 2)
            extra["frac_unique"] = round(unique_bytes / (ms[0] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        self._record(key, "pa_decode" if share is None else "pa_decode_shared", desc, ms,
                     kv_bytes(w), "GB/s", HBM_PEAK_GBS, "hbm",
                     self._oracle(orc, sample_bytes / 1e9, "GB/s",
                                  f"decode of the first {ns} sequences (pool after the step's "
                                  f"copy and append), fp64 NumPy, {self.cores} BLAS threads"),
                     rotated=n, **extra)

    def prefix_rows(self, make_workload, prefix_len: int, suffix: str):
        """Copy-on-write, then decode over the shared blocks, of the shared-prefix batch."""
        import oracle
        pa = self.pa
        w = make_workload("prefix", prefix_len=prefix_len)
        d = self.device(w)
        blk_bytes = w.block_elems * w.elem_bytes
        P = len(w.copy_pairs)
        if P:
            n = self.rotate(d, rotations(2.0 * P * blk_bytes))

            def copy(i):
                pa.pa_copy_blocks(d["pools"][i], d["pairs"], w.num_kv_heads, w.head_dim,
                                  w.block_size)

            for i in range(n):
                copy(i)
            ms = time_calls(self.cycled(copy, n), self.torch, self.reps(n))
            self._record("a2_copy_blocks" + suffix, "pa_copy_blocks",
                         f"shared-prefix CoW: {P} pairs of {blk_bytes // 1024} KiB blocks", ms,
                         2.0 * P * blk_bytes, "GB/s", HBM_PEAK_GBS, "hbm",
                         self._oracle(lambda: oracle.copy_blocks(w.pool, w.copy_pairs),
                                      2.0 * P * blk_bytes / 1e9, "GB/s",
                                      f"all {P} pairs, NumPy block copy (the oracle snapshots "
                                      "the pool first), 1 thread"), rotated=n)
        for pool in d["pools"]:
            pa.pa_append_kv(pool, d["k_new"], d["v_new"], d["slots"], w.block_size)
        self.torch.cuda.synchronize()
        pool_np = oracle.copy_blocks(w.pool, w.copy_pairs)
        pool_np = oracle.append(pool_np, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads,
                                w.block_size, w.head_dim)
        w.pool = pool_np  # the oracle sample below attends to the pool after the step
        uniq = np.unique(np.concatenate([row[: -(-int(n) // w.block_size)]
                                         for row, n in zip(w.block_tables, w.context_lens)]))
        unique_bytes = float(len(uniq)) * blk_bytes
        desc = (f"shared-prefix decode: 32 prompts x 8 samples, prefix {prefix_len}, "
                f"suffix U[1,512], 32 q / 8 kv heads, bf16, {P} copy pairs")
        self.decode_row("a3_a7_decode_prefix" + suffix, w, d, desc, unique_bytes=unique_bytes)
        from workloads import share_prev_hint
        self.decode_row("a3_a7_decode_prefix_shared" + suffix, w, d,
                        desc + "; pa_decode_shared with the sharing hint", unique_bytes=unique_bytes,
                        hint=share_prev_hint(w.block_tables, w.context_lens, w.block_size))

    def run(self, make_workload, sections=("prefix", "prefix1024", "mha", "mixed", "swap")):
        # -- shared-prefix batch: the 1032-token reading (a half-full shared last
        # prefix block, copied on the first divergent write), then the literal
        # 1024-token prefix (whole blocks only: nothing to copy) ------------------
        if "prefix" in sections:
            self.prefix_rows(make_workload, 1032, "")
            self.torch.cuda.empty_cache()
        if "prefix1024" in sections:
            self.prefix_rows(make_workload, 1024, "_len1024")
            self.torch.cuda.empty_cache()
        if "mha" in sections:
            self.mha_rows(make_workload)
        if "mixed" in sections:
            self.mixed_rows(make_workload)
        if "swap" in sections:
            self.swap_rows(make_workload)
        return self.out

    def mha_rows(self, make_workload):
        import oracle
        pa = self.pa
        w = make_workload("mha")
        d = self.device(w)
        pa.pa_append_kv(d["pool"], d["k_new"], d["v_new"], d["slots"], w.block_size)
        w.pool = oracle.append(w.pool, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads,
                               w.block_size, w.head_dim)
        self.decode_row("a3_a7_decode_mha", w, d, WORKLOAD_DESC["mha"])
        del d, w
        self.torch.cuda.empty_cache()

    def mixed_rows(self, make_workload):
        """The mixed iteration: append of 8432 tokens, decode, chunked prefill,
        and the decode and prefill together in one pa_mixed_attention call."""
        import oracle
        pa = self.pa
        w = make_workload("mixed")
        d = self.device(w)
        T = len(w.slot_mapping)
        row_bytes = T * w.num_kv_heads * w.head_dim * w.elem_bytes
        n = self.rotate(d, rotations(4.0 * row_bytes))
        kvs = [(d["k_new"], d["v_new"])] + [(d["k_new"].clone(), d["v_new"].clone())
                                            for _ in range(n - 1)]

        def append(i):
            pa.pa_append_kv(d["pools"][i], kvs[i][0], kvs[i][1], d["slots"], w.block_size)

        for i in range(n):
            append(i)
        ms = time_calls(self.cycled(append, n), self.torch, self.reps(n))
        self._record("a1_append_kv", "pa_append_kv",
                     f"mixed iteration: {T} new tokens (16 x 512 prefill + 240 decode), "
                     "8 kv heads, head_dim 128, block_size 32, bf16", ms,
                     4.0 * row_bytes, "GB/s", HBM_PEAK_GBS, "hbm",
                     self._oracle(lambda: oracle.append(w.pool, w.k_new, w.v_new, w.slot_mapping,
                                                        w.num_kv_heads, w.block_size, w.head_dim),
                                  4.0 * row_bytes / 1e9, "GB/s",
                                  f"all {T} tokens, NumPy scatter, 1 thread"),
                     rotated=n,
                     bytes_note="K and V rows read from k_new/v_new and written to the pool; "
                                "each rotated set has its own pool and k_new/v_new")
        del kvs
        w.pool = oracle.append(w.pool, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads,
                               w.block_size, w.head_dim)
        self.decode_row("a3_a7_decode_mixed", w, d,
                        "mixed iteration decode: 240 seqs U[256,4096], 32 q / 8 kv heads, "
                        "head_dim 128, block_size 32, bf16")
        pq = to_dev(w.prefill_q, w.dtype, self.torch)
        pt, pl = i32(w.prefill_block_tables, self.torch), i32(w.prefill_context_lens, self.torch)
        qsl = i32(w.query_start_loc, self.torch)
        pout = self.torch.empty_like(pq)
        Lc = np.diff(w.query_start_loc)
        max_chunk = int(Lc.max())
        npool = len(d["pools"])

        def prefill(i):
            pa.pa_prefill_chunk(pout, pq, d["pools"][i], pt, pl, qsl, max_chunk, w.num_kv_heads,
                                w.block_size, w.scale)

        ms = time_calls(self.cycled(prefill, npool), self.torch, self.reps(npool))
        keys = 0
        for c in range(len(Lc)):
            nc, L = int(w.prefill_context_lens[c]), int(Lc[c])
            keys += L * (nc - L) + L * (L + 1) // 2  # query i attends to n - L + i + 1 keys
        flops = 4.0 * w.head_dim * w.num_q_heads * keys

        def orc():
            oracle.prefill(w.prefill_q[: int(Lc[0])], w.pool, w.prefill_block_tables[:1],
                           w.prefill_context_lens[:1], w.query_start_loc[:2], w.num_kv_heads,
                           w.block_size, w.scale, w.dtype)

        n0, L0 = int(w.prefill_context_lens[0]), int(Lc[0])
        flops0 = 4.0 * w.head_dim * w.num_q_heads * (L0 * (n0 - L0) + L0 * (L0 + 1) // 2)
        self._record("a8_prefill_chunk", "pa_prefill_chunk",
                     f"mixed iteration prefill: {len(Lc)} chunks x {max_chunk} queries, prior "
                     "U[0,2048], causal, 32 q / 8 kv heads, bf16", ms, flops, "TFLOP/s",
                     MFMA_BF16_PEAK_TFLOPS, "mfma",
                     self._oracle(orc, flops0 / 1e12, "TFLOP/s",
                                  f"chunk 0 only (512 queries), fp64 NumPy, {self.cores} BLAS "
                                  "threads"),
                     rotated=npool, flops_note="4*d per (query, head, attended key): q.k and p.v")

        # -- the same decode batch and prefill chunks in one pa_mixed_attention call --------
        out2, pout2 = self.torch.empty_like(d["out"]), self.torch.empty_like(pout)

        def mixed(i):
            pa.pa_mixed_attention(out2, d["q"], d["tables"], d["lens"], w.max_context_len, pout2,
                                  pq, pt, pl, qsl, max_chunk, d["pools"][i], w.num_kv_heads,
                                  w.block_size, w.scale, d["ws"])

        ms = time_calls(self.cycled(mixed, npool), self.torch, self.reps(npool))
        sep = self.out["a3_a7_decode_mixed"]["us"] + self.out["a8_prefill_chunk"]["us"]
        bound_us = max(kv_bytes(w) / (HBM_PEAK_GBS * 1e9), flops / (MFMA_BF16_PEAK_TFLOPS * 1e12))
        self._record("f2_mixed_single_launch", "pa_mixed_attention",
                     "mixed iteration decode + prefill in one call (the two rows above)", ms,
                     kv_bytes(w), "GB/s", HBM_PEAK_GBS, "hbm", rotated=npool,
                     separate_us=round(sep, 2),
                     speedup_vs_separate=round(sep / (ms[0] * 1e3), 3),
                     roofline_us=round(bound_us * 1e6, 2),
                     roofline_note="max(decode K+V bytes / 8 TB/s, prefill flops / 2.5 "
                                   "PFLOP/s): the time if both parts ran at peak, fully "
                                   "overlapped; frac counts the decode bytes only",
                     frac_of_overlap_bound=round(bound_us * 1e6 / (ms[0] * 1e3), 4),
                     prefill_flops=flops)
        del d, w, pq, pout, out2, pout2
        self.torch.cuda.empty_cache()

    def swap_rows(self, make_workload):
        """1024 blocks of 64 KiB out to pinned host memory and back."""
        import oracle
        pa = self.pa
        w = make_workload("gqa")
        pool = to_dev(w.pool, w.dtype, self.torch)
        E = w.block_elems
        n = 1024
        host = self.torch.empty(n * E, dtype=pool.dtype).pin_memory()
        rng = np.random.default_rng(1)
        src = rng.choice(w.num_blocks, n, replace=False).astype(np.int32)
        out_pairs = i32(np.stack([src, np.arange(n, dtype=np.int32)], 1), self.torch)
        in_pairs = i32(np.stack([np.arange(n, dtype=np.int32), src], 1), self.torch)
        nbytes = float(n * E * w.elem_bytes)
        for key, pairs, direction, what in (("f3_swap_out", out_pairs, pa.SWAP_OUT, "device -> host"),
                                            ("f3_swap_in", in_pairs, pa.SWAP_IN, "host -> device")):
            def swap(pairs=pairs, direction=direction):
                pa.pa_swap_blocks(pool, host, pairs, direction, w.num_kv_heads, w.head_dim,
                                  w.block_size)

            ms = time_calls(swap, self.torch, self.repeats)
            self._record(key, "pa_swap_blocks", f"{n} blocks of 64 KiB (64 MiB), {what}, "
                         "pinned host memory", ms, nbytes, "GB/s", PCIE_PEAK_GBS, "host link",
                         self._oracle(lambda: oracle.swap_blocks(w.pool[src], w.pool[src],
                                                                 np.stack([np.arange(n)] * 2, 1),
                                                                 0 if direction == 0 else 1),
                                      nbytes / 1e9, "GB/s",
                                      f"all {n} blocks, NumPy block copy, 1 thread"),
                         peak_note="PCIe Gen5 x16 nominal, per direction")
        del pool, host


ENGINE_DESC = ("iteration-level serving loop (no model weights): 1024 requests arriving at "
               "once, prompts U[32, 512], outputs round(lognormal(median 128, sigma 1)) "
               "clipped [1, 1536], 20% of requests with 4 parallel samples; 32 q / 8 kv heads, "
               "head_dim 128, block_size 16, bf16; pool 8192 blocks (512 MB); at most 256 "
               "running samples, 2048 tokens and 512-token prefill chunks per iteration, "
               "max_len 2048 (reservation: 128 blocks per sample); the paged policy also on "
               "a 3072-block pool, evicting by recomputation or by swapping to pinned host memory; "
               "and a second stream whose requests name one of 16 shared 512-token prompt "
               "prefixes (suffixes U[32, 256], outputs clipped at 1280), with and without prefix "
               "caching")


def engine_rows(pa, torch, oracle_on: bool) -> dict:
    """The C++ engine loop under the three policies on one request stream.

    tokens/s counts each request's output tokens once (work lost to eviction
    is not counted); wall time runs from the first iteration to the final
    stream synchronisation, host scheduling and kernel time together. The
    host's own time (planning, packing, enqueueing) is reported apart from
    the time it waits for the device to free a ring slot.
    """
    from paged_kv_cache_282_amd import runtime
    from workloads.requests import make_request_stream

    cfg = dict(num_blocks=8192, block_size=16, max_seqs=256, max_tokens=2048, max_chunk=512,
               max_len=2048)
    HQ, HKV, D = 32, 8, 128
    reqs = make_request_stream(282, 1024, prompt=(32, 512), multi_frac=0.2, samples=4,
                               output_lognormal=(128, 1.0, 1536))
    order = np.random.default_rng(282).permutation(cfg["num_blocks"])
    T, S = cfg["max_tokens"], cfg["max_seqs"]
    g = torch.Generator(device="cuda").manual_seed(282)
    pool = torch.randn(cfg["num_blocks"] * 2 * HKV * cfg["block_size"] * D, generator=g,
                       device="cuda").bfloat16()
    k, v = (torch.randn(T, HKV, D, generator=g, device="cuda").bfloat16() for _ in range(2))
    qp = torch.randn(T, HQ, D, generator=g, device="cuda").bfloat16()
    qd = torch.randn(S, HQ, D, generator=g, device="cuda").bfloat16()
    outp, outd = torch.empty_like(qp), torch.empty_like(qd)
    scale = 1.0 / np.sqrt(D)

    # a second stream for prefix caching: 16 shared 512-token prompt prefixes
    preqs = make_request_stream(283, 1024, prompt=(32, 256), multi_frac=0.2, samples=4,
                                output_lognormal=(128, 1.0, 1280), prefix_groups=16,
                                prefix_tokens=512)

    def run(policy, stream_reqs, num_blocks=None, host_blocks=0, prefix=False):
        c = dict(cfg, num_blocks=num_blocks or cfg["num_blocks"], num_host_blocks=host_blocks,
                 prefix_caching=prefix)
        ws = pa.new_decode_workspace(S, HQ, D, cfg["max_len"])
        sched = runtime.Scheduler(policy=policy, requests=stream_reqs, **c,
                                  free_order=order if num_blocks is None
                                  else np.random.default_rng(282).permutation(num_blocks))
        blk = 2 * HKV * cfg["block_size"] * D
        eng = runtime.Engine(sched, pool[: c["num_blocks"] * blk], HKV, qp, qd, k, v, outp, outd,
                             ws, scale)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st = eng.run()
        wall = time.perf_counter() - t0
        eng.close()
        sched.close()
        return st, wall

    run("paged", reqs[:64])   # first launches of every kernel, outside the timed runs
    out = {"workload": ENGINE_DESC, "output_tokens": sum(sum(x[1]) for x in reqs),
           "prefix_stream_output_tokens": sum(sum(x[1]) for x in preqs), "policies": {}}
    # the paged policy again on a pool of 3072 blocks (192 MB), where it must
    # evict: dropping and recomputing victims, or swapping them to 4096
    # pinned host blocks (256 MB)
    # and the paged policy on the prefix stream, without and with prefix caching
    runs = [("paged", "paged", reqs, None, 0, False), ("reserve", "reserve", reqs, None, 0, False),
            ("static", "static", reqs, None, 0, False),
            ("paged_3072_recompute", "paged", reqs, 3072, 0, False),
            ("paged_3072_swap", "paged", reqs, 3072, 4096, False),
            ("prefix_stream_paged", "paged", preqs, None, 0, False),
            ("prefix_stream_paged_cached", "paged", preqs, None, 0, True)]
    for name, policy, rq, nblk, hblk, prefix in runs:
        st, wall = run(policy, rq, nblk, hblk, prefix)
        want = sum(sum(x[1]) for x in rq)
        kv = st["decode_context_tokens"] * 2 * HKV * D * 2
        it = st["iterations"]
        out["policies"][name] = {
            "tokens_per_s": round(want / wall, 1), "wall_ms": round(wall * 1e3, 2),
            "iterations": it, "us_per_iteration": round(wall * 1e6 / it, 2),
            "host_us_per_iteration": round(st["host_us"] / it, 2),
            "host_fraction": round(st["host_us"] * 1e-6 / wall, 4),
            "host_wait_fraction": round(st["wait_us"] * 1e-6 / wall, 4),
            "mean_decodes_per_iteration": round(st["decode_tokens"] / it, 1),
            "generated": st["generated"], "evictions": st["evictions"],
            "copies": st["copies"], "prefill_tokens": st["prefill_tokens"],
            "swapped_blocks": st["swapped_blocks"],
            "decode_kv_GBps": round(kv / wall / 1e9, 1),
            "decode_kv_frac_of_hbm_peak": round(kv / wall / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"  engine {name:20s} {want / wall:10.0f} tok/s  {it:6d} iterations  "
            f"{wall * 1e3:8.1f} ms  host {st['host_us'] / it:6.1f} us/iter  "
            f"decode KV {kv / wall / 1e9:7.1f} GB/s  evictions {st['evictions']}  "
            f"swapped {st['swapped_blocks']}")
    pol = out["policies"]
    out["paged_vs_static"] = round(pol["paged"]["tokens_per_s"] / pol["static"]["tokens_per_s"], 2)
    out["reserve_vs_static"] = round(pol["reserve"]["tokens_per_s"]
                                     / pol["static"]["tokens_per_s"], 2)
    if oracle_on:
        from oracle.scheduler import SchedConfig, Scheduler
        t0 = time.perf_counter()
        plans = Scheduler(SchedConfig(policy="paged", **cfg), order, reqs).run()
        dt = time.perf_counter() - t0
        agree = (len(plans) == pol["paged"]["iterations"] and
                 sum(p.generated for p in plans) == pol["paged"]["generated"] and
                 sum(len(p.preempted) for p in plans) == pol["paged"]["evictions"])
        out["cpu_oracle"] = {"value": round(len(plans) / dt, 1), "unit": "iterations/s",
                             "cores": 1, "kind": "oracle",
                             "sample": "the paged policy's whole schedule (plans only, no "
                                       "attention), pure Python",
                             "seconds": round(dt, 2), "native_plan_totals_agree": agree,
                             "native_host_iterations_per_s": round(
                                 1e6 / pol["paged"]["host_us_per_iteration"], 1)}
        log(f"  oracle scheduler: {len(plans)} iterations in {dt:.1f} s, totals agree: {agree}")
    del pool
    return out


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this "
              "library has no multi-GPU path", file=sys.stderr)
        return 2

    import torch

    import paged_kv_cache_282_amd as pa
    from workloads import make_workload

    if not os.path.exists(pa.lib_path()):
        from paged_kv_cache_282_amd.build import build
        build()
    pa.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.loop:
        print(json.dumps(loop_calls(pa, torch, make_workload, args.loop, args.loop_seconds)),
              flush=True)
        return 0

    if args.rows_only:
        result = {"metric": METRIC, "value": None, "unit": "GB/s", "n_gpus": 1,
                  "rows_only": True, "dtype": "bf16", "data": "synthetic"}
        result["rows"] = Rows(pa, torch, args.repeats, not args.no_cpu_baseline).run(
            make_workload, args.sections.split(","))
        if not args.no_engine:
            result["engine"] = engine_rows(pa, torch, not args.no_cpu_baseline)
        print(json.dumps(result), flush=True)
        return 0

    t = time.time()
    w = make_workload(args.workload)
    log(f"workload {args.workload}: B={w.num_seqs} tokens={int(w.context_lens.sum())} "
        f"pool={w.pool.nbytes / 1e9:.2f} GB (generated in {time.time() - t:.1f}s)")
    L = args.layers
    pool0 = to_dev(w.pool, w.dtype, torch)
    pools = [pool0] + [pool0.clone() for _ in range(L - 1)]
    q = to_dev(w.q, w.dtype, torch)
    k_new = to_dev(w.k_new, w.dtype, torch)
    v_new = to_dev(w.v_new, w.dtype, torch)
    slots, tables, lens = i32(w.slot_mapping, torch), i32(w.block_tables, torch), \
        i32(w.context_lens, torch)
    outs = [torch.empty_like(q) for _ in range(L)]
    ws = pa.new_decode_workspace(w.num_seqs, w.num_q_heads, w.head_dim, w.max_context_len)
    max_ctx, hkv, bs, scale = w.max_context_len, w.num_kv_heads, w.block_size, w.scale
    torch.cuda.synchronize()

    def append(l):
        pa.pa_append_kv(pools[l], k_new, v_new, slots, bs)

    def decode(l):
        pa.pa_decode(outs[l], q, pools[l], tables, lens, max_ctx, hkv, bs, scale, ws)

    def step():
        for l in range(L):
            append(l)
            decode(l)

    # One step (every layer's append + decode) is captured once into a HIP
    # graph, as a serving loop would launch it; the library's calls enqueue
    # kernels only (no memsets, no host synchronisation), so replays are exact.
    # The timed region is K replays between two events on the launch stream.
    launch_how = "hip graph of one step (every layer's append + decode), replayed"
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    try:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        run_step = graph.replay
    except Exception as e:  # pragma: no cover - depends on the runtime
        log(f"graph capture unavailable ({e}); timing host-launched steps")
        launch_how = "host-launched steps"
        run_step = step
    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # timed region: K whole steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        run_step()
    ev1.record()
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # Per-call durations: a graph of back-to-back calls (cycling the layer
    # pools, so no call finds its pool in a cache), replayed between events.
    k = [0]

    def decode_next():
        decode(k[0] % L)
        k[0] += 1

    def append_next():
        append(k[0] % L)
        k[0] += 1

    dec = time_calls(decode_next, torch, 4 * L)
    app = time_calls(append_next, torch, 4 * L)
    decode_ms, append_ms = dec[0], app[0]
    dec_p10, dec_p90 = dec[1], dec[2]

    # The same step with each layer's append and decode in one call
    # (pa_decode_append, bit-identical outputs and pool): the whole step as a
    # graph, and one call, both timed like the rows above. Reported beside the
    # headline, which keeps the two calls of the step as the pages describe it.
    def fused_step():
        for l in range(L):
            pa.pa_decode_append(outs[l], q, pools[l], tables, lens, k_new, v_new, slots, max_ctx,
                                hkv, bs, scale, ws)

    def fused_next():
        l = k[0] % L
        pa.pa_decode_append(outs[l], q, pools[l], tables, lens, k_new, v_new, slots, max_ctx,
                            hkv, bs, scale, ws)
        k[0] += 1

    fstep = time_calls(fused_step, torch, 2)
    fcall = time_calls(fused_next, torch, 4 * L)
    split_step = time_calls(step, torch, 2)

    # A measured streaming rate beside the vendor figure: one pa_copy_blocks
    # call copying half of the first layer's pool onto its other half (pairs
    # (j, half + j): disjoint, inside the pool), far more than the 256 MB
    # last-level cache holds; bytes read + bytes written per call.
    half = w.num_blocks // 2
    cpairs = torch.stack([torch.arange(half, dtype=torch.int32),
                          torch.arange(half, 2 * half, dtype=torch.int32)], 1).contiguous().cuda()
    cbytes = half * w.block_elems * w.elem_bytes

    def big_copy():
        pa.pa_copy_blocks(pools[0], cpairs, hkv, w.head_dim, bs)

    cp = time_calls(big_copy, torch, 4)
    copy_peak = 2.0 * cbytes / (cp[0] * 1e-3) / 1e9
    log(f"measured copy rate: {cbytes / 1e6:.0f} MB read + written in {cp[0] * 1e3:.1f} us "
        f"-> {copy_peak:.0f} GB/s")

    kv_bytes_layer = kv_bytes(w)
    value = kv_bytes_layer * L / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes_layer / (decode_ms * 1e-3) / 1e9
    traffic = measured_traffic() if args.workload == "gqa" else None
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOAD_DESC[args.workload], "layers": L,
                   "step": "per layer: pa_append_kv (1 token/seq) + pa_decode",
                   "kv_bytes_per_layer": int(kv_bytes_layer)},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_layers_per_s": round(w.num_seqs * L / (ms_per_step * 1e-3), 1),
        "fused_step": {"entry": "pa_decode_append (per layer: the append and the decode in one "
                                "launch; outputs and pool bit-identical to the two calls)",
                       "ms_per_step": round(fstep[0], 4),
                       "split_ms_per_step": round(split_step[0], 4),
                       "timing": "per step, median of graph replays of two back-to-back steps; "
                                 "both forms in the same run",
                       "pa_decode_append_ms": round(fcall[0], 4),
                       "value": round(kv_bytes(w) * L / (fstep[0] * 1e-3) / 1e9, 2)},
        "kernels_ms": {"pa_decode": round(decode_ms, 4),
                       "pa_decode_p10": round(dec_p10, 4),
                       "pa_decode_p90": round(dec_p90, 4),
                       "pa_decode_mean": round(dec[4], 4),
                       "pa_append_kv": round(append_ms, 4),
                       "stat": "median over graph replays",
                       "timing": f"{dec[3]}, cycling {L} layer pools"},
        "launch": launch_how,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["hbm_bytes_per_call"],
                     "kernel": "pa_decode = decode_bf16_persistent_kernel<128,16> (one "
                               "launch: split-K partitions are folded inside it)",
                     "algorithmic_bytes_per_launch": int(kv_bytes_layer),
                     "measured_peak": round(copy_peak, 1),
                     "frac_of_measured_peak": round(achieved / copy_peak, 4),
                     "measured_peak_note": f"pa_copy_blocks of {cbytes / 1e6:.0f} MB (read + "
                                           "written) in one call, median of graph replays"},
        "cpu_baseline": None,
    }
    if traffic is not None:
        result["roofline"]["traffic_detail"] = {k: traffic[k] for k in traffic
                                                if k != "kernel_source_sha256"}
    log(f"step {ms_per_step:.3f} ms, decode {decode_ms * 1e3:.1f} us "
        f"({achieved:.0f} GB/s), append {append_ms * 1e3:.1f} us")
    if not args.no_cpu_baseline:
        log("timing the oracle on full layers (CPU, about 10 s)...")
        gpu0 = outs[0].float().cpu().numpy().astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(w, gpu0)
        log(f"oracle: {result['cpu_baseline']['seconds']} s, "
            f"max abs err vs GPU {result['cpu_baseline']['gpu_vs_oracle_max_abs_err']:.3e}")
    if args.calibrate_copy:
        # one more copy call of known size, on its own, for counter scaling
        torch.cuda.synchronize()
        big_copy()
        torch.cuda.synchronize()
        result["calibration_copy"] = {"pairs": half, "bytes_read": cbytes,
                                      "bytes_written": cbytes}
        log(f"calibration copy: {half} blocks, {cbytes / 1e6:.1f} MB read and written")
    del pools, pool0, outs, ws
    if not args.headline_only:
        torch.cuda.empty_cache()
        log("rows:")
        result["rows"] = Rows(pa, torch, args.repeats, not args.no_cpu_baseline,
                              measured_peak=copy_peak).run(make_workload,
                                                           args.sections.split(","))
        torch.cuda.empty_cache()
        if not args.no_engine:
            log("engine loop:")
            result["engine"] = engine_rows(pa, torch, not args.no_cpu_baseline)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
