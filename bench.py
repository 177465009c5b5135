#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Workload (default): the GQA long-tail decode batch -- 256 sequences, 64 query
heads / 8 KV heads, head_dim 128, block_size 16, bfloat16 with float32
accumulation, context lengths lognormal (median 800, ln-sigma 1) clipped to
[16, 8192], blocks placed by a seeded random permutation.

One step = one decode iteration over L layers (default 4, each its own pool so
repeated calls do not hit in the 256 MB last-level cache): per layer, append
every sequence's new token (pa_append_kv) and run paged decode attention
(pa_decode). Inputs are resident in HBM before timing starts.

Reported (one JSON line on stdout):
  value      effective KV bandwidth = algorithmic K+V bytes attended / time, GB/s
             (each attended token's K and V read once per (sequence, kv head))
  roofline   the decode kernel alone: algorithmic bytes per launch / its mean
             duration (HIP events on the launch stream), against 8 TB/s
  cpu_baseline  the fp64 NumPy oracle on one full layer on the host, 1 thread
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
METRIC = "paged decode attention: effective KV HBM GB/s (% of peak) and seq-layers/s"
WORKLOAD_DESC = {
    "gqa": "GQA long-tail decode: 256 seqs, 64 q / 8 kv heads, head_dim 128, block_size 16, "
           "bf16, context lengths lognormal(median 800, sigma 1) clipped [16, 8192]",
    "mha": "MHA decode (7B-like layer): 64 seqs, 32/32 heads, head_dim 128, block_size 16, "
           "bf16, context lengths uniform [128, 2048]",
}


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--workload", default="gqa", choices=sorted(WORKLOAD_DESC))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def to_dev(arr, dtype, torch):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, np.float32)).cuda()


def cpu_baseline(w, gpu_out0: np.ndarray) -> dict:
    """Time the fp64 oracle on one full layer (append + decode of every sequence)."""
    import oracle
    from threadpoolctl import threadpool_limits

    with threadpool_limits(1):
        t0 = time.perf_counter()
        pool_after = oracle.append(w.pool, w.k_new, w.v_new, w.slot_mapping, w.num_kv_heads,
                                   w.block_size, w.head_dim)
        ref = oracle.decode(w.q, pool_after, w.block_tables, w.context_lens, w.num_kv_heads,
                            w.block_size, w.scale, w.dtype)
        dt = time.perf_counter() - t0
    kv_bytes = float(w.context_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_dim \
        * w.elem_bytes
    err = float(np.abs(gpu_out0 - ref).max())
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"one full layer: append of {w.num_seqs} tokens + decode of all "
                      f"{w.num_seqs} sequences, fp64 NumPy, 1 BLAS thread",
            "seconds": round(dt, 3), "seq_layers_per_s": round(w.num_seqs / dt, 2),
            "gpu_vs_oracle_max_abs_err": err}


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
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
    slots, tables, lens = i32(w.slot_mapping), i32(w.block_tables), i32(w.context_lens)
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms_per_step = ev0.elapsed_time(ev1) / args.steps

    # per-kernel durations (events on the launch stream around each call)
    n = args.steps * L
    ea = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    eb = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ec = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    i = 0
    for _ in range(args.steps):
        for l in range(L):
            ea[i].record()
            append(l)
            eb[i].record()
            decode(l)
            ec[i].record()
            i += 1
    torch.cuda.synchronize()
    append_ms = float(np.mean([ea[k].elapsed_time(eb[k]) for k in range(n)]))
    dec_times = np.array([eb[k].elapsed_time(ec[k]) for k in range(n)])
    decode_ms = float(dec_times.mean())

    kv_bytes_layer = float(w.context_lens.astype(np.int64).sum()) * 2 * hkv * w.head_dim \
        * w.elem_bytes
    value = kv_bytes_layer * L / (ms_per_step * 1e-3) / 1e9
    achieved = kv_bytes_layer / (decode_ms * 1e-3) / 1e9
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
        "kernels_ms": {"pa_decode": round(decode_ms, 4),
                       "pa_decode_p10": round(float(np.percentile(dec_times, 10)), 4),
                       "pa_decode_p90": round(float(np.percentile(dec_times, 90)), 4),
                       "pa_append_kv": round(append_ms, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "decode_bf16_kernel<128,16> (pa_decode)",
                     "algorithmic_bytes_per_launch": int(kv_bytes_layer)},
        "cpu_baseline": None,
    }
    log(f"step {ms_per_step:.3f} ms, decode {decode_ms * 1e3:.1f} us "
        f"({achieved:.0f} GB/s), append {append_ms * 1e3:.1f} us")
    if not args.no_cpu_baseline:
        log("timing the oracle on one layer (CPU)...")
        gpu0 = outs[0].float().cpu().numpy().astype(np.float64)
        result["cpu_baseline"] = cpu_baseline(w, gpu0)
        log(f"oracle: {result['cpu_baseline']['seconds']} s, "
            f"max abs err vs GPU {result['cpu_baseline']['gpu_vs_oracle_max_abs_err']:.3e}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
