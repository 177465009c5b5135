"""Seeded synthetic request streams for the scheduler and the engine loop.

Input construction only: prompt lengths, per-sample output lengths and arrival
iterations. The stand-in for the pages' serving workloads is a stream whose
output lengths spread widely, capped at 1536 tokens (the benchmark described in
the worksonmygpu.com continuous-batching post, section "What this is worth,
measured"), some of whose requests ask for parallel samples of one prompt
("Module 4 · Batching, Scheduling, and Paging", section "Block sharing").
"""
from __future__ import annotations

import numpy as np


def make_request_stream(seed: int, n: int, prompt=(1, 60), output=(1, 80),
                        multi_frac: float = 0.0, samples: int = 1, arrival_every: int = 0,
                        output_lognormal=None, prefix_groups: int = 0, prefix_tokens: int = 0):
    """``n`` requests as (prompt_len, [output_len per sample], arrival_iteration).

    prompt: inclusive uniform integer range. output: inclusive uniform range,
    or, when ``output_lognormal=(median, sigma, max)`` is given, round(lognormal)
    clipped to [1, max]. A fraction ``multi_frac`` of the requests asks for
    ``samples`` samples, each with its own output length. Request i arrives at
    iteration ``i // arrival_every`` (all at 0 when arrival_every is 0).

    With ``prefix_groups`` > 0, request i also names prefix i % prefix_groups:
    its prompt is that prefix's ``prefix_tokens`` tokens followed by its own
    ``prompt``-range suffix, and the tuple grows to (prompt_len, outputs,
    arrival, prefix_id, prefix_len).
    """
    rng = np.random.default_rng(np.random.SeedSequence([seed, 0x5EED]))
    prompts = rng.integers(prompt[0], prompt[1] + 1, n)
    multi = rng.random(n) < multi_frac
    reqs = []
    for i in range(n):
        k = samples if multi[i] else 1
        if output_lognormal is None:
            outs = rng.integers(output[0], output[1] + 1, k)
        else:
            med, sig, top = output_lognormal
            outs = np.clip(np.rint(np.exp(np.log(med) + sig * rng.standard_normal(k))), 1, top)
        arr = i // arrival_every if arrival_every else 0
        if prefix_groups > 0:
            reqs.append((int(prefix_tokens + prompts[i]), [int(o) for o in outs], int(arr),
                         i % prefix_groups, int(prefix_tokens)))
        else:
            reqs.append((int(prompts[i]), [int(o) for o in outs], int(arr)))
    return reqs
