"""The online softmax's rescale paths, on inputs built to reach them.

The bfloat16 kernels keep a reference maximum m per row and rescale their
running state only when a score passes m by more than 8 (base 2); the prefill
takes a row's maximum only when some lane's weight sum reaches 2^8. Random
inputs rarely leave the first step's reference, so these inputs steer the
scores (base-2 units, x = q.k * scale * log2 e) along one key dimension:

  ramp     x rises by 0.5 a token: m is passed by more than 8 every few
           steps, so rows rescale over and over.
  plateau  x = 0 for the first 32 tokens, then 4: weights of 16 in whole
           32-token steps, lane sums of 256 -- the prefill's slow path with
           no rescale.
  jump     x = 0 except one token at +30 in mid-context: a single rescale by
           2^-30, then weights of 2^-30 for everything after it.
  fall     x falls from 20 by 0.02 a token: no rescale after the first step.

Every pattern runs at a short and a long length (the long one spans two
decode partitions), through the decode, the prefill and the single-launch
mixed batch, at block sizes 16 and 32 (head dim 128) and at head dim 64.
Outputs are checked against the fp64 oracle under the bfloat16 rounding bound
of test_gpu_discriminating.py, and the mixed launch must equal the separate
calls bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_282_amd as pa
from tests.gpu_helpers import bits, i32, values
from tests.pool_writer import contiguous_pool
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu

HKV, HQ = 2, 8
BETA = 16.0  # query component along the steering dimension (bf16-exact)
LENGTHS = (300, 1100)
PATTERNS = ("ramp", "plateau", "jump", "fall")


def _say(msg):
    print(msg, flush=True)


def _x(pattern, n):
    """Target base-2 scores of tokens 0 .. n-1."""
    t = np.arange(n, dtype=np.float64)
    if pattern == "ramp":
        return 0.5 * t
    if pattern == "plateau":
        return np.where(t < 32, 0.0, 4.0)
    if pattern == "jump":
        x = np.zeros(n)
        x[n // 2] = 30.0
        return x
    return 20.0 - 0.02 * t


def _bf16_values(x):
    return (f32_to_bf16_bits(np.asarray(x, np.float32)).astype(np.uint32) << 16).view(np.float32)


def _inputs(seed, D):
    rng = np.random.default_rng(seed)
    scale = 1.0 / np.sqrt(D)
    per_unit = BETA * float(np.float32(scale)) * np.log2(np.e)  # x per unit of the key component
    K, V, lens = [], [], []
    for length in LENGTHS:
        for pattern in PATTERNS:
            k = rng.normal(0.0, 0.05, (length, HKV, D))
            k[:, :, 0] = _x(pattern, length)[:, None] / per_unit
            K.append(_bf16_values(k).astype(np.float64))
            V.append(_bf16_values(rng.normal(0.0, 1.0, (length, HKV, D))).astype(np.float64))
            lens.append(length)
    return K, V, np.array(lens, np.int32), rng


def _queries(rng, rows, D):
    q = rng.normal(0.0, 0.05, (rows, HQ, D))
    q[:, :, 0] = BETA
    return f32_to_bf16_bits(q.astype(np.float32))


def _ulp_bf16(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _check_bound(got, o, ma, md, label):
    err = np.abs(got - o)
    bound = 2.0 ** -8 * np.abs(o) + (2.0 ** -8 + 2.0 ** -10) * ma + \
        (2.0 ** -7 + 2.0 ** -10) * md + 1e-6
    _say(f"  {label}: max abs err {err.max():.3e}, max {float((err / _ulp_bf16(o)).max()):.2f} "
         f"output ulps, worst err / bound {float((err / bound).max()):.3f}")
    assert np.isfinite(got).all()
    assert (err <= bound).all(), f"{int((err > bound).sum())} elements exceed the bound"


@pytest.mark.parametrize("bs,D", [(16, 128), (32, 128), (16, 64)])
def test_rescale_patterns_within_the_rounding_bound(bs, D):
    scale = 1.0 / np.sqrt(D)
    K, V, lens, rng = _inputs(900 + bs + D, D)
    pool_f, tables = contiguous_pool(K, V, bs, np.float32)
    pool = f32_to_bf16_bits(pool_f.astype(np.float32))  # the pad block's NaN stays NaN
    B = len(lens)
    max_len = int(lens.max())
    qd = _queries(rng, B, D)
    Lc = np.minimum(lens, 256)
    qsl = np.concatenate([[0], np.cumsum(Lc)]).astype(np.int32)
    qp = _queries(rng, int(qsl[-1]), D)
    _say(f"[case] rescale patterns bs={bs}: B={B} Hq={HQ} Hkv={HKV} d={D} "
         f"lens={sorted(set(lens.tolist()))} prefill rows={int(qsl[-1])}")

    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    pool_d, qd_d, qp_d = dev(pool), dev(qd), dev(qp)
    tab_d, len_d, qsl_d = i32(tables), i32(lens), i32(qsl)
    ws = pa.new_decode_workspace(B, HQ, D, max_len)
    out = torch.empty_like(qd_d)
    pout = torch.empty_like(qp_d)
    pa.pa_decode(out, qd_d, pool_d, tab_d, len_d, max_len, HKV, bs, scale, ws)
    pa.pa_prefill_chunk(pout, qp_d, pool_d, tab_d, len_d, qsl_d, int(Lc.max()), HKV, bs, scale)
    out2, pout2 = torch.empty_like(out), torch.empty_like(pout)
    pa.pa_mixed_attention(out2, qd_d, tab_d, len_d, max_len, pout2, qp_d, tab_d, len_d, qsl_d,
                          int(Lc.max()), pool_d, HKV, bs, scale, ws)
    torch.cuda.synchronize()

    o, ma, md = oracle.decode_moments(qd, pool, tables, lens, HKV, bs, scale, "bf16")
    _check_bound(values(out), o, ma, md, "decode")
    o, ma, md = oracle.prefill_moments(qp, pool, tables, lens, qsl, HKV, bs, scale, "bf16")
    _check_bound(values(pout), o, ma, md, "prefill")
    assert np.array_equal(bits(out2), bits(out)), "mixed launch decode differs from pa_decode"
    assert np.array_equal(bits(pout2), bits(pout)), "mixed launch prefill differs from pa_prefill_chunk"
