"""The allocation-free decode entry point, through the C ABI, against pa_decode.

pa_decode_noalloc keeps its split-K partials and queue counters in the
library's own device array instead of a caller's workspace; its outputs must
be the bits pa_decode writes for the same inputs. Two calls in a row (the
second on a smaller batch, so the array holds the first call's partials when
it starts), at both dtypes, each batch with sequences of several partitions.
"""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_282_amd as pa

from tests.gpu_helpers import DeviceStep, bits
from workloads import build_decode_workload

pytestmark = pytest.mark.gpu


def _noalloc_raw(st, out):
    """pa_decode_noalloc called through ctypes with raw device pointers."""
    w = st.w
    lib = pa.load()
    status = lib.pa_decode_noalloc(
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.q.data_ptr()),
        ctypes.c_void_p(st.pool.data_ptr()), ctypes.c_void_p(st.tables.data_ptr()),
        ctypes.c_void_p(st.lens.data_ptr()), w.num_seqs, st.tables.shape[1],
        w.max_context_len, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
        w.num_blocks, ctypes.c_float(w.scale), 1 if w.dtype == "bf16" else 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert status == 0, pa.pa_status_string(status)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_pa_decode_on_two_calls(dtype):
    rng = np.random.default_rng(31)
    big = build_decode_workload("na_big", 3101, rng.integers(1, 5000, 96), 32, 4, 128, 16, dtype)
    small = build_decode_workload("na_small", 3102, rng.integers(1, 2500, 17), 8, 2, 64, 32,
                                  dtype)
    for w in (big, small):
        print(f"[case] noalloc {dtype} B={w.num_seqs} Hq={w.num_q_heads} d={w.head_dim} "
              f"bs={w.block_size} max_ctx={w.max_context_len}", flush=True)
        st = DeviceStep(w)
        st.run()  # copy -> append -> pa_decode into st.out
        want = bits(st.out).copy()
        got = torch.full_like(st.out, float("nan"))
        _noalloc_raw(st, got)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), want)
        # the binding's wrapper reaches the same entry point
        got2 = torch.full_like(st.out, float("nan"))
        pa.pa_decode_noalloc(got2, st.q, st.pool, st.tables, st.lens, w.max_context_len,
                             w.num_kv_heads, w.block_size, w.scale)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got2), want)
