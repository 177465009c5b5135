"""Python binding of libpa's host runtime (include/pa_sched.h).

Argument marshalling only: the block manager, the scheduler and the engine
loop run in libpa's C++ code; the engine's kernels are libpa's HIP kernels.
``Scheduler.step()`` returns the iteration's plan as a dict of Python ints and
lists, decoded from the packet layout documented in include/pa_sched.h.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import PAError, _dev, _dtype_code, _stream, load

POLICIES = {"paged": 0, "reserve": 1, "static": 2}
SCHED_FINISHED = 64

_p = ctypes.c_void_p
_i = ctypes.c_int32
_i64 = ctypes.c_int64


class _Config(ctypes.Structure):
    _fields_ = [("num_blocks", _i), ("block_size", _i), ("max_seqs", _i), ("max_tokens", _i),
                ("max_chunk", _i), ("max_len", _i), ("policy", _i), ("num_host_blocks", _i),
                ("prefix_caching", _i)]


class EngineStats(ctypes.Structure):
    _fields_ = [("iterations", _i64), ("generated", _i64), ("prefill_tokens", _i64),
                ("decode_tokens", _i64), ("decode_context_tokens", _i64), ("copies", _i64),
                ("evictions", _i64), ("swapped_blocks", _i64),
                ("host_us", ctypes.c_double), ("wait_us", ctypes.c_double)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


def _lib():
    lib = load()
    if not getattr(lib, "_sched_ready", False):
        lib.pa_sched_create.argtypes = [ctypes.POINTER(_Config), _p, _i, _p, _p, _p, _p, _p, _p,
                                        ctypes.POINTER(_p)]
        lib.pa_sched_create.restype = ctypes.c_int
        lib.pa_sched_destroy.argtypes = [_p]
        lib.pa_sched_destroy.restype = None
        lib.pa_sched_plan_capacity.argtypes = [_p]
        lib.pa_sched_plan_capacity.restype = _i64
        lib.pa_sched_num_free.argtypes = [_p]
        lib.pa_sched_num_free.restype = _i
        lib.pa_sched_step.argtypes = [_p, _p, _i64, ctypes.POINTER(_i64)]
        lib.pa_sched_step.restype = ctypes.c_int
        lib.pa_engine_create.argtypes = [_p, _p, _i, _i, _i, _i, ctypes.c_float, _p, _p, _p, _p,
                                         _p, _p, _p, ctypes.c_size_t, _p, ctypes.POINTER(_p)]
        lib.pa_engine_create.restype = ctypes.c_int
        lib.pa_engine_destroy.argtypes = [_p]
        lib.pa_engine_destroy.restype = None
        lib.pa_engine_step.argtypes = [_p, _p, _i64, ctypes.POINTER(_i64)]
        lib.pa_engine_step.restype = ctypes.c_int
        lib.pa_engine_run.argtypes = [_p, ctypes.POINTER(EngineStats)]
        lib.pa_engine_run.restype = ctypes.c_int
        lib._sched_ready = True
    return lib


def _arr(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def parse_plan(buf: np.ndarray) -> dict:
    """Decode one plan packet (int32 words) into lists."""
    h = [int(v) for v in buf[:16]]
    it, gen, nc, ns, npre, nch, nd, na, npr, nf, mb, longest, nso, nsi = h[:14]
    w = 16

    def take(n):
        nonlocal w
        out = buf[w:w + n]
        w += n
        return [int(v) for v in out]

    copies = take(2 * nc)
    slots = take(ns)
    creq, cqsl, cctx = take(nch), take(nch + 1), take(nch)
    ctab = take(nch * mb)
    dreq, dsmp, dctx = take(nd), take(nd), take(nd)
    dtab = take(nd * mb)
    return {
        "iteration": it, "generated": gen, "max_blocks": mb, "longest_chunk": longest,
        "prefill_tokens": npre,
        "copies": [(copies[2 * i], copies[2 * i + 1]) for i in range(nc)],
        "slots": slots,
        "chunks": [(creq[c], cqsl[c], cqsl[c + 1] - cqsl[c], cctx[c], ctab[c * mb:(c + 1) * mb])
                   for c in range(nch)],
        "decodes": [(dreq[i], dsmp[i], dctx[i], dtab[i * mb:(i + 1) * mb]) for i in range(nd)],
        "admitted": take(na), "preempted": take(npr), "finished": take(nf),
        "swap_out": [tuple(x) for x in np.asarray(take(2 * nso)).reshape(-1, 2).tolist()],
        "swap_in": [tuple(x) for x in np.asarray(take(2 * nsi)).reshape(-1, 2).tolist()],
    }


class Scheduler:
    """The C++ scheduler. ``requests``: (prompt_len, [output_len per sample], arrival)
    or (prompt_len, [output_len per sample], arrival, prefix_id, prefix_len)."""

    def __init__(self, num_blocks, block_size, max_seqs, max_tokens, max_chunk, max_len,
                 policy, free_order, requests, num_host_blocks=0, prefix_caching=False):
        self._lib = _lib()
        cfg = _Config(num_blocks, block_size, max_seqs, max_tokens, max_chunk, max_len,
                      POLICIES[policy], num_host_blocks, int(bool(prefix_caching)))
        prompts = _arr([r[0] for r in requests])
        arrival = _arr([r[2] for r in requests])
        offs = _arr(np.concatenate([[0], np.cumsum([len(r[1]) for r in requests])]))
        outs = _arr([o for r in requests for o in r[1]] or [0])
        pids = _arr([r[3] if len(r) > 3 else -1 for r in requests] or [0])
        plens = _arr([r[4] if len(r) > 4 else 0 for r in requests] or [0])
        order = _arr(free_order)
        if order.shape[0] != num_blocks:
            raise ValueError("free_order must list num_blocks ids")
        handle = _p()
        st = self._lib.pa_sched_create(ctypes.byref(cfg), order.ctypes.data, len(requests),
                                       prompts.ctypes.data, arrival.ctypes.data,
                                       offs.ctypes.data, outs.ctypes.data, pids.ctypes.data,
                                       plens.ctypes.data, ctypes.byref(handle))
        if st != 0:
            raise PAError("pa_sched_create", st)
        self.handle = handle
        self.capacity = int(self._lib.pa_sched_plan_capacity(handle))
        self._buf = np.zeros(self.capacity, np.int32)

    def num_free(self) -> int:
        return int(self._lib.pa_sched_num_free(self.handle))

    def step(self):
        used = _i64(0)
        st = self._lib.pa_sched_step(self.handle, self._buf.ctypes.data, self.capacity,
                                     ctypes.byref(used))
        if st == SCHED_FINISHED:
            return None
        if st != 0:
            raise PAError("pa_sched_step", st)
        return parse_plan(self._buf[:used.value])

    def run(self):
        plans = []
        while (p := self.step()) is not None:
            plans.append(p)
        return plans

    def close(self):
        if getattr(self, "handle", None):
            self._lib.pa_sched_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()


class Engine:
    """The C++ engine loop over a Scheduler, enqueuing libpa's kernels on one stream."""

    def __init__(self, sched: Scheduler, kv_pool, num_kv_heads, q_prefill, q_decode, k_rows,
                 v_rows, out_prefill, out_decode, workspace, scale, stream=None):
        self._lib = _lib()
        self.sched = sched          # the engine borrows it
        self._keep = (kv_pool, q_prefill, q_decode, k_rows, v_rows, out_prefill, out_decode,
                      workspace)
        hq, d = q_decode.shape[1], q_decode.shape[2]
        handle = _p()
        st = self._lib.pa_engine_create(
            sched.handle, _dev(kv_pool, "kv_pool"), num_kv_heads, hq, d,
            _dtype_code(kv_pool, q_prefill, q_decode, k_rows, v_rows, out_prefill, out_decode),
            float(scale), _dev(q_prefill, "q_prefill"), _dev(q_decode, "q_decode"),
            _dev(k_rows, "k_rows"), _dev(v_rows, "v_rows"), _dev(out_prefill, "out_prefill"),
            _dev(out_decode, "out_decode"), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream), ctypes.byref(handle))
        if st != 0:
            raise PAError("pa_engine_create", st)
        self.handle = handle
        self._buf = np.zeros(sched.capacity, np.int32)

    def step(self):
        used = _i64(0)
        st = self._lib.pa_engine_step(self.handle, self._buf.ctypes.data, self.sched.capacity,
                                      ctypes.byref(used))
        if st == SCHED_FINISHED:
            return None
        if st != 0:
            raise PAError("pa_engine_step", st)
        return parse_plan(self._buf[:used.value])

    def run(self) -> dict:
        stats = EngineStats()
        st = self._lib.pa_engine_run(self.handle, ctypes.byref(stats))
        if st != 0:
            raise PAError("pa_engine_run", st)
        return stats.as_dict()

    def close(self):
        if getattr(self, "handle", None):
            self._lib.pa_engine_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()

