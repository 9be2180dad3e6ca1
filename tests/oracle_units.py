"""FP64 oracle outputs for many (layer, sequence) units of a named workload,
computed on the host in worker processes.

Each worker rebuilds the seeded workload and regenerates, from the generator's
host path, only the pages of the units it is given; the GPU is not touched and
nothing comes from the HIP library. Used by the GPU parity tests to compare
full-size launches element by element within a few seconds of wall time.

Workers are started with the "spawn" method, so they are fresh interpreters
that import numpy, the generator and the oracle only (no torch, no HIP).
"""

from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

import oracle
from paged_kv_decode_02_amd import workloads as W

_W = None
_Q = None
_KN = None
_VN = None


def _init(name: str):
    global _W, _Q, _KN, _VN
    try:   # one BLAS thread per worker: the workers already use every core
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    _W = W.make_workload(name)
    _Q = _W.q_bits()
    if _W.append:
        _KN = _W.new_kv_bits("k")
        _VN = _W.new_kv_bits("v")


def unit_output(w, layer: int, b: int, q_host, k_new_host=None, v_new_host=None) -> np.ndarray:
    """Oracle output ``[Hq][d]`` of sequence b in one layer, from the pages that
    sequence references (after the oracle's own append when the workload
    appends)."""
    n = int(w.ctx_lens[b])
    if n == 0:
        return np.zeros((w.num_q_heads, w.head_dim))
    pages = w.sequence_pages(layer, b)
    kp = w.pool_pages_bits("k", pages)
    vp = w.pool_pages_bits("v", pages)
    bt = np.arange(pages.size, dtype=np.int32)[None, :]
    if w.append:
        kp, vp = oracle.kv_append(kp, vp, k_new_host[layer][b:b + 1], v_new_host[layer][b:b + 1],
                                  bt, np.array([n - 1], np.int32))
    return oracle.decode_attention(q_host[layer][b:b + 1], kp, vp, bt, np.array([n], np.int32),
                                   w.scale)[0]


def _work(unit):
    layer, b = unit
    return layer, b, unit_output(_W, layer, b, _Q, _KN, _VN)


def host_workers() -> int:
    """Worker processes for the host oracle: the cores this process may run on,
    at most 8 (the GPU machine gives one GPU's job 16 cores)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(8, n))


def oracle_units(name: str, units, workers: int | None = None) -> dict:
    """{(layer, b): FP64 [Hq][d]} for every unit of the named workload."""
    units = [(int(l), int(b)) for l, b in units]
    workers = workers or host_workers()
    # longest sequences first so that the pool ends on short units
    w = W.make_workload(name)
    units.sort(key=lambda u: -int(w.ctx_lens[u[1]]))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_init, initargs=(name,)) as pool:
        res = pool.map(_work, units, chunksize=1)
    return {(l, b): o for l, b, o in res}
