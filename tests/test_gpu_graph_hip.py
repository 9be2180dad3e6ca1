"""The decode step captured into a HIP graph through the HIP runtime itself,
from plain C (tests/c_client/pakv_graph.c): hipStreamBeginCapture of one
step (per layer pa_kv_append when the workload appends, then
pa_decode_planned on a device plan), kernel nodes only, instantiated once;
each replay copies the step's plan into the device plan buffer outside the
graph, then launches it. For the tiny workload, C2 and the full C4 step
(16 layers x (append + decode), 256 sequences): every replay, with eager
work and synchronisations between replays, gives the eager step's outputs
and pool bit for bit, and matches the FP64 oracle within the parity bar
(every output at tiny and C2; all 256 sequences of layers 0 and 15 at C4).
The eager step and the replay are both timed from C with HIP events and
logged ("[graph] ..." lines)."""

import ctypes
import os

import numpy as np
import pytest

from gpu_helpers import Uploaded, check_parity, device, full_oracle, log
from oracle_units import oracle_units
from paged_kv_decode_02_amd import binding as B
from paged_kv_decode_02_amd import workloads as W

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "libpakv_graph.so")
MAXL = 64
c = ctypes


class PgStep(c.Structure):
    _fields_ = [("pool", c.c_void_p), ("layers", c.c_int32), ("num_seqs", c.c_int32),
                ("num_q_heads", c.c_int32), ("max_pages_per_seq", c.c_int32), ("scale", c.c_float),
                ("q", c.c_void_p * MAXL), ("k_new", c.c_void_p * MAXL), ("v_new", c.c_void_p * MAXL),
                ("block_tables", c.c_void_p * MAXL), ("out", c.c_void_p * MAXL),
                ("context_lens", c.c_void_p), ("positions", c.c_void_p), ("workspace", c.c_void_p),
                ("workspace_bytes", c.c_size_t), ("plan_dev", c.c_void_p), ("plan_words", c.c_int32)]


def _lib():
    assert os.path.exists(LIB), f"{LIB} is not built (run __graft_entry__.build())"
    B.lib()                                   # libpakv.so first, from the package directory
    g = c.CDLL(LIB)
    g.pg_eager.argtypes = [c.POINTER(PgStep), c.c_void_p, c.c_void_p, c.c_int, c.POINTER(c.c_float),
                           c.POINTER(c.c_double)]
    g.pg_capture.argtypes = [c.POINTER(PgStep), c.c_void_p, c.POINTER(c.c_void_p), c.POINTER(c.c_int)]
    g.pg_replay.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p, c.c_int32, c.c_void_p, c.c_int,
                            c.POINTER(c.c_float), c.POINTER(c.c_double)]
    g.pg_destroy.argtypes = [c.c_void_p]
    for f in (g.pg_eager, g.pg_capture, g.pg_replay):
        f.restype = c.c_int
    g.pg_destroy.restype = None
    return g


def _step(up, w, plan_dev, words):
    s = PgStep()
    s.pool = up.pool.handle.value if hasattr(up.pool.handle, "value") else up.pool.handle
    s.layers, s.num_seqs, s.num_q_heads, s.max_pages_per_seq = w.num_layers, w.num_seqs, w.num_q_heads, w.stride
    s.scale = float(w.scale)
    for l in range(w.num_layers):
        s.q[l] = up.q[l].data_ptr()
        s.block_tables[l] = up.bt[l].data_ptr()
        s.out[l] = up.out[l].data_ptr()
        if w.append:
            s.k_new[l] = up.k_new[l].data_ptr()
            s.v_new[l] = up.v_new[l].data_ptr()
    s.context_lens = up.ctx.data_ptr()
    s.positions = up.pos.data_ptr() if w.append else None
    s.workspace = up.workspace.data_ptr()
    s.workspace_bytes = up.workspace.numel()
    s.plan_dev = plan_dev.data_ptr()
    s.plan_words = words
    return s


CASES = [("tiny", 200), ("c2", 200), ("c4", 20)]


@pytest.mark.parametrize("name,timed", CASES, ids=[c[0] for c in CASES])
def test_hip_graph_step(name, timed):
    import torch
    dev = device()
    g = _lib()
    w = W.make_workload(name)
    log(f"hip graph: {name} L={w.num_layers} B={w.num_seqs} append={w.append} "
        f"entry=pa_kv_append+pa_decode_planned captured with hipStreamBeginCapture")
    up = Uploaded(w, dev)
    plan_host = B.decode_plan(up.pool, w.ctx_lens, w.num_q_heads, w.stride)
    plan_dev = torch.from_numpy(plan_host).to(dev)
    step = _step(up, w, plan_dev, plan_host.size)
    stream = torch.cuda.Stream(device=dev)
    h = stream.cuda_stream
    ms, host = c.c_float(0.0), c.c_double(0.0)
    words = plan_host.size
    pp = plan_host.ctypes.data
    assert g.pg_eager(c.byref(step), pp, h, 1, c.byref(ms), c.byref(host)) == 0
    torch.cuda.synchronize()
    eager = up.out.clone()
    k_eager, v_eager = up.k_pool.clone(), up.v_pool.clone()
    graph, nodes = c.c_void_p(), c.c_int(0)
    assert g.pg_capture(c.byref(step), h, c.byref(graph), c.byref(nodes)) == 0, "capture (kernel nodes only)"
    launches = w.num_layers * (2 if w.append else 1)
    assert nodes.value >= launches, f"{nodes.value} graph nodes for {launches} launches"
    if name in ("tiny", "c2"):
        ref = full_oracle(w, up)
        refs = {l: ref[l] for l in range(w.num_layers)}
    else:
        units = oracle_units(name, [(l, b) for l in (0, 15) for b in range(w.num_seqs)])
        refs = {l: np.stack([units[(l, b)] for b in range(w.num_seqs)]) for l in (0, 15)}
    scratch = torch.randn(1 << 20, device=dev)
    try:
        for rep in range(3):
            up.out.fill_(float("nan"))
            scratch.mul_(1.0001).add_(0.5)             # eager work between replays
            torch.cuda.synchronize()
            assert g.pg_replay(graph, pp, plan_dev.data_ptr(), words, h, 1, c.byref(ms), c.byref(host)) == 0
            torch.cuda.synchronize()
            assert bool((up.out.view(torch.int32) == eager.view(torch.int32)).all()), f"replay {rep} != eager"
            assert bool((up.k_pool == k_eager).all()) and bool((up.v_pool == v_eager).all()), \
                f"replay {rep}: pool differs from the eager step"
            out = up.out.cpu().numpy()
            for l, r in refs.items():
                a, rel = check_parity(out[l], r, f"{name} replay {rep} layer {l} vs oracle")
        log(f"{name}: 3 replays bitwise equal to eager and within the bar of the oracle "
            f"(layers {sorted(refs)}; last max abs {a:.2e} max rel {rel:.2e}); {nodes.value} kernel nodes")
        # timing: the same steps (each with its plan copy) eager, queued from
        # C, and replayed; device time from HIP events, host time to queue
        for _ in range(3):
            assert g.pg_eager(c.byref(step), pp, h, timed, c.byref(ms), c.byref(host)) == 0
        eager_us, eager_host = ms.value * 1e3 / timed, host.value / timed
        for _ in range(3):
            assert g.pg_replay(graph, pp, plan_dev.data_ptr(), words, h, timed, c.byref(ms), c.byref(host)) == 0
        graph_us, graph_host = ms.value * 1e3 / timed, host.value / timed
        log(f"[graph] {name}: eager {eager_us:.1f} us/step (host {eager_host:.1f}), graph replay "
            f"{graph_us:.1f} us/step (host {graph_host:.1f}); {timed} steps each, plan copied per step, "
            f"{launches} launches per step")
    finally:
        torch.cuda.synchronize()
        g.pg_destroy(graph)
