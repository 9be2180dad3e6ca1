"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4]

A step is one pass of the whole path over one batch: for the default workload
(16 layers, 256 sequences, lognormal contexts, 32q/8kv, d=64) that is the
launch plan made on the host from the host's context lengths, then per layer
the paged append of the new token's K/V and paged decode attention, the plan
carried in the decode kernel's arguments (pa_decode_planned_host), launched
from Python through calls prepared once (--graph replays each step's launches
from a HIP graph captured once per input replica instead, with the plan in
device memory). Inputs are resident in HBM before timing. Prints one JSON
line: achieved KV-read GB/s over the timed steps, the roofline of the dominant
kernel (the decode kernel, timed with HIP events on the launch stream in a
separate pass over the same steps), the same figures for the other decode
configurations (tiny, c2, c3, c5) under "configs", and a CPU baseline (the
FP64 oracle on a bounded sample of the same workload, on the host cores).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E peak
MALL_BYTES = 256 << 20   # device last-level (Infinity) cache
PROFILE = os.path.join(ROOT, "profiles", "decode_kernel_c4.md")
PREFILL_PROFILE = os.path.join(ROOT, "profiles", "prefill_kernel_prefill.md")
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense BF16 matrix-core peak
KERNEL_SOURCES = ("paged_kv_decode_02_amd/csrc/pakv_kernels.h", "paged_kv_decode_02_amd/csrc/pakv.hip")
PREFILL_SOURCES = KERNEL_SOURCES + ("paged_kv_decode_02_amd/csrc/pakv_prefill.h",)


def counted_traffic(workload, profile=PROFILE, profiled_workload="c4", sources=KERNEL_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 counter summary, only if
    it was taken on this workload with the kernel sources as they are now
    (sha256 of the sources); None otherwise."""
    import hashlib
    if workload != profiled_workload or not os.path.exists(profile):
        return None
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    for line in open(profile):
        if line.startswith("traffic_json:"):
            t = json.loads(line.split(":", 1)[1])
            if t.get("source_sha256") == h.hexdigest():
                return t
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4",
                    choices=["tiny", "c2", "c3", "c4", "c5", "prefill", "prefill_d128", "prefill_chunked"])
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget of timed oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only --workload (default: also every other decode configuration)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step's launches from a HIP graph captured once per replica "
                         "(default: launch from Python; measured faster on this stack)")
    return ap.parse_args()


class Inputs:
    """One replica of a workload's device inputs, with the step's launches
    prepared once (arguments checked and marshalled) and a host plan buffer."""

    def __init__(self, w, dev, B, stream):
        import torch
        self.k = w.pool_device("k", dev)
        self.v = w.pool_device("v", dev)
        self.pool = B.Pool(self.k, self.v)
        self.bt = torch.from_numpy(np.ascontiguousarray(w.block_tables)).to(dev)
        self.ctx = torch.from_numpy(w.ctx_lens).to(dev)
        self.q = torch.from_numpy(w.q_bits().view(np.int16)).to(dev)
        if w.append:
            self.k_new = torch.from_numpy(w.new_kv_bits("k").view(np.int16)).to(dev)
            self.v_new = torch.from_numpy(w.new_kv_bits("v").view(np.int16)).to(dev)
            self.pos = torch.from_numpy(w.positions).to(dev)
        need = B.decode_workspace_bytes(self.pool, w.num_seqs, w.num_q_heads, w.stride)
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        self.out = torch.empty((w.num_layers, w.num_seqs, w.num_q_heads, w.head_dim),
                               dtype=torch.float32, device=dev)
        # launch plan: made on the host from the host copy of the context
        # lengths once per step (every layer shares it); a small plan travels
        # in each decode launch's arguments, a larger one is copied to the
        # device once per step
        self.ctx_host = np.ascontiguousarray(w.ctx_lens, dtype=np.int32).copy()
        self.plan = B.HostPlan(self.pool, self.ctx_host, w.num_q_heads, w.stride)
        if self.plan.make() > B.INLINE_PLAN_WORDS:
            self.plan = B.DevicePlan(self.pool, self.ctx_host, w.num_q_heads, w.stride, dev)
        self.decode = [B.PreparedDecode(self.pool, self.q[l], self.bt[l], self.ctx, float(w.scale), self.plan,
                                        self.out[l], workspace=self.ws, stream=stream)
                       for l in range(w.num_layers)]
        self.append = ([B.PreparedAppend(self.pool, self.k_new[l], self.v_new[l], self.bt[l], self.pos,
                                         stream=stream) for l in range(w.num_layers)] if w.append else [])
        # --graph: the plan in device memory, copied from pinned host memory
        self.graph = None
        self.graph_words = -1
        self.plan_dev = None


def run_step(w, x, B, stream):
    """One step: the launch plan (host), then per layer the paged append of the
    new token's K/V (pa_kv_append) and paged decode attention with the plan in
    the kernel's arguments (pa_decode_planned_host). Replayed from a HIP graph
    instead when one was captured for this replica."""
    import torch
    if x.graph is not None:
        words = upload_plan(w, x, B, stream)
        if words == x.graph_words:
            with torch.cuda.stream(stream):
                x.graph.replay()
            return
    if isinstance(x.plan, B.DevicePlan):
        x.plan.upload(stream)
    else:
        x.plan.make()
    for layer in range(w.num_layers):
        if w.append:
            x.append[layer]()
        x.decode[layer]()


def upload_plan(w, x, B, stream):
    """--graph: this step's plan made on the host into a pinned buffer and
    copied on the launch stream into the device buffer the captured launches
    read (two pinned buffers, so a plan is never rewritten while its copy may
    still be pending). Returns its length in words."""
    import torch
    hp = x.plan.host if isinstance(x.plan, B.DevicePlan) else x.plan
    words = hp.make()
    k = x.step_no & 1
    x.step_no += 1
    if x.plan_copied[k] is not None:
        x.plan_copied[k].synchronize()
    x.plan_pin[k][:words].copy_(torch.from_numpy(hp.buf[:words]))
    with torch.cuda.stream(stream):
        x.plan_dev[:words].copy_(x.plan_pin[k][:words], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        x.plan_copied[k] = ev
    return words


def capture_step(w, x, B, stream):
    """Capture one step's launches (all layers, the plan in device memory) into
    a HIP graph through torch; a replay serves any plan of the same length."""
    import torch
    hp = x.plan.host if isinstance(x.plan, B.DevicePlan) else x.plan
    x.plan_pin = [torch.empty(hp.cap, dtype=torch.int32, pin_memory=True) for _ in range(2)]
    x.plan_copied = [None, None]
    x.step_no = 0
    x.plan_dev = torch.empty(hp.cap, dtype=torch.int32, device=stream.device)
    words = upload_plan(w, x, B, stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for layer in range(w.num_layers):
            if w.append:
                B.kv_append(x.pool, x.k_new[layer], x.v_new[layer], x.bt[layer], x.pos, stream=stream)
            B.decode_planned(x.pool, x.q[layer], x.bt[layer], x.ctx, float(w.scale), x.plan_dev[:words],
                             out=x.out[layer], workspace=x.ws, stream=stream)
    torch.cuda.synchronize()
    x.graph, x.graph_words = g, words


def step_percentiles(run_one, steps, stream):
    """A pass of its own after the timed region: each of `steps` steps
    bracketed alone by a pair of HIP events on the launch stream. Returns the
    10th, 50th and 90th percentile of the step time in us."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            run_one(i)
            b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return {"p10": round(float(np.percentile(t, 10)), 1), "p50": round(float(np.percentile(t, 50)), 1),
            "p90": round(float(np.percentile(t, 90)), 1),
            "note": "each step timed alone by HIP events in a separate pass"}


def flushed_steps(run_one, steps, stream, dev):
    """For workloads whose K/V fits the device cache: each step timed alone by
    HIP events after writing a 1 GiB scratch buffer on the launch stream, so
    that none of the step's pages is still cached. Returns the median and the
    10th and 90th percentile in us."""
    import torch
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(evs):
            scratch.fill_(i & 0xFF)
            a.record(stream)
            run_one(i)
            b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    del scratch
    return {"p10": round(float(np.percentile(t, 10)), 1), "p50": round(float(np.percentile(t, 50)), 1),
            "p90": round(float(np.percentile(t, 90)), 1)}


def stream_ceiling(B, dev, stream):
    """Achievable HBM read bandwidth: pa_stream_read over a 4 GiB buffer, each
    of 10 runs timed alone; returns (best, median) GB/s. Run-to-run spread is
    large on this device, so the best run is the ceiling."""
    import torch
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(2):
        B.stream_read(buf, sink, stream=stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
    for e0, e1 in evs:
        e0.record(stream)
        B.stream_read(buf, sink, stream=stream)
        e1.record(stream)
    torch.cuda.synchronize()
    rates = sorted(buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9 for e0, e1 in evs)
    del buf
    return rates[-1], rates[len(rates) // 2]


def host_cores() -> int:
    """Cores this process may run on (the box's share of the host)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w, budget_s):
    """The FP64 oracle on (layer, sequence) units of the same workload until about
    budget_s seconds of oracle time have run. Page regeneration is not timed."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    q = w.q_bits()
    kn = w.new_kv_bits("k") if w.append else None
    vn = w.new_kv_bits("v") if w.append else None
    rng = np.random.default_rng(2024)
    units = [(l, b) for l in range(w.num_layers) for b in range(w.num_seqs)]
    order = rng.permutation(len(units))
    t_oracle = 0.0
    nbytes = 0
    done = 0
    for i in order:
        layer, b = units[i]
        n = int(w.ctx_lens[b])
        pages = w.sequence_pages(layer, b)
        kp = w.pool_pages_bits("k", pages)
        vp = w.pool_pages_bits("v", pages)
        bt = np.arange(pages.size, dtype=np.int32)[None, :]
        t0 = time.perf_counter()
        if w.append:
            kp, vp = oracle.kv_append(kp, vp, kn[layer][b:b + 1], vn[layer][b:b + 1], bt,
                                      np.array([n - 1], np.int32))
        oracle.decode_attention(q[layer][b:b + 1], kp, vp, bt, np.array([n], np.int32), w.scale)
        t_oracle += time.perf_counter() - t0
        nbytes += n * w.num_kv_heads * w.head_dim * 4
        done += 1
        if t_oracle >= budget_s:
            break
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    gbps = nbytes / t_oracle / 1e9
    return {"value": round(gbps, 6), "unit": "GB/s", "cores": 1, "host_cores": host_cores(), "kind": "oracle",
            "sample": f"{done} of {len(units)} (layer, sequence) units, random order, "
                      f"{nbytes / 1e6:.1f} MB of KV in {t_oracle:.1f} s of oracle time; "
                      f"BLAS limited to 1 thread",
            "us_per_step_extrapolated": round(t_oracle / nbytes * w.kv_bytes_per_step() * 1e6, 1)}


# ------------------------------------------------------------------ prefill
PREFILL_NAMES = {
    "prefill": "16-layer prefill of 8 prompts x 2048 tokens, 32q/8kv d64, empty caches",
    "prefill_d128": "prefill of 4 prompts x 4096 tokens, 28q/4kv d128, one layer, empty caches",
    "prefill_chunked": "512-token chunks continuing 8 caches of U[0,4096] tokens, 32q/8kv d64, one layer",
}


class PrefillInputs:
    def __init__(self, w, dev, B):
        import torch
        base = w.base
        self.k = base.pool_device("k", dev)
        self.v = base.pool_device("v", dev)
        self.pool = B.Pool(self.k, self.v)
        self.bt = torch.from_numpy(np.ascontiguousarray(base.block_tables)).to(dev)
        self.qs = torch.from_numpy(w.query_start).to(dev)
        self.before = torch.from_numpy(w.ctx_before).to(dev)
        self.q = w.rows_device("q", dev)
        self.k_rows = w.rows_device("k", dev)
        self.v_rows = w.rows_device("v", dev)
        self.out = torch.empty((base.num_layers, w.num_rows, base.num_q_heads, base.head_dim),
                               dtype=torch.float32, device=dev)
        self.max_chunk = int(w.chunks.max())
        # launch plan: made on the host from the host copies of the cache and
        # chunk lengths once per step (every layer shares it), as for decode
        self.before_host = w.ctx_before.copy()
        self.chunks_host = w.chunks.copy()
        self.stride = int(base.block_tables.shape[2])
        cap = B.prefill_plan_capacity(self.pool, len(w.chunks), base.num_q_heads, self.max_chunk)
        self.plan_pin = [torch.empty(max(cap, 1), dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.plan_copied = [None, None]
        self.plan_dev = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
        self.step_no = 0


def upload_prefill_plan(w, x, B, stream):
    """The prefill launch plan for this step's lengths, made on the host into a
    pinned buffer and copied to the device on the launch stream."""
    import torch
    k = x.step_no & 1
    x.step_no += 1
    if x.plan_copied[k] is not None:
        x.plan_copied[k].synchronize()
    n = B.prefill_plan_into(x.pool, x.before_host, x.chunks_host, w.base.num_q_heads, x.stride,
                            x.max_chunk, x.plan_pin[k])
    plan = x.plan_dev[:n]
    with torch.cuda.stream(stream):
        plan.copy_(x.plan_pin[k][:n], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        x.plan_copied[k] = ev
    return plan


def run_prefill_step(w, x, B, stream):
    """One step: the launch plan, then per layer pa_prefill_planned (the
    chunk's K/V written into the pages, then causal attention for every chunk
    token, row blocks in the plan's order; bit-identical to pa_prefill)."""
    plan = upload_prefill_plan(w, x, B, stream)
    for layer in range(w.base.num_layers):
        B.prefill_planned(x.pool, x.q[layer], x.k_rows[layer], x.v_rows[layer], x.qs, x.bt[layer], x.before,
                          float(w.base.scale), x.max_chunk, plan, out=x.out[layer], stream=stream)


def prefill_cpu_baseline(w, budget_s):
    """The FP64 oracle on random (layer, sequence, chunk row) units of the same
    workload for about budget_s seconds: each row attends over its causal
    prefix, gathered from pages that hold the cache and the written chunk
    (regeneration and the chunk write are not timed)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(1)
    except Exception:  # pragma: no cover
        limiter = None
    base = w.base
    rng = np.random.default_rng(2025)
    qs = w.query_start
    g = base.num_q_heads // base.num_kv_heads
    t_oracle, flops, rows_done = 0.0, 0, 0
    while t_oracle < budget_s:
        layer = int(rng.integers(base.num_layers))
        b = int(rng.integers(len(w.chunks)))
        n_tot = int(w.ctx_before[b]) + int(w.chunks[b])
        pages = base.block_tables[layer, b, :-(-n_tot // 16)]
        kp = base.pool_pages_bits("k", pages)
        vp = base.pool_pages_bits("v", pages)
        rows = np.arange(qs[b], qs[b + 1])
        bt = np.arange(pages.size, dtype=np.int32)[None, :]
        kp, vp = oracle.kv_write(kp, vp, w.rows_bits("k", layer, rows), w.rows_bits("v", layer, rows),
                                 np.array([0, rows.size]), bt, np.array([w.ctx_before[b]]))
        pick = rng.integers(0, rows.size, 16)
        qsel = w.rows_bits("q", layer, rows[pick])
        t0 = time.perf_counter()
        kc, vc = oracle.gather_sequence(kp, vp, bt[0], n_tot)
        for j, i in enumerate(pick):
            p = int(w.ctx_before[b]) + int(i)
            qr = oracle.bf16_bits_to_f64(qsel[j])
            for h in range(base.num_q_heads):
                oracle.attend_one_head(qr[h], kc[:p + 1, h // g], vc[:p + 1, h // g], float(base.scale))
            flops += 4 * base.head_dim * base.num_q_heads * (p + 1)
            rows_done += 1
        t_oracle += time.perf_counter() - t0
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    return {"value": round(flops / t_oracle / 1e12, 9), "unit": "TFLOP/s", "cores": 1, "host_cores": host_cores(),
            "kind": "oracle",
            "sample": f"{rows_done} random chunk rows (all query heads each) of random (layer, sequence) "
                      f"units, {flops / 1e9:.2f} GFLOP in {t_oracle:.1f} s of oracle time (gather "
                      f"included); BLAS limited to 1 thread"}


def prefill_main(args):
    import torch
    from paged_kv_decode_02_amd import binding as B
    from paged_kv_decode_02_amd import workloads as W

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    B.lib()
    w = W.make_prefill_workload(args.workload)
    base = w.base
    stream = torch.cuda.Stream(device=dev)
    t0 = time.time()
    x = PrefillInputs(w, dev, B)
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: {w.num_rows} chunk rows x {base.num_layers} layer(s), pool "
          f"{base.pool_bytes() / 1e9:.2f} GB, inputs made in {time.time() - t0:.1f} s",
          file=sys.stderr, flush=True)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            run_prefill_step(w, x, B, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(args.steps):
            run_prefill_step(w, x, B, stream)
        e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    flops_step = w.flops_per_layer() * base.num_layers
    value = flops_step / (ms_step * 1e-3) / 1e12
    pct = step_percentiles(lambda i: run_prefill_step(w, x, B, stream), args.steps, stream)

    B.profile_start()
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            run_prefill_step(w, x, B, stream)
    torch.cuda.synchronize()
    prof = B.profile_stop()
    pre_ms, pre_n = prof["prefill"]
    wr_ms, wr_n = prof["write"]
    pre_avg = pre_ms / max(pre_n, 1)
    achieved = w.flops_per_layer() / (pre_avg * 1e-3) / 1e12
    print(f"[bench] step {ms_step * 1e3:.1f} us; prefill kernel avg {pre_avg * 1e3:.1f} us x {pre_n}, "
          f"chunk write {wr_ms / max(wr_n, 1) * 1e3:.1f} us x {wr_n}", file=sys.stderr, flush=True)
    ceiling = ceiling_median = None
    if not args.no_ceiling:
        ceiling, ceiling_median = stream_ceiling(B, dev, stream)
    cpu = None if args.no_cpu_baseline else prefill_cpu_baseline(w, args.cpu_seconds)
    traffic = counted_traffic(w.name, PREFILL_PROFILE, "prefill", PREFILL_SOURCES)
    result = {
        "metric": "paged prefill attention: achieved TFLOP/s (% of BF16 matrix-core peak) + us/step",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "us_per_step": round(ms_step * 1e3, 1),
        "us_per_step_percentiles": pct,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": PREFILL_NAMES[w.name],
            "global_batch": int(len(w.chunks)),
            "layers": base.num_layers,
            "q_heads": base.num_q_heads,
            "kv_heads": base.num_kv_heads,
            "head_dim": base.head_dim,
            "chunk_rows": w.num_rows,
            "cache_before_mean": round(float(w.ctx_before.mean()), 1),
            "flops_per_step": flops_step,
            "entry": "pa_prefill_planned per layer (plan made on the host each step)",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_kernel",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
            "avg_launch_us": round(pre_avg * 1e3, 2),
            "algorithmic_flops_per_launch": w.flops_per_layer(),
            "note": "algorithmic flops: 4 d per (query head, causal pair); the kernel also runs the "
                    "P low half through the matrix cores and whole 32-key pairs past the diagonal",
        },
        "kernels_us_per_step": {"prefill": round(pre_ms / args.steps * 1e3, 1),
                                "chunk_write": round(wr_ms / args.steps * 1e3, 1),
                                "note": "separate profiled pass; each kernel bracketed by HIP events"},
        "stream_read_ceiling_GBps": None if ceiling is None else round(ceiling, 1),
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


DECODE_NAMES = {
    "tiny": "tiny: 1 seq x ctx 128, 32q/8kv d64, 1 layer",
    "c2": "batch 8, ctx U[1,512], 32q/8kv d64, 1 layer",
    "c3": "batch 64, ctx U[256,2048], 32q/8kv d64, 1 layer",
    "c4": "full decode step: 16 layers x (append + decode), batch 256, ctx lognormal median 1024 "
          "clipped [16,8192], 32q/8kv d64",
    "c5": "batch 64, ctx U[4096,16384], 28q/4kv d128, 1 layer",
}


def measure_decode(name, steps, warmup, B, W, dev, stream, graph=False, detail=True):
    """Time one decode workload: K steps back to back between two events
    (the value), each step alone (percentiles), each step after a cache flush
    (workloads that fit the device cache), and a pass with every library
    launch bracketed by events (kernel averages)."""
    import torch
    w = W.make_workload(name)
    # Workloads whose per-step K/V fits the device cache twice over rotate over
    # replicas, so that at least 4x the cache is touched between reuses.
    replicas = 1
    if w.kv_bytes_per_step() < 2 * MALL_BYTES:
        replicas = min(16, max(2, math.ceil(4 * MALL_BYTES / w.kv_bytes_per_step())))
    t0 = time.time()
    xs = [Inputs(w, dev, B, stream) for _ in range(replicas)]
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: pool {w.pool_bytes() / 1e9:.2f} GB x {replicas} replica(s), "
          f"inputs made in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    with torch.cuda.stream(stream):
        for i in range(max(warmup, replicas)):
            run_step(w, xs[i % replicas], B, stream)
    torch.cuda.synchronize()
    if graph:
        for x in xs:
            capture_step(w, x, B, stream)
        with torch.cuda.stream(stream):
            for i in range(replicas):
                run_step(w, xs[i % replicas], B, stream)
        torch.cuda.synchronize()

    # Timed region: K steps between two events on the launch stream.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        t_host0 = time.perf_counter()
        for i in range(steps):
            run_step(w, xs[i % replicas], B, stream)
        t_host1 = time.perf_counter()
        e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    kv_step = w.kv_bytes_per_step()
    value = kv_step / (ms_step * 1e-3) / 1e9
    res = {"workload": DECODE_NAMES[name], "w": w, "replicas": replicas, "ms_per_step": ms_step,
           "value": value, "kv_bytes_per_step": kv_step,
           "host_us_per_step": (t_host1 - t_host0) / steps * 1e6}
    run_one = lambda i: run_step(w, xs[i % replicas], B, stream)
    if detail:
        res["pct"] = step_percentiles(run_one, steps, stream)
    res["flushed"] = None
    if replicas > 1:
        fl = flushed_steps(run_one, steps, stream, dev)
        res["flushed"] = {"us_per_step": fl, "GBps_at_p50": round(kv_step / (fl["p50"] * 1e-6) / 1e9, 1),
                          "note": "each step timed alone after a 1 GiB write that evicts the device cache"}
    # Kernel durations: the same K steps again with every kernel the library
    # queues bracketed by HIP events on the launch stream (the brackets add
    # small gaps between kernels, so the step time above is taken without
    # them). This pass launches eagerly: graph replays bypass the brackets.
    for x in xs:
        x.graph = None
    B.profile_start()
    with torch.cuda.stream(stream):
        for i in range(steps):
            run_step(w, xs[i % replicas], B, stream)
    torch.cuda.synchronize()
    prof = B.profile_stop()
    res["prof"] = prof
    dec_ms, dec_n = prof["decode"]
    res["decode_avg_ms"] = dec_ms / max(dec_n, 1)
    mer_ms, mer_n = prof["merge"]
    app_ms, app_n = prof["append"]
    res["kernels_us_per_step"] = {"decode": round(dec_ms / steps * 1e3, 1), "merge": round(mer_ms / steps * 1e3, 1),
                                  "append": round(app_ms / steps * 1e3, 1)}
    print(f"[bench] {name}: step {ms_step * 1e3:.1f} us (host {res['host_us_per_step']:.1f} us); decode "
          f"kernel avg {res['decode_avg_ms'] * 1e3:.1f} us x {dec_n}, merge "
          f"{mer_ms / max(mer_n, 1) * 1e3:.1f} us x {mer_n}, append {app_ms / max(app_n, 1) * 1e3:.1f} us x "
          f"{app_n}", file=sys.stderr, flush=True)
    del xs
    torch.cuda.empty_cache()
    return res


def config_summary(res):
    w = res["w"]
    dec_us = res["decode_avg_ms"] * 1e3
    out = {
        "workload": res["workload"],
        "us_per_step": round(res["ms_per_step"] * 1e3, 2),
        "kv_GBps": round(res["value"], 1),
        "frac_of_hbm_peak": round(res["value"] / HBM_PEAK_GBPS, 4),
        "decode_kernel_avg_us": round(dec_us, 2),
        "decode_kernel_GBps": round(w.kv_bytes_per_layer() / (dec_us * 1e-6) / 1e9, 1),
        "kernels_us_per_step": res["kernels_us_per_step"],
        "host_us_per_step": round(res["host_us_per_step"], 1),
        "kv_bytes_per_step": res["kv_bytes_per_step"],
        "replicas": res["replicas"],
    }
    if res.get("flushed"):
        out["cache_flushed_p50_us"] = res["flushed"]["us_per_step"]["p50"]
        out["cache_flushed_GBps_at_p50"] = res["flushed"]["GBps_at_p50"]
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path runs on a "
              f"single MI355X and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    if args.workload.startswith("prefill"):
        prefill_main(args)
        return

    import torch
    from paged_kv_decode_02_amd import binding as B
    from paged_kv_decode_02_amd import workloads as W

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    B.lib()
    stream = torch.cuda.Stream(device=dev)     # default priority

    head = measure_decode(args.workload, args.steps, args.warmup, B, W, dev, stream, graph=args.graph)
    w = head["w"]
    configs = {}
    if not args.no_configs:
        for name in ("tiny", "c2", "c3", "c4", "c5"):
            if name == args.workload:
                continue
            r = measure_decode(name, args.steps, args.warmup, B, W, dev, stream, detail=False)
            configs[name] = config_summary(r)

    ceiling = ceiling_median = None
    if not args.no_ceiling:
        ceiling, ceiling_median = stream_ceiling(B, dev, stream)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    dec_avg_ms = head["decode_avg_ms"]
    achieved = w.kv_bytes_per_layer() / (dec_avg_ms * 1e-3) / 1e9
    traffic = counted_traffic(w.name)
    ms_step = head["ms_per_step"]
    value = head["value"]
    result = {
        "metric": "paged decode attention: achieved KV-read GB/s (% of HBM peak) + us/step",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "us_per_step": round(ms_step * 1e3, 1),
        "us_per_step_percentiles": head.get("pct"),
        "cache_flushed": head["flushed"],
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": head["workload"],
            "global_batch": w.num_seqs,
            "layers": w.num_layers,
            "q_heads": w.num_q_heads,
            "kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "page_tokens": W.PAGE,
            "mean_ctx": round(float(w.ctx_lens.mean()), 1),
            "kv_bytes_per_step": head["kv_bytes_per_step"],
            "pool_pages": w.num_pages,
            "replicas": head["replicas"],
            "launch": ("hip graph replay per step (plan copied to the device before it)" if args.graph
                       else "eager; plan made on the host each step, carried in the kernel arguments "
                            "when it fits 1 KiB, else copied to the device once per step"),
            "host_us_per_step": round(head["host_us_per_step"], 1),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_kernel",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
            "traffic_detail": ({"fetch_bytes": traffic["fetch_bytes_per_launch"],
                                "write_bytes": traffic["write_bytes_per_launch"],
                                "source": "profiles/decode_kernel_c4.md"} if traffic else None),
            "avg_launch_us": round(dec_avg_ms * 1e3, 2),
            "algorithmic_bytes_per_launch": w.kv_bytes_per_layer(),
        },
        "kernels_us_per_step": dict(head["kernels_us_per_step"],
                                    note="separate profiled pass; each kernel bracketed by HIP events"),
        "configs": configs,
        "stream_read_ceiling_GBps": None if ceiling is None else round(ceiling, 1),
        "stream_read_median_GBps": None if ceiling_median is None else round(ceiling_median, 1),
        "frac_of_stream_ceiling": None if ceiling is None else round(value / ceiling, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
