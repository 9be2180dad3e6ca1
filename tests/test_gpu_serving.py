"""A small continuous-batching loop on the GPU over pages handed out by the host
scheduler (pakv_sched.h): requests are admitted in order as pages free up, one
shares its parent's prefix pages, every running request writes one token per
step (pa_kv_append) and attends over its cache (pa_decode). Every step's
output is checked against the oracle over a host mirror of the pool, and the
pool itself is compared bit for bit at the end."""

import numpy as np
import pytest

import oracle
from gpu_helpers import check_parity, device, log
from oracle_pins import f32_to_bf16_bits
from paged_kv_decode_02_amd import binding as B

pytestmark = pytest.mark.gpu

NAN = 0x7FC0


def test_serving_loop_over_scheduler_pages():
    import torch
    dev = device()
    P, L, MB, STRIDE = 48, 2, 4, 16
    HQ, HKV, D = 32, 8, 64
    scale = 0.125
    rng = np.random.default_rng(2024)
    sched = B.Scheduler(P, L, MB, STRIDE)
    k_host = np.full((P, HKV, D // 32, 16, 32), NAN, np.uint16)
    v_host = np.full((P, HKV, D, 16), NAN, np.uint16)
    k_dev = torch.from_numpy(k_host.view(np.int16).copy()).to(dev)
    v_dev = torch.from_numpy(v_host.view(np.int16).copy()).to(dev)
    pool = B.Pool(k_dev, v_dev)
    ws = torch.empty(max(B.decode_workspace_bytes(pool, MB, HQ, STRIDE), 16), dtype=torch.uint8, device=dev)

    budget = {}                                     # id -> prompt + max_new
    r1 = sched.submit(40, 6)
    r2 = sched.submit(100, 4)
    budget[r1], budget[r2] = 46, 104
    pending_shared = True
    r4 = None
    steps = 0
    checked = 0
    while True:
        admitted = sched.admit()
        if admitted:
            log(f"step {steps}: admitted {admitted}, stats {sched.stats()}")
        slot_of = {rid: sched.slot(rid) for rid in budget}
        active = {rid: s for rid, s in slot_of.items() if s >= 0}
        if not active and sched.stats()["queued"] == 0:
            break
        # one token per running request: K/V rows for every layer
        pos = np.full(MB, -1, np.int32)
        for rid, slot in active.items():
            pos[slot] = sched.context_lens[slot]
        bt_all = sched.block_tables.copy()
        for layer in range(L):
            kn = f32_to_bf16_bits(rng.standard_normal((MB, HKV, D), dtype=np.float32))
            vn = f32_to_bf16_bits(rng.standard_normal((MB, HKV, D), dtype=np.float32))
            bt = np.ascontiguousarray(bt_all[layer])
            B.kv_append(pool, torch.from_numpy(kn.view(np.int16)).to(dev),
                        torch.from_numpy(vn.view(np.int16)).to(dev), torch.from_numpy(bt).to(dev),
                        torch.from_numpy(pos).to(dev))
            k_host, v_host = oracle.kv_append(k_host, v_host, kn, vn, bt, pos)
        for rid, slot in active.items():
            sched.advance(rid, 1)
        ctx = sched.context_lens.copy()
        for layer in range(L):
            q = f32_to_bf16_bits(rng.standard_normal((MB, HQ, D), dtype=np.float32))
            bt = np.ascontiguousarray(bt_all[layer])
            out = B.decode(pool, torch.from_numpy(q.view(np.int16)).to(dev), torch.from_numpy(bt).to(dev),
                           torch.from_numpy(ctx).to(dev), scale, workspace=ws).cpu().numpy()
            ref = oracle.decode_attention(q, k_host, v_host, np.where(bt < 0, 0, bt), ctx, scale)
            check_parity(out, ref, f"step {steps} layer {layer}")
            checked += 1
        steps += 1
        # the shared-prefix request joins once r1's prompt is in the cache
        if pending_shared and slot_of.get(r1, -1) >= 0 and sched.context_lens[slot_of[r1]] >= 40:
            r3 = sched.submit_shared(r1, 35, 50, 5)            # two full pages per layer shared
            budget[r3] = 55
            r4 = sched.submit(200, 3)                          # 26 pages: waits for free pages
            budget[r4] = 203
            pending_shared = False
            log(f"step {steps}: submitted shared {r3} (parent {r1}) and {r4}, stats {sched.stats()}")
        for rid, slot in list(active.items()):
            if sched.context_lens[slot] >= budget[rid]:
                sched.finish(rid)
                del budget[rid]
        assert steps < 400
    assert r4 is not None and not budget
    assert sched.stats() == {"free_pages": P, "queued": 0, "running": 0}
    assert np.array_equal(k_dev.cpu().numpy().view(np.uint16), k_host)
    assert np.array_equal(v_dev.cpu().numpy().view(np.uint16), v_host)
    log(f"serving loop: {steps} steps, {checked} decode launches checked against the oracle")


def test_chunked_prefill_then_decode_over_scheduler_pages():
    """Requests from the scheduler are prefilled in chunks with pa_prefill (a
    shared-prefix request continues from its parent's cached pages), then
    decode one token per step. Every prefill row and decode output is checked
    against the oracle over a host mirror of the pool."""
    import torch
    dev = device()
    P, L, MB, STRIDE = 80, 2, 4, 24
    HQ, HKV, D = 28, 4, 128
    scale = float(np.float32(1.0 / np.sqrt(D)))
    rng = np.random.default_rng(77)
    sched = B.Scheduler(P, L, MB, STRIDE)
    k_host = np.full((P, HKV, D // 32, 16, 32), NAN, np.uint16)
    v_host = np.full((P, HKV, D, 16), NAN, np.uint16)
    k_dev = torch.from_numpy(k_host.view(np.int16).copy()).to(dev)
    v_dev = torch.from_numpy(v_host.view(np.int16).copy()).to(dev)
    pool = B.Pool(k_dev, v_dev)
    t = lambda a, dt=np.int32: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).to(dev)
    bits = lambda shape: f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))

    a = sched.submit(150, 3)
    b = sched.submit(37, 4)
    assert sched.admit() == [a, b]
    prompt = {a: 150, b: 37}
    budget = {a: 153, b: 41}
    CHUNK = 64
    child = None
    checked = 0
    for step in range(40):
        if not budget:
            break
        ctx0 = sched.context_lens.copy()
        bt_all = sched.block_tables.copy()
        # every running request takes its next chunk: up to CHUNK prompt tokens, or one decode token
        lens = np.zeros(MB, np.int64)
        owner = {}
        for rid in list(budget):
            slot = sched.slot(rid)
            if slot < 0:
                continue
            owner[slot] = rid
            c = int(ctx0[slot])
            lens[slot] = min(CHUNK, prompt[rid] - c) if c < prompt[rid] else 1
        qs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        n = int(qs[-1])
        q, kr, vr = bits((n, HQ, D)), bits((n, HKV, D)), bits((n, HKV, D))
        for layer in range(L):
            bt = np.where(bt_all[layer] < 0, 0, bt_all[layer]).astype(np.int32)
            out = B.prefill(pool, t(q.view(np.int16), np.int16), t(kr.view(np.int16), np.int16),
                            t(vr.view(np.int16), np.int16), t(qs), t(bt), t(ctx0), scale,
                            int(lens.max())).cpu().numpy()
            ref, k_host, v_host = oracle.prefill_attention(q, k_host, v_host, kr, vr, qs, bt, ctx0, scale)
            check_parity(out, ref, f"step {step} layer {layer}")
            checked += 1
        for slot, rid in owner.items():
            sched.advance(rid, int(lens[slot]))
        if child is None and sched.context_lens[sched.slot(a)] >= 150:
            child = sched.submit_shared(a, 150, 170, 2)          # 9 full pages per layer shared
            prompt[child], budget[child] = 170, 172
            assert sched.admit() == [child]
            assert sched.context_lens[sched.slot(child)] == 144
        for rid in list(budget):
            slot = sched.slot(rid)
            if slot >= 0 and sched.context_lens[slot] >= budget[rid]:
                sched.finish(rid)
                del budget[rid]
    assert not budget and child is not None
    assert np.array_equal(k_dev.cpu().numpy().view(np.uint16), k_host)
    assert np.array_equal(v_dev.cpu().numpy().view(np.uint16), v_host)
    assert sched.stats() == {"free_pages": P, "queued": 0, "running": 0}
    log(f"chunked prefill loop: {checked} prefill launches checked")
