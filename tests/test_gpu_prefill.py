"""Paged prefill on the GPU (pa_kv_write, pa_prefill) against the oracle:
chunk writes bit for bit, causal attention rows within the parity bar, on
chunks that start and end inside pages, continue an existing cache (up to
5000 tokens), or are empty; grouped heads G = 1, 2, 4, 7, 8, 16; head_dim 64
and 128; and long prompts and the benchmark's workloads checked on sampled
rows."""

import numpy as np
import pytest

import oracle
from gpu_helpers import check_parity, device, log
from oracle_pins import make_prefill_case
from paged_kv_decode_02_amd import binding as B

pytestmark = pytest.mark.gpu


class PrefillCase:
    def __init__(self, seed, hq, hkv, d, befores, chunks, sigma=1.0, scale=None):
        import torch
        dev = device()
        rng = np.random.default_rng(seed)
        (self.q, self.kc, self.vc, self.k_pool, self.v_pool, self.bt, self.qs, self.bef,
         self.k_rows, self.v_rows) = make_prefill_case(rng, hq, hkv, d, befores, chunks, sigma=sigma)
        self.scale = np.float32(1.0 / np.sqrt(d)) if scale is None else np.float32(scale)
        t = lambda a, dt=np.int16: torch.from_numpy(np.ascontiguousarray(a).view(dt) if dt == np.int16
                                                     else np.ascontiguousarray(a.astype(dt))).to(dev)
        self.k_dev, self.v_dev = t(self.k_pool), t(self.v_pool)
        self.pool = B.Pool(self.k_dev, self.v_dev)
        self.q_dev, self.kr_dev, self.vr_dev = t(self.q), t(self.k_rows), t(self.v_rows)
        self.qs_dev, self.bt_dev, self.bef_dev = t(self.qs, np.int32), t(self.bt, np.int32), t(self.bef, np.int32)
        self.max_chunk = int(max(chunks)) if len(chunks) else 0

    def run(self, max_chunk=None):
        return B.prefill(self.pool, self.q_dev, self.kr_dev, self.vr_dev, self.qs_dev, self.bt_dev,
                         self.bef_dev, float(self.scale), self.max_chunk if max_chunk is None else max_chunk)

    def run_planned(self):
        """pa_prefill_planned with the host-made plan for this case's lengths."""
        import torch
        plan = B.prefill_plan(self.pool, self.bef, np.diff(self.qs), self.q.shape[1], self.bt.shape[1],
                              self.max_chunk)
        plan_dev = torch.from_numpy(plan).to(self.q_dev.device)
        return B.prefill_planned(self.pool, self.q_dev, self.kr_dev, self.vr_dev, self.qs_dev, self.bt_dev,
                                 self.bef_dev, float(self.scale), self.max_chunk, plan_dev)

    def pools(self):
        return (self.k_dev.cpu().numpy().view(np.uint16), self.v_dev.cpu().numpy().view(np.uint16))


CASES = [
    # (label, Hq, Hkv, d, cache before the chunk, chunk lengths)
    ("fresh_d64", 32, 8, 64, [0, 0, 0], [1, 16, 75]),
    ("continue_d64", 32, 8, 64, [17, 100, 16, 5], [64, 3, 33, 0]),
    ("g7_d128", 28, 4, 128, [0, 33, 250], [130, 7, 1]),
    ("g16_d64", 32, 2, 64, [9], [70]),
    ("g1_d64", 8, 8, 64, [40, 0], [25, 48]),
    ("g8_d128", 8, 1, 128, [15], [49]),
    ("g16_d128", 32, 2, 128, [0, 40], [33, 90]),
    ("g2_d64", 4, 2, 64, [3], [130]),
    # rows that see more than 2048 keys (caches of up to 5000 tokens)
    ("long_cache_d64", 32, 8, 64, [3000, 70, 5000], [40, 200, 130]),
    ("long_cache_d128", 28, 4, 128, [4100, 2000], [33, 150]),
    ("across_2048_d64", 8, 2, 64, [1990], [300]),
    ("long_fresh_g8", 8, 1, 64, [0], [2500]),
]


@pytest.mark.parametrize("label,hq,hkv,d,befores,chunks", CASES, ids=[c[0] for c in CASES])
def test_prefill_matches_oracle(label, hq, hkv, d, befores, chunks):
    import zlib
    c = PrefillCase(zlib.crc32(label.encode()) % 10_000, hq, hkv, d, befores, chunks)
    log(f"prefill {label}: before={befores} chunks={chunks} Hq={hq} Hkv={hkv} d={d} entry=pa_prefill")
    out = c.run().cpu().numpy()
    ref, k_ref, v_ref = oracle.prefill_attention(c.q, c.k_pool, c.v_pool, c.k_rows, c.v_rows, c.qs,
                                                 c.bt, c.bef, c.scale)
    k_got, v_got = c.pools()
    assert np.array_equal(k_got, k_ref), f"{label}: K pool differs from the oracle's write"
    assert np.array_equal(v_got, v_ref), f"{label}: V pool differs from the oracle's write"
    a, r = check_parity(out, ref, label)
    # a looser grid bound changes nothing; a second run gives the same bits
    again = c.run(max_chunk=c.max_chunk + 37).cpu().numpy()
    assert np.array_equal(again, out), f"{label}: result depends on the grid bound or the run"
    # the launch plan changes only the order of the row blocks
    planned = c.run_planned().cpu().numpy()
    assert np.array_equal(planned, out), f"{label}: pa_prefill_planned differs from pa_prefill"
    log(f"prefill {label}: max abs {a:.2e} max rel {r:.2e}")


def test_prefill_plan_items_out_of_range_are_skipped():
    """A plan holding items that name a sequence or a row block past the grid
    gives the same rows as pa_prefill (those items do nothing)."""
    import torch
    c = PrefillCase(77, 32, 8, 64, [17, 100, 16, 5], [64, 3, 33, 0])
    log("prefill plan with out-of-range items: before=[17, 100, 16, 5] chunks=[64, 3, 33, 0]")
    plain = c.run().cpu().numpy()
    plan = B.prefill_plan(c.pool, c.bef, np.diff(c.qs), 32, c.bt.shape[1], c.max_chunk)
    row_blocks = -(-c.max_chunk * 4 // 128)
    bogus = np.array([4 + 5, row_blocks << 20], dtype=np.int32)       # sequence 9; row block past the grid
    p = np.concatenate([plan, bogus])
    assert p.size <= B.prefill_plan_capacity(c.pool, 4, 32, c.max_chunk)
    out = torch.full((c.q.shape[0], 32, 64), float("nan"), device=c.q_dev.device)
    B.prefill_planned(c.pool, c.q_dev, c.kr_dev, c.vr_dev, c.qs_dev, c.bt_dev, c.bef_dev, float(c.scale),
                      c.max_chunk, torch.from_numpy(p).to(c.q_dev.device), out=out)
    assert np.array_equal(out.cpu().numpy(), plain), "out-of-range plan items changed the result"


def test_prefill_batch_invariance_bitwise():
    """A sequence's rows do not depend on the rest of the batch: each sequence
    prefilled alone (same pages, same block-table row) gives the rows it got
    inside the batch bit for bit, planned or not."""
    import torch
    befores, chunks = [0, 300, 17, 2100], [200, 45, 130, 64]
    c = PrefillCase(91, 32, 8, 64, befores, chunks)
    log(f"prefill batch invariance: before={befores} chunks={chunks}")
    batch = c.run().cpu().numpy()
    planned = c.run_planned().cpu().numpy()
    assert np.array_equal(batch, planned)
    dev = c.q_dev.device
    for b in range(len(chunks)):
        r0, r1 = int(c.qs[b]), int(c.qs[b + 1])
        qs1 = torch.tensor([0, r1 - r0], dtype=torch.int32, device=dev)
        out = B.prefill(c.pool, c.q_dev[r0:r1].contiguous(), c.kr_dev[r0:r1].contiguous(),
                        c.vr_dev[r0:r1].contiguous(), qs1, c.bt_dev[b:b + 1].contiguous(),
                        c.bef_dev[b:b + 1].contiguous(), float(c.scale), chunks[b])
        assert np.array_equal(out.cpu().numpy(), batch[r0:r1]), f"sequence {b}: rows differ alone vs in the batch"


def test_kv_write_alone_bit_exact():
    c = PrefillCase(5, 32, 8, 64, [0, 7, 31, 48], [40, 9, 1, 16])
    log("kv_write: before=[0,7,31,48] chunks=[40,9,1,16] entry=pa_kv_write")
    B.kv_write(c.pool, c.kr_dev, c.vr_dev, c.qs_dev, c.bt_dev, c.bef_dev, c.max_chunk)
    k_ref, v_ref = oracle.kv_write(c.k_pool, c.v_pool, c.k_rows, c.v_rows, c.qs, c.bt, c.bef)
    k_got, v_got = c.pools()
    assert np.array_equal(k_got, k_ref) and np.array_equal(v_got, v_ref)


def test_prefill_then_decode_continues_the_cache():
    """Prefill a prompt, then one decode step over prompt + 1 tokens: both
    match the oracle run on the same sequence of operations."""
    import torch
    dev = device()
    c = PrefillCase(6, 32, 8, 64, [0, 0], [100, 37])
    log("prefill then decode: chunks=[100,37] entry=pa_prefill+pa_kv_append+pa_decode")
    c.run()
    k1, v1 = oracle.kv_write(c.k_pool, c.v_pool, c.k_rows, c.v_rows, c.qs, c.bt, c.bef)
    rng = np.random.default_rng(7)
    from oracle_pins import random_bf16
    kn, vn = random_bf16(rng, (2, 8, 64)), random_bf16(rng, (2, 8, 64))
    qd = random_bf16(rng, (2, 32, 64))
    pos = (c.bef + np.diff(c.qs)).astype(np.int32)
    B.kv_append(c.pool, torch.from_numpy(kn.view(np.int16)).to(dev), torch.from_numpy(vn.view(np.int16)).to(dev),
                c.bt_dev, torch.from_numpy(pos).to(dev))
    out = B.decode(c.pool, torch.from_numpy(qd.view(np.int16)).to(dev), c.bt_dev,
                   torch.from_numpy(pos + 1).to(dev), float(c.scale)).cpu().numpy()
    k2, v2 = oracle.kv_append(k1, v1, kn, vn, c.bt, pos)
    check_parity(out, oracle.decode_attention(qd, k2, v2, c.bt, pos + 1, c.scale), "decode after prefill")


@pytest.mark.parametrize("d,hq,hkv", [(64, 32, 8), (128, 28, 4)])
def test_long_prompt_sampled_rows(d, hq, hkv):
    """A 2048-token prompt (and a 700-token one continuing a 1000-token cache):
    sampled rows against the oracle computed row by row."""
    c = PrefillCase(8 + d, hq, hkv, d, [0, 1000], [2048, 700])
    log(f"prefill long: d={d} chunks=[2048,700] before=[0,1000] entry=pa_prefill")
    out = c.run().cpu().numpy()
    k_ref, v_ref = oracle.kv_write(c.k_pool, c.v_pool, c.k_rows, c.v_rows, c.qs, c.bt, c.bef)
    k_got, v_got = c.pools()
    assert np.array_equal(k_got, k_ref) and np.array_equal(v_got, v_ref)
    rng = np.random.default_rng(9)
    g = hq // hkv
    for b in range(2):
        n = int(c.bef[b]) + int(c.qs[b + 1] - c.qs[b])
        kc, vc = oracle.gather_sequence(k_ref, v_ref, c.bt[b], n)
        rows = sorted({0, int(c.qs[b + 1] - c.qs[b]) - 1, *rng.integers(0, c.qs[b + 1] - c.qs[b], 6).tolist()})
        for i in rows:
            p = int(c.bef[b]) + i
            row = int(c.qs[b]) + i
            qr = oracle.bf16_bits_to_f64(c.q[row])
            ref = np.stack([oracle.attend_one_head(qr[h], kc[:p + 1, h // g], vc[:p + 1, h // g], float(c.scale))
                            for h in range(hq)])
            check_parity(out[row], ref, f"long prefill b={b} row {i}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 3.0])
def test_prefill_any_scale(scale):
    """Negative, zero and large softmax scales (a negative scale reverses the
    order of the scores; zero gives the mean of the visible values)."""
    c = PrefillCase(12, 32, 8, 64, [0, 21], [70, 45], scale=scale)
    log(f"prefill scale {scale}: chunks=[70,45] before=[0,21] entry=pa_prefill")
    out = c.run().cpu().numpy()
    ref, _, _ = oracle.prefill_attention(c.q, c.k_pool, c.v_pool, c.k_rows, c.v_rows, c.qs, c.bt, c.bef,
                                         c.scale)
    check_parity(out, ref, f"prefill scale {scale}")


@pytest.mark.parametrize("name", ["prefill", "prefill_d128", "prefill_chunked"])
def test_prefill_workload_full_size_sampled(name):
    """The benchmark's prefill workloads at full size, launched as the
    benchmark launches them (one pa_prefill_planned per layer over the whole
    batch, with the host-made plan): the same bits as pa_prefill; on sampled
    sequences of the first and last layer, the pages after the chunk write
    equal the oracle's write bit for bit, and sampled chunk rows (always the
    first and the last) match the oracle computed row by row."""
    import torch
    from paged_kv_decode_02_amd import workloads as W
    dev = device()
    w = W.make_prefill_workload(name)
    base = w.base
    k_dev, v_dev = base.pool_device("k", dev), base.pool_device("v", dev)
    pool = B.Pool(k_dev, v_dev)
    bt = torch.from_numpy(np.ascontiguousarray(base.block_tables)).to(dev)
    qs = torch.from_numpy(w.query_start).to(dev)
    before = torch.from_numpy(w.ctx_before).to(dev)
    q, k_rows, v_rows = w.rows_device("q", dev), w.rows_device("k", dev), w.rows_device("v", dev)
    g = base.num_q_heads // base.num_kv_heads
    rng = np.random.default_rng(31)
    max_chunk = int(w.chunks.max())
    plan = torch.from_numpy(B.prefill_plan(pool, w.ctx_before, w.chunks, base.num_q_heads,
                                           base.block_tables.shape[2], max_chunk)).to(dev)
    for layer in sorted({0, base.num_layers - 1}):
        log(f"{name}: layer {layer}, {w.num_rows} rows, before={w.ctx_before.tolist()} "
            f"entry=pa_prefill_planned ({plan.numel()} items)")
        out = B.prefill_planned(pool, q[layer], k_rows[layer], v_rows[layer], qs, bt[layer], before,
                                float(base.scale), max_chunk, plan).cpu().numpy()
        plain = B.prefill(pool, q[layer], k_rows[layer], v_rows[layer], qs, bt[layer], before,
                          float(base.scale), max_chunk).cpu().numpy()
        assert np.array_equal(plain, out), f"{name} layer {layer}: pa_prefill_planned != pa_prefill"
        del plain
        for b in sorted(rng.choice(len(w.chunks), size=min(3, len(w.chunks)), replace=False).tolist()):
            n_tot = int(w.ctx_before[b]) + int(w.chunks[b])
            pages = base.block_tables[layer, b, :-(-n_tot // 16)].astype(np.int64)
            rows = np.arange(w.query_start[b], w.query_start[b + 1])
            local_bt = np.arange(pages.size, dtype=np.int32)[None, :]
            kp, vp = oracle.kv_write(base.pool_pages_bits("k", pages), base.pool_pages_bits("v", pages),
                                     w.rows_bits("k", layer, rows), w.rows_bits("v", layer, rows),
                                     np.array([0, rows.size]), local_bt, np.array([w.ctx_before[b]]))
            idx = torch.from_numpy(pages).to(dev)
            assert np.array_equal(k_dev[idx].cpu().numpy().view(np.uint16), kp), f"{name} K pages, seq {b}"
            assert np.array_equal(v_dev[idx].cpu().numpy().view(np.uint16), vp), f"{name} V pages, seq {b}"
            kc, vc = oracle.gather_sequence(kp, vp, local_bt[0], n_tot)
            pick = sorted({0, rows.size - 1, *rng.integers(0, rows.size, 4).tolist()})
            qsel = w.rows_bits("q", layer, rows[pick])
            for j, i in enumerate(pick):
                p = int(w.ctx_before[b]) + i
                qr = oracle.bf16_bits_to_f64(qsel[j])
                ref = np.stack([oracle.attend_one_head(qr[h], kc[:p + 1, h // g], vc[:p + 1, h // g],
                                                       float(base.scale)) for h in range(base.num_q_heads)])
                check_parity(out[rows[i]], ref, f"{name} layer {layer} seq {b} row {i}")
        del out
