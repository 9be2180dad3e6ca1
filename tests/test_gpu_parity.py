"""GPU parity: the HIP path through the C ABI against the FP64 oracle on the
same seeded BF16 inputs.

* Tiny, C2 and C3 workloads: every output element.
* C5 (64 x up to 16K tokens, 28q/4kv, d=128) and C4 (16 layers x 256 seqs,
  append then decode): launched at full size exactly as the benchmark does,
  checked on sampled sequences the oracle computes one by one (including the
  longest and shortest contexts).
* Edge cases on small custom workloads: empty contexts, one token, page and
  split boundaries, ragged tails, group sizes 1..16, one KV head, contexts
  filling the whole block table.
"""

import zlib

import numpy as np
import pytest

import oracle
from gpu_helpers import Uploaded, check_parity, device, log, oracle_rows
from paged_kv_decode_02_amd import binding as B
from paged_kv_decode_02_amd import workloads as W

pytestmark = pytest.mark.gpu


def full_oracle(w, up):
    k = w.pool_bits("k")
    v = w.pool_bits("v")
    outs = []
    for layer in range(w.num_layers):
        kk, vv = k, v
        if w.append:
            kk, vv = oracle.kv_append(k, v, up.k_new_host[layer], up.v_new_host[layer],
                                      w.block_tables[layer], w.positions)
        outs.append(oracle.decode_attention(up.q_host[layer], kk, vv, w.block_tables[layer],
                                            w.ctx_lens, w.scale))
    return np.stack(outs)


@pytest.mark.parametrize("name", ["tiny", "c2", "c3"])
def test_named_workload_all_outputs(name):
    import torch
    dev = device()
    w = W.make_workload(name)
    log(f"{name}: B={w.num_seqs} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"pages={w.num_pages} max_ctx={w.ctx_lens.max()} entry=pa_decode")
    up = Uploaded(w, dev)
    out = up.step().cpu().numpy()
    torch.cuda.synchronize()
    ref = full_oracle(w, up)
    a, r = check_parity(out, ref, name)
    log(f"{name}: max abs {a:.2e} max rel {r:.2e}")


def _sample(w, k=8):
    order = np.argsort(w.ctx_lens, kind="stable")
    picks = {int(order[0]), int(order[-1]), int(order[len(order) // 2])}
    rng = np.random.default_rng(7)
    picks.update(int(x) for x in rng.choice(w.num_seqs, size=k, replace=False))
    return sorted(picks)


def test_c5_full_launch_sampled():
    dev = device()
    w = W.make_workload("c5")
    log(f"c5: B=64 Hq=28 Hkv=4 d=128 pages={w.num_pages} max_ctx={w.ctx_lens.max()} entry=pa_decode")
    up = Uploaded(w, dev)
    out = up.step().cpu().numpy()
    seqs = _sample(w)
    ref = oracle_rows(w, 0, seqs, up.q_host)
    a, r = check_parity(out[0, seqs], ref, "c5 sampled")
    log(f"c5 sampled {seqs}: max abs {a:.2e} max rel {r:.2e}")


def test_c4_full_step_sampled():
    import torch
    dev = device()
    w = W.make_workload("c4")
    log(f"c4: L=16 B=256 pages={w.num_pages} max_ctx={w.ctx_lens.max()} entry=pa_kv_append+pa_decode_planned")
    up = Uploaded(w, dev)
    out = up.step(fused=False, planned=True).cpu().numpy()   # the step the benchmark times
    torch.cuda.synchronize()
    # the plan changes only the launch order: pa_decode gives the same bits
    for layer in (0, 15):
        plain = B.decode(up.pool, up.q[layer], up.bt[layer], up.ctx, float(w.scale), workspace=up.workspace)
        assert np.array_equal(plain.cpu().numpy(), out[layer]), f"c4 layer {layer}: planned != plain"
    rng = np.random.default_rng(3)
    order = np.argsort(w.ctx_lens, kind="stable")
    cases = [(0, int(order[-1])), (15, int(order[0])), (7, int(order[128]))]
    cases += [(int(rng.integers(16)), int(rng.integers(256))) for _ in range(6)]
    for layer, b in cases:
        ref = oracle_rows(w, layer, [b], up.q_host, up.k_new_host, up.v_new_host)
        a, r = check_parity(out[layer, [b]], ref, f"c4 layer {layer} seq {b}")
        # the appended slot, and the rest of its page, bit for bit
        n = int(w.ctx_lens[b])
        page = int(w.block_tables[layer, b, (n - 1) // 16])
        exp_k, exp_v = oracle.kv_append(w.pool_pages_bits("k", [page]), w.pool_pages_bits("v", [page]),
                                        up.k_new_host[layer][b:b + 1], up.v_new_host[layer][b:b + 1],
                                        np.zeros((1, 1), np.int32), np.array([(n - 1) % 16], np.int32))
        got_k = up.k_pool[page].cpu().numpy().view(np.uint16)
        got_v = up.v_pool[page].cpu().numpy().view(np.uint16)
        assert np.array_equal(got_k, exp_k[0]), f"c4 append K page {page}"
        assert np.array_equal(got_v, exp_v[0]), f"c4 append V page {page}"
        log(f"c4 layer {layer} seq {b} ctx {n}: max abs {a:.2e} max rel {r:.2e}")


EDGE_CASES = [
    # (label, ctx_lens, Hq, Hkv, d)
    ("empty_and_one", [0, 1, 0, 2, 3], 32, 8, 64),
    ("page_boundaries", [15, 16, 17, 31, 32, 33, 47, 48, 49], 32, 8, 64),
    ("split_boundaries", [511, 512, 513, 1023, 1024, 1025, 1535], 32, 8, 64),
    ("long_d64", [8192, 4099, 6000], 32, 8, 64),
    ("mha_group1", [100, 300, 7], 8, 8, 64),
    ("group2_one_kv", [77, 600], 2, 1, 64),
    ("group16", [250, 513, 33], 32, 2, 64),
    ("group7_d128", [1, 17, 512, 513, 2000, 4097], 28, 4, 128),
    ("group8_d128", [300, 1100], 8, 1, 128),
    ("group16_d128", [65, 1500], 32, 2, 128),
    ("long_d128", [16384, 12345], 28, 4, 128),
    ("beyond_64_splits_d64", [70000, 3, 65537], 32, 8, 64),
    ("ragged_many", list(np.random.default_rng(4).integers(0, 700, 37)), 32, 8, 64),
]


@pytest.mark.parametrize("label,ctx,hq,hkv,d", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_cases(label, ctx, hq, hkv, d):
    dev = device()
    w = W.custom(seed=zlib.crc32(label.encode()) % 10_000, ctx_lens=ctx, num_q_heads=hq, num_kv_heads=hkv,
                 head_dim=d, name=label)
    log(f"edge {label}: ctx={list(map(int, ctx))[:12]} Hq={hq} Hkv={hkv} d={d} entry=pa_decode")
    up = Uploaded(w, dev)
    out = up.step().cpu().numpy()
    ref = full_oracle(w, up)
    a, r = check_parity(out, ref, label)
    planned = up.step(fused=False, planned=True).cpu().numpy()
    assert np.array_equal(planned, out), f"{label}: pa_decode_planned differs from pa_decode"
    for b, n in enumerate(w.ctx_lens):
        if n == 0:
            assert np.array_equal(out[0, b], np.zeros_like(out[0, b])), "ctx 0 must give zeros"
    log(f"edge {label}: max abs {a:.2e} max rel {r:.2e}")


def test_full_block_table_context():
    """Contexts that fill every entry of the block table (stride * 16 tokens)."""
    dev = device()
    for d, hq, hkv, stride in [(64, 32, 8, 40), (128, 28, 4, 70)]:
        ctx = [stride * 16, stride * 16 - 5, 1]
        w = W.custom(seed=31 + d, ctx_lens=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                     stride=stride)
        log(f"full table d={d} stride={stride} ctx={ctx} entry=pa_decode")
        up = Uploaded(w, dev)
        out = up.step().cpu().numpy()
        check_parity(out, full_oracle(w, up), f"full table d={d}")
