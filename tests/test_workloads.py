"""The seeded input generator (CPU only): determinism, host/torch agreement,
placement and poison rules, and shapes against the printed architecture."""

import json
import os

import numpy as np
import pytest

from paged_kv_decode_02_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_hash_matches_python_ints():
    idx = np.array([0, 1, 2, 12345, (1 << 32) - 1, 1 << 32, (1 << 33) + 7, 6_000_000_000], np.int64)
    got = W.hash32(7, 3, idx)
    key = W.stream_key(7, 3)
    for i, g in zip(idx.tolist(), got.tolist()):
        ref = W._mix32_int((i & W.MASK32) ^ W._mix32_int((i >> 32) ^ key))
        assert g == ref


def test_uint32_host_hash_matches_int64_form():
    rng = np.random.default_rng(11)
    idx = np.concatenate([np.arange(5000, dtype=np.int64),
                          rng.integers(0, 1 << 40, 20000, dtype=np.int64),
                          np.array([(1 << 32) - 1, 1 << 32, (1 << 33) + 7], np.int64)])
    for seed, stream in [(7, 3), (1004, 1), (1005, 5)]:
        assert np.array_equal(W.hash32_np(seed, stream, idx).astype(np.int64),
                              W.hash32(seed, stream, idx))


def test_torch_and_numpy_generators_agree():
    import torch
    w = W.custom(5, [1, 17, 40, 3], num_q_heads=8, num_kv_heads=2, head_dim=64)
    for which in "kv":
        host = w.pool_bits(which)
        dev = w.pool_device(which, "cpu", chunk_elems=1 << 12).numpy().view(np.uint16)
        assert np.array_equal(host, dev)


def test_normal_table():
    t = W.normal_table_bits(1.0)
    v = (t.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.diff(v) >= 0) and np.all(np.isfinite(v))
    assert np.array_equal(v, -v[::-1])
    assert abs(v.mean()) < 1e-9 and abs(v.std() - 1.0) < 2e-3
    h = (W.normal_table_bits(0.5).astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(h.astype(np.float64), v * 0.5)


@pytest.mark.parametrize("name", ["tiny", "c2", "c3", "c5"])
def test_named_workloads_deterministic_and_valid(name):
    a, b = W.make_workload(name), W.make_workload(name)
    assert np.array_equal(a.ctx_lens, b.ctx_lens)
    assert np.array_equal(a.block_tables, b.block_tables)
    _check_placement(a)


def test_c4_placement():
    w = W.make_workload("c4")
    assert w.num_layers == 16 and w.num_seqs == 256 and w.append
    assert w.ctx_lens.min() >= 16 and w.ctx_lens.max() <= 8192
    assert abs(np.median(w.ctx_lens) - 1024) < 200
    _check_placement(w)


def _check_placement(w):
    used = []
    for layer in range(w.num_layers):
        for b in range(w.num_seqs):
            pages = w.sequence_pages(layer, b)
            assert pages.size == -(-int(w.ctx_lens[b]) // 16)
            assert np.all((w.block_tables[layer, b] >= 0) & (w.block_tables[layer, b] < w.num_pages))
            used.append(pages)
    used = np.concatenate(used)
    assert np.unique(used).size == used.size, "a page is owned by two (layer, seq) units"
    present = w.ctx_lens - 1 if w.append else w.ctx_lens
    assert int(w.page_valid.sum()) == int(present.sum()) * w.num_layers
    spare = np.setdiff1d(np.arange(w.num_pages), used)
    assert np.all(w.page_valid[spare] == 0)


def test_poison_marks_exactly_the_empty_slots():
    w = W.custom(9, [5, 16, 33], num_q_heads=4, num_kv_heads=2, head_dim=64, append=True)
    k, v = w.pool_bits("k"), w.pool_bits("v")
    for b, n in enumerate(w.ctx_lens):
        pages = w.sequence_pages(0, b)
        for t in range(int(n)):
            p, s = pages[t // 16], t % 16
            is_nan = t == n - 1          # the append slot stays empty until written
            assert np.all((k[p, :, :, s, :] == W.NAN_BITS) == is_nan)
            assert np.all((v[p, :, :, s] == W.NAN_BITS) == is_nan)
    assert w.positions.tolist() == [4, 15, 32]


def test_shapes_follow_printed_architecture():
    arch = json.load(open(os.path.join(GOLDEN, "llama32_1b_architecture.json")))
    geo = json.load(open(os.path.join(GOLDEN, "page_geometry.json")))
    assert W.PAGE == geo["tokens_per_page"]
    for name in ["tiny", "c2", "c3", "c4"]:
        w = W.make_workload(name)
        assert w.num_q_heads * w.head_dim == arch["q_proj"][1]
        assert w.num_kv_heads * w.head_dim == arch["k_proj"][1] == arch["v_proj"][1]
        assert w.group == arch["q_heads_per_kv_head"]
    assert W.make_workload("c4").num_layers == arch["num_layers"]
    # 32 KiB of K+V per page per layer, so the default pool holds 4096 pages
    w = W.make_workload("c3")
    assert w.num_kv_heads * 16 * w.head_dim * 2 * 2 == 32 << 10
    assert (geo["default_pool_mib"] << 20) // (32 << 10) == 4096


@pytest.mark.parametrize("name", W.PREFILL_WORKLOADS)
def test_prefill_workloads(name):
    import torch
    w = W.make_prefill_workload(name)
    again = W.make_prefill_workload(name)
    assert np.array_equal(w.ctx_before, again.ctx_before) and np.array_equal(w.chunks, again.chunks)
    assert np.array_equal(w.base.block_tables, again.base.block_tables)
    qs = w.query_start
    assert qs[0] == 0 and qs[-1] == w.num_rows and np.all(np.diff(qs) == w.chunks)
    total = w.ctx_before + w.chunks
    assert np.array_equal(w.base.ctx_lens, total)
    assert int(total.max()) <= w.base.stride * W.PAGE
    used = np.concatenate([w.base.sequence_pages(l, b) for l in range(w.base.num_layers)
                           for b in range(len(total))])
    assert np.unique(used).size == used.size and used.min() >= 0 and used.max() < w.base.num_pages
    assert int(w.base.page_valid.sum()) == int(w.ctx_before.sum()) * w.base.num_layers
    # only the cached tokens are valid in the pool; the chunk's slots are poison
    b = int(np.argmax(w.ctx_before)) if w.ctx_before.max() > 0 else 0
    c = int(w.ctx_before[b])
    page = int(w.base.block_tables[0, b, c // W.PAGE])
    kp = w.base.pool_pages_bits("k", [page])[0]
    slots = np.arange(W.PAGE)
    assert np.all((kp[:, :, slots >= c % W.PAGE] == W.NAN_BITS))
    assert not np.any(kp[:, :, slots < c % W.PAGE] == W.NAN_BITS)
    # row generators: host rows equal the device-path rows, layers differ
    rows = np.array([0, 1, w.num_rows - 1])
    small = W.PrefillWorkload(base=w.base, ctx_before=w.ctx_before, chunks=w.chunks)
    dev = small.rows_device("k", "cpu") if w.base.num_layers * w.num_rows * w.base.num_kv_heads * w.base.head_dim < (1 << 26) else None
    host0 = w.rows_bits("k", 0, rows)
    if dev is not None:
        assert np.array_equal(dev[0, rows].numpy().view(np.uint16), host0)
    if w.base.num_layers > 1:
        assert not np.array_equal(w.rows_bits("k", 1, rows), host0)
    assert w.flops_per_layer() == 4 * w.base.head_dim * w.base.num_q_heads * sum(
        int(n) * int(cb) + int(n) * (int(n) + 1) // 2 for n, cb in zip(w.chunks, w.ctx_before))
