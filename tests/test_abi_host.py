"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments with the documented status codes before
queueing any GPU work (fake device pointers; no kernel is launched)."""

import ctypes
import os
import re

import pytest

from paged_kv_decode_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pakv.h")

OK, NULL, INVALID, UNSUPPORTED, ALIGN, WORKSPACE = 0, 1, 2, 3, 4, 5
P = 0x10000          # fake 16-byte-aligned "device" addresses
P2 = 0x20000
MIS = 0x10008


def header_functions():
    text = "".join(open(os.path.join(ROOT, "include", f)).read() for f in sorted(os.listdir(os.path.join(ROOT, "include"))) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = B.lib()
    names = header_functions()
    assert names, "no declarations parsed"
    for n in names:
        assert hasattr(L, n), f"libpakv.so does not export {n}"
    assert sorted(B.EXPORTS) == names


def make_pool(num_pages=64, hkv=8, d=64):
    h = ctypes.c_void_p()
    st = B.lib().pa_pool_create(ctypes.byref(h), P, P2, num_pages, 16, hkv, d)
    assert st == OK
    return h


def test_pool_create_validation():
    L = B.lib()
    h = ctypes.c_void_p()
    assert L.pa_pool_create(None, P, P2, 4, 16, 8, 64) == NULL
    assert L.pa_pool_create(ctypes.byref(h), 0, P2, 4, 16, 8, 64) == NULL
    assert L.pa_pool_create(ctypes.byref(h), P, 0, 4, 16, 8, 64) == NULL
    assert L.pa_pool_create(ctypes.byref(h), P, P2, 0, 16, 8, 64) == INVALID
    assert L.pa_pool_create(ctypes.byref(h), P, P2, 4, 16, 0, 64) == INVALID
    assert L.pa_pool_create(ctypes.byref(h), P, P2, 4, 32, 8, 64) == UNSUPPORTED
    assert L.pa_pool_create(ctypes.byref(h), P, P2, 4, 16, 8, 96) == UNSUPPORTED
    assert L.pa_pool_create(ctypes.byref(h), MIS, P2, 4, 16, 8, 64) == ALIGN
    assert L.pa_pool_create(ctypes.byref(h), P, P2, 4, 16, 8, 128) == OK
    L.pa_pool_destroy(h)
    L.pa_pool_destroy(None)


def test_decode_validation():
    L = B.lib()
    pool = make_pool()
    f = lambda **kw: L.pa_decode(kw.get("pool", pool), kw.get("q", P), kw.get("B", 4), kw.get("Hq", 32),
                                 kw.get("bt", P), kw.get("stride", 600), kw.get("ctx", P),
                                 kw.get("scale", 0.125), kw.get("out", P), kw.get("ws", P),
                                 kw.get("ws_bytes", 1 << 30), None)
    assert f(pool=None) == NULL
    assert f(q=0) == NULL
    assert f(bt=0) == NULL
    assert f(ctx=0) == NULL
    assert f(out=0) == NULL
    assert f(B=-1) == INVALID
    assert f(Hq=0) == INVALID
    assert f(Hq=12) == INVALID                # not a multiple of 8 KV heads
    assert f(Hq=8 * 17) == UNSUPPORTED        # 17 query heads per KV head
    assert f(stride=0) == INVALID
    assert f(scale=float("inf")) == INVALID
    assert f(scale=float("nan")) == INVALID
    assert f(scale=3.0e38) == INVALID          # scale * log2(e) overflows FP32
    assert f(q=MIS) == ALIGN
    assert f(out=MIS) == ALIGN
    assert f(ctx=MIS + 1) == ALIGN
    assert f(ws=0) == WORKSPACE                # 600 pages: 5 splits, more than a workgroup finishes
    need = L.pa_decode_workspace_bytes(pool, 4, 32, 600)
    assert need > 0
    assert f(ws_bytes=need - 1) == WORKSPACE
    assert f(ws=MIS, ws_bytes=need) == ALIGN
    assert f(B=0) == OK                       # nothing to do, nothing queued
    L.pa_pool_destroy(pool)


def test_decode_append_validation():
    L = B.lib()
    pool = make_pool()
    f = lambda **kw: L.pa_decode_append(kw.get("pool", pool), kw.get("q", P), kw.get("k", P),
                                        kw.get("v", P), kw.get("pos", P), kw.get("B", 4),
                                        kw.get("Hq", 32), kw.get("bt", P), kw.get("stride", 600),
                                        kw.get("ctx", P), kw.get("scale", 0.125), kw.get("out", P),
                                        kw.get("ws", P), kw.get("ws_bytes", 1 << 30), None)
    assert f(pool=None) == NULL
    assert f(k=0) == NULL
    assert f(v=0) == NULL
    assert f(pos=0) == NULL
    assert f(q=0) == NULL
    assert f(k=MIS) == ALIGN
    assert f(pos=MIS + 2) == ALIGN
    assert f(Hq=12) == INVALID
    assert f(ws=0) == WORKSPACE
    assert f(B=0) == OK
    L.pa_pool_destroy(pool)


def test_workspace_sizes():
    L = B.lib()
    pool = make_pool()                        # 8 KV heads, d = 64
    split = L.pa_split_tokens(64)
    assert split == 2048 and L.pa_split_tokens(128) == 1024
    assert L.pa_split_tokens(80) == 0
    pages_one_split = split // 16
    # up to 4 splits (G <= 8) are finished inside the workgroup: no workspace
    assert L.pa_decode_workspace_bytes(pool, 8, 32, 4 * pages_one_split) == 0
    n = L.pa_decode_workspace_bytes(pool, 8, 32, 4 * pages_one_split + 1)
    assert n >= 8 * 32 * 5 * (64 + 2) * 4
    # more than 8 query heads per KV head: 2 splits per workgroup
    assert L.pa_decode_workspace_bytes(pool, 8, 128, 2 * pages_one_split) == 0
    assert L.pa_decode_workspace_bytes(pool, 8, 128, 2 * pages_one_split + 1) >= 8 * 128 * 3 * 66 * 4
    assert L.pa_decode_workspace_bytes(None, 8, 32, 100) == 0
    assert L.pa_decode_workspace_bytes(pool, 0, 32, 100) == 0
    assert L.pa_decode_workspace_bytes(pool, 8, 12, 100) == 0     # 12 heads over 8 KV heads
    L.pa_pool_destroy(pool)


def test_append_validation():
    L = B.lib()
    pool = make_pool()
    f = lambda **kw: L.pa_kv_append(kw.get("pool", pool), kw.get("k", P), kw.get("v", P),
                                    kw.get("B", 4), kw.get("bt", P), kw.get("stride", 8),
                                    kw.get("pos", P), None)
    assert f(pool=None) == NULL
    assert f(k=0) == NULL
    assert f(v=0) == NULL
    assert f(bt=0) == NULL
    assert f(pos=0) == NULL
    assert f(B=-2) == INVALID
    assert f(stride=0) == INVALID
    assert f(k=MIS) == ALIGN
    assert f(pos=MIS + 2) == ALIGN
    assert f(v=MIS) == ALIGN
    assert f(B=0) == OK
    L.pa_pool_destroy(pool)


def test_profile_and_status_strings():
    L = B.lib()
    assert L.pa_profile_start() == OK
    kinds = len(B.PROFILE_KINDS)
    ms = (ctypes.c_double * kinds)()
    n = (ctypes.c_int64 * kinds)()
    assert L.pa_profile_stop(ms, n) == OK and list(n) == [0] * kinds
    assert L.pa_profile_stop(None, n) == NULL
    for s in range(9):
        assert B.status_str(s) and B.status_str(s) != "unknown status"
    assert L.pa_stream_read(P, 15, P2, None) == INVALID
    assert L.pa_stream_read(0, 16, P2, None) == NULL


# ---- launch plan (pure host code)

def expected_plan(ctx, stride, group=4, d=64, kv_heads=8):
    """The decode plan, restated: units are splits (2048 tokens at d = 64,
    1024 at d = 128); a sequence with at most ucap splits (4, or 2 when
    G > 8) is one group, a longer one a group per split, an empty context one
    zero-pair unit. A group costs its pairs plus 2 per unit. Groups by cost
    (largest first, stable) go each to the bin of least cost so far (then the
    lowest index), over min(groups, 256 / kv_heads) bins; in each bin, its
    groups in that order go to the first of the bin's items with room for
    their units, else to a new item. Bin b's first item is item b; the bins'
    other items follow, bin by bin, each named by the item before it. An item
    is 8 words: units b | s << 20 (-1 for none), the rotations (pairs before
    the unit in its item, mod W, 4 bits per unit), the index of the bin's next
    item (0: none), two zeros."""
    import heapq
    sp, w = (128, 16) if d == 64 else (64, 8)
    ucap = 4 if group <= 8 else 2
    groups = []          # (cost, [(b, s, unit pairs)])
    for b, n in enumerate(ctx):
        n = min(max(int(n), 0), stride * 16)
        pages = (n + 15) // 16
        ns = (pages + sp - 1) // sp
        units = [(b, s, (min(pages - s * sp, sp) + 1) // 2) for s in range(ns)]
        if ns == 0:
            groups.append((2, [(b, 0, 0)]))
        elif ns <= ucap:
            groups.append((sum(u[2] for u in units) + 2 * ns, units))
        else:
            groups.extend((u[2] + 2, [u]) for u in units)
    groups.sort(key=lambda g: -g[0])
    nb = min(len(groups), max(1, 256 // kv_heads))
    heap = [(0, i) for i in range(nb)]
    bins = [[] for _ in range(nb)]
    for cost, units in groups:
        c, i = heapq.heappop(heap)
        bins[i].append(units)
        heapq.heappush(heap, (c + cost, i))
    bin_items = []
    for members in bins:
        items = []
        for units in members:
            for it in items:
                if len(it) + len(units) <= ucap:
                    it.extend(units)
                    break
            else:
                items.append(list(units))
        bin_items.append(items)
    out = [None] * sum(len(x) for x in bin_items)
    extra = nb
    for b, items in enumerate(bin_items):
        idx = b
        for k, units in enumerate(items):
            nxt = 0
            if k + 1 < len(items):
                nxt, extra = extra, extra + 1
            words = [-1] * 4 + [0] * 4
            before = rot = 0
            for j, (bb, s, p) in enumerate(units):
                words[j] = bb | (s << 20)
                rot |= (before % w) << (4 * j)
                before += p
            words[4], words[5] = rot, nxt
            out[idx] = words
            idx = nxt
    return [x for words in out for x in words]


def _plan_units(plan):
    items = []
    for i in range(0, len(plan), 8):
        it = plan[i:i + 8]
        items.append(([(x & 0xFFFFF, x >> 20) for x in it[:4] if x >= 0], it[4], it[5:]))
    return items


def test_plan_matches_its_statement_and_covers_every_unit():
    import numpy as np
    L = B.lib()
    rng = np.random.default_rng(7)
    for d, hkv, hq in [(64, 8, 32), (64, 8, 128), (128, 4, 28), (64, 2, 2)]:
        h = make_pool(d=d, hkv=hkv)
        pool = type("P", (), {"handle": h})()
        g = hq // hkv
        sp = 128 if d == 64 else 64
        ucap = 4 if g <= 8 else 2
        for stride in (1, 5, 64, 65, 129, 512, 700):
            ctx = rng.integers(-3, stride * 16 + 40, 37).astype(np.int32)
            ctx[:3] = [0, stride * 16, 1]
            got = B.decode_plan(pool, ctx, hq, stride)
            assert got.tolist() == expected_plan(ctx, stride, g, d, hkv)
            cap = L.pa_decode_plan_capacity(h, len(ctx), stride)
            assert cap == len(ctx) * -(-stride // sp) * 8 and len(got) <= cap
            # every unit exactly once; short sequences whole and in split order
            seen = {}
            items = _plan_units(got.tolist())
            for units, rot, tail in items:
                assert 1 <= len(units) <= ucap and list(tail[1:]) == [0, 0]
                for k, (b, s) in enumerate(units):
                    assert (b, s) not in seen
                    seen[(b, s)] = (units, k)
            # the chains from the bins' first items reach every item once,
            # each step forward and past the first items
            nb = min(len(items), 256 // hkv)
            reached = []
            for b in range(nb):
                i = b
                while True:
                    reached.append(i)
                    nxt = items[i][2][0]
                    if nxt == 0:
                        break
                    assert i < nxt < len(items) and nxt >= nb
                    i = nxt
            assert sorted(reached) == list(range(len(items)))
            for b, n in enumerate(ctx):
                n = min(max(int(n), 0), stride * 16)
                ns = -(-((n + 15) // 16) // sp)
                want = [(b, s) for s in range(max(ns, 1))]
                assert sorted(k for k in seen if k[0] == b) == want
                if 1 < ns <= ucap:
                    units, k = seen[(b, 0)]
                    assert units[k:k + ns] == want
        L.pa_pool_destroy(h)


def test_plan_one_round_pairs_large_with_small():
    """64 sequences of U[256, 2048] tokens over 8 KV heads (one split each):
    32 items, one per CU of a device round, each the k-th largest sequence
    with the k-th smallest."""
    import numpy as np
    h = make_pool(d=64)
    pool = type("P", (), {"handle": h})()
    ctx = np.random.default_rng(1003).integers(256, 2049, 64).astype(np.int32)
    items = _plan_units(B.decode_plan(pool, ctx, 32, 128).tolist())
    assert len(items) == 32
    pages = -(-ctx // 16)
    order = sorted(range(64), key=lambda b: -((pages[b] + 1) // 2))
    pairs = sorted(((units[0][0], units[1][0]) for units, _, _ in items), key=lambda t: order.index(t[0]))
    assert [p[0] for p in pairs] == order[:32]
    loads = [((pages[a] + 1) // 2 + (pages[b] + 1) // 2) for a, b in pairs]
    assert max(loads) - min(loads) <= 8
    B.lib().pa_pool_destroy(h)


def test_plan_validation():
    import numpy as np
    L = B.lib()
    h = make_pool(d=128, hkv=4)
    n = ctypes.c_int32(-1)
    ctx = np.array([100, 5000, 0], dtype=np.int32)
    buf = np.zeros(64, dtype=np.int32)
    assert L.pa_decode_plan_capacity(None, 3, 10) == -1
    assert L.pa_decode_plan_capacity(h, 3, 0) == -1
    assert L.pa_decode_plan_capacity(h, (1 << 20) + 1, 10) == -1
    assert L.pa_decode_plan_capacity(h, 1, 64 * 2048 + 1) == -1
    assert L.pa_decode_plan(h, ctx.ctypes.data, 3, 28, 400, buf.ctypes.data, 64, None) == NULL
    assert L.pa_decode_plan(h, None, 3, 28, 400, buf.ctypes.data, 64, ctypes.byref(n)) == NULL
    assert L.pa_decode_plan(h, ctx.ctypes.data, 3, 28, 400, None, 64, ctypes.byref(n)) == NULL
    assert L.pa_decode_plan(h, ctx.ctypes.data, 3, 30, 400, buf.ctypes.data, 64, ctypes.byref(n)) == INVALID
    assert L.pa_decode_plan(h, ctx.ctypes.data, 3, 4 * 17, 400, buf.ctypes.data, 64, ctypes.byref(n)) == UNSUPPORTED
    # 5000 tokens = 5 splits of 1024 (more than 4: one group each), 100 tokens
    # and the empty context one each: 7 units over 64 bins -> 7 items, 56 words
    assert L.pa_decode_plan(h, ctx.ctypes.data, 3, 28, 400, buf.ctypes.data, 55, ctypes.byref(n)) == INVALID
    assert L.pa_decode_plan(h, ctx.ctypes.data, 3, 28, 400, buf.ctypes.data, 56, ctypes.byref(n)) == OK
    assert n.value == 56
    assert buf[:56].tolist() == expected_plan(ctx, 400, 7, 128, 4)
    assert L.pa_decode_plan(h, ctx.ctypes.data, 0, 28, 400, None, 0, ctypes.byref(n)) == OK and n.value == 0
    L.pa_pool_destroy(h)


def test_static_decode_validation():
    """pa_decode_static checks its arguments and its scratch limit before it
    touches a device: nothing here reaches the HIP runtime."""
    L = B.lib()
    h = make_pool(d=64)
    f = L.pa_decode_static
    assert f(None, P, 2, 32, P, 600, P, 0.125, P2, None) == NULL
    assert f(h, P, -1, 32, P, 600, P, 0.125, P2, None) == INVALID
    assert f(h, P, 2, 30, P, 600, P, 0.125, P2, None) == INVALID
    assert f(h, P, 2, 32, P, 0, P, 0.125, P2, None) == INVALID
    assert f(h, P, 0, 32, P, 600, P, 0.125, P2, None) == OK
    # 600 sequences x 32 heads x 40 splits x (64 + 2) floats: past 32 MiB
    assert L.pa_decode_workspace_bytes(h, 600, 32, 40 * 128) > 32 << 20
    assert f(h, P, 600, 32, P, 40 * 128, P, 0.125, P2, None) == WORKSPACE
    L.pa_pool_destroy(h)


def test_planned_decode_validation():
    L = B.lib()
    h = make_pool(d=64)
    ws = 1 << 24

    def call(plan=P, words=8, num_seqs=2, stride=600, ws_ptr=P, ws_bytes=ws):
        return L.pa_decode_planned(h, P, num_seqs, 32, P, stride, P, 0.125, P2, ws_ptr, ws_bytes, plan,
                                   words, None)

    assert call(plan=None) == NULL
    assert call(plan=P + 2) == ALIGN
    assert call(words=-8) == INVALID
    assert call(words=12) == INVALID         # not whole items of 8 words
    assert call(words=2 * 5 * 8 + 8) == INVALID   # 2 sequences x 5 splits at most
    assert call(ws_ptr=None, ws_bytes=0) == WORKSPACE   # 600 pages: 5 splits, more than 4
    assert call(num_seqs=0, plan=None, words=0) == OK

    def host(plan=P, words=8, num_seqs=300, stride=600):
        return L.pa_decode_planned_host(h, P, num_seqs, 32, P, stride, P, 0.125, P2, P, ws, plan, words, None)

    assert host(plan=None) == NULL
    assert host(words=12) == INVALID
    assert host(words=2048 + 8) == INVALID    # more than the kernel arguments carry
    assert host(words=-8) == INVALID
    assert host(num_seqs=0, plan=None, words=0) == OK
    L.pa_pool_destroy(h)


def test_prefill_and_write_validation():
    L = B.lib()
    h = make_pool(d=64)

    def pre(q=P, kr=P, vr=P, num_seqs=2, hq=32, rows=10, max_chunk=8, qs=P, bt=P, stride=4, ctx=P,
            scale=0.125, out=P2):
        return L.pa_prefill(h, q, kr, vr, num_seqs, hq, rows, max_chunk, qs, bt, stride, ctx, scale, out,
                            None)

    assert pre(q=None) == NULL
    assert pre(out=None) == NULL
    assert pre(qs=None) == NULL
    assert pre(q=MIS) == ALIGN
    assert pre(qs=P + 2) == ALIGN
    assert pre(hq=12) == INVALID              # not a multiple of 8 KV heads
    assert pre(hq=8 * 17) == UNSUPPORTED      # 17 query heads per KV head
    assert pre(rows=-1) == INVALID
    assert pre(max_chunk=-1) == INVALID
    assert pre(stride=0) == INVALID
    assert pre(scale=float("nan")) == INVALID
    assert pre(num_seqs=0, q=None, qs=None) == OK
    assert pre(max_chunk=0, q=None) == OK
    assert L.pa_prefill(None, P, P, P, 1, 32, 1, 1, P, P, 1, P, 0.1, P2, None) == NULL
    assert L.pa_kv_write(h, None, P, 1, 4, 4, P, P, 2, P, None) == NULL
    assert L.pa_kv_write(h, MIS, P, 1, 4, 4, P, P, 2, P, None) == ALIGN
    assert L.pa_kv_write(h, P, P, 1, 4, 4, P, P, 0, P, None) == INVALID
    assert L.pa_kv_write(h, None, None, 0, 4, 4, None, None, 2, None, None) == OK
    L.pa_pool_destroy(h)


def expected_prefill_plan(ctx, chunks, hq, hkv, stride, max_chunk, d=64):
    """Every row block of 128 query rows that holds rows, costed by the page
    pairs its last row can see, largest first (ties: the later row block, then
    the sequence); when the grid fits the device at once (items x kv heads <=
    256 CUs x prefill workgroups per CU: 4 at d = 64, 2 at d = 128), every
    other tier of 32 x 8 / kv_heads items is reversed."""
    g = hq // hkv
    block_rows = 128
    row_blocks = (max_chunk * g + block_rows - 1) // block_rows
    items = []
    for rb in range(row_blocks - 1, -1, -1):
        for b in range(len(ctx)):
            c = min(max(int(ctx[b]), 0), stride * 16)
            n = min(max(int(chunks[b]), 0), max_chunk, stride * 16 - c)
            rows = n * g
            if rb * block_rows >= rows:
                continue
            last = c + min(rb * block_rows + block_rows - 1, rows - 1) // g
            pages = (last + 16) // 16
            items.append(((pages + 1) // 2, b | (rb << 20)))
    items.sort(key=lambda t: -t[0])          # stable: keeps the visiting order among ties
    out = [code for _, code in items]
    tier = 32 * (8 // hkv)
    if len(out) * hkv <= 256 * (4 if d == 64 else 2):
        for t0 in range(tier, len(out), 2 * tier):
            out[t0:t0 + tier] = out[t0:t0 + tier][::-1]
    return out


@pytest.mark.parametrize("d,hq,hkv", [(64, 32, 8), (64, 8, 2), (128, 28, 4)])
def test_prefill_plan_matches_its_definition(d, hq, hkv):
    import numpy as np
    L = B.lib()
    h = make_pool(hkv=hkv, d=d)
    pool = type("P", (), {"handle": h})()
    rng = np.random.default_rng(11 + d + hkv)
    for n_seq, max_chunk, stride in ((8, 512, 300), (3, 40, 10), (20, 2048, 200), (1, 4096, 300)):
        ctx = rng.integers(-2, stride * 16 + 30, n_seq).astype(np.int32)
        chunks = rng.integers(-1, max_chunk + 20, n_seq).astype(np.int32)
        ctx[0], chunks[0] = 0, max_chunk                 # a fresh prompt at the bound
        got = B.prefill_plan(pool, ctx, chunks, hq, stride, max_chunk)
        assert got.tolist() == expected_prefill_plan(ctx, chunks, hq, hkv, stride, max_chunk, d)
        cap = L.pa_prefill_plan_capacity(h, n_seq, hq, max_chunk)
        assert cap == n_seq * ((max_chunk * (hq // hkv) + 127) // 128)
        # every item once: (sequence, row block) pairs are distinct
        assert len(set(got.tolist())) == len(got) <= cap
    L.pa_pool_destroy(h)


def test_prefill_plan_reverses_tiers_only_for_one_round_grids():
    import numpy as np
    h = make_pool(d=64)                       # 8 KV heads, 4 prefill workgroups per CU: 1024 resident
    pool = type("P", (), {"handle": h})()
    ctx = np.array([1457, 685, 1980, 3331, 2261, 890, 373, 4030], np.int32)
    one = B.prefill_plan(pool, ctx, np.full(8, 512, np.int32), 32, 300, 512)   # 128 items x 8 = 1024
    assert len(one) == 128
    plain = expected_prefill_plan(ctx, [512] * 8, 32, 8, 300, 512)
    assert one.tolist() == plain
    costs = {}
    for b in range(8):
        for rb in range(16):
            last = int(ctx[b]) + min(rb * 128 + 127, 2047) // 4
            costs[b | (rb << 20)] = ((last + 16) // 16 + 1) // 2
    c = [costs[x] for x in one.tolist()]
    assert c[:32] == sorted(c[:32], reverse=True) and c[32:64] == sorted(c[32:64])
    assert c[64:96] == sorted(c[64:96], reverse=True) and c[96:] == sorted(c[96:])
    # 256 items x 8 = 2048 workgroups: two rounds, so plain largest-first order
    many = B.prefill_plan(pool, ctx, np.full(8, 1024, np.int32), 32, 400, 1024)
    last_pos = lambda x: int(ctx[x & 0xFFFFF]) + min((x >> 20) * 128 + 127, 4095) // 4
    pairs = [((last_pos(x) + 16) // 16 + 1) // 2 for x in many.tolist()]
    assert len(many) == 256 and pairs == sorted(pairs, reverse=True)
    B.lib().pa_pool_destroy(h)


def test_prefill_plan_and_planned_validation():
    import numpy as np
    L = B.lib()
    h = make_pool(d=64)
    n = ctypes.c_int32(-1)
    ctx = np.array([100, 5000, 0], dtype=np.int32)
    chunks = np.array([64, 0, 300], dtype=np.int32)
    buf = np.zeros(16, dtype=np.int32)
    assert L.pa_prefill_plan_capacity(None, 3, 32, 300) == -1
    assert L.pa_prefill_plan_capacity(h, 3, 12, 300) == -1           # not a multiple of 8 KV heads
    assert L.pa_prefill_plan_capacity(h, 3, 8 * 17, 300) == -1       # 17 query heads per KV head
    assert L.pa_prefill_plan_capacity(h, (1 << 20) + 1, 32, 1) == -1
    assert L.pa_prefill_plan_capacity(h, 1, 32, 32 * 2048 + 1) == -1  # more than 2^11 row blocks
    assert L.pa_prefill_plan_capacity(h, 3, 32, 300) == 3 * 10
    args = lambda cap, out=buf.ctypes.data, nptr=ctypes.byref(n), c=ctx.ctypes.data, k=chunks.ctypes.data: \
        L.pa_prefill_plan(h, c, k, 3, 32, 400, 300, out, cap, nptr)
    assert args(16, nptr=None) == NULL
    assert args(16, c=None) == NULL
    assert args(16, k=None) == NULL
    assert args(16, out=None) == NULL
    # rows: 64 x 4 = 256 (2 blocks), 0, 300 x 4 = 1200 (10 blocks): 12 items
    assert args(11) == INVALID
    assert args(16) == OK and n.value == 12
    assert L.pa_prefill_plan(h, None, None, 0, 32, 400, 300, None, 0, ctypes.byref(n)) == OK and n.value == 0
    assert L.pa_prefill_plan(h, ctx.ctypes.data, chunks.ctypes.data, 3, 32, 0, 300, buf.ctypes.data, 16,
                             ctypes.byref(n)) == INVALID

    def pre(plan=P, items=4, num_seqs=2, max_chunk=8):
        return L.pa_prefill_planned(h, P, P, P, num_seqs, 32, 10, max_chunk, P, P, 4, P, 0.125, P2, plan,
                                    items, None)

    assert pre(plan=None) == NULL
    assert pre(plan=P + 2) == ALIGN
    assert pre(items=-1) == INVALID
    assert pre(items=2 * 1 + 1) == INVALID     # 2 sequences x 1 row block of 8 x 4 rows
    assert pre(num_seqs=0, plan=None, items=0) == OK
    assert L.pa_prefill_planned(None, P, P, P, 1, 32, 1, 1, P, P, 1, P, 0.1, P2, P, 1, None) == NULL
    L.pa_pool_destroy(h)
