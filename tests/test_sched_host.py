"""The host page allocator and admission policy (pakv_sched.h) against a plain
Python model of the policy the pages state ("Curso gratuito recorre la
inferencia de LLM ..." (news-factory.app), section "¿Cómo administra el motor
la memoria de la caché KV?"): budget reserved whole at admission, first in
first out, oversize requests rejected, static vs continuous batching, pages
freed on finish; shared-prefix pages referenced, not copied.

The model decides admissions from page counts alone, so admissions and free
page counts must match it exactly; the physical page ids the library picks are
free to differ and are checked for validity instead (a consistent bijection
between the model's live pages and the library's, no page in two requests
unless shared)."""

import ctypes

import numpy as np
import pytest

from paged_kv_decode_02_amd import binding as B

PAGE = 16


def pages_for(tokens):
    return -(-tokens // PAGE)


class Model:
    """Pages are abstract labels; a label lives while something references it."""

    def __init__(self, num_pages, layers, max_batch, stride, static):
        self.P, self.L, self.max_batch, self.stride, self.static = num_pages, layers, max_batch, stride, static
        self.refs = {}            # label -> references
        self.next_label = 0
        self.queue = []           # ids in arrival order
        self.req = {}             # id -> dict
        self.slots = [None] * max_batch

    def free(self):
        return self.P - len(self.refs)

    def _ref(self, lab):
        self.refs[lab] = self.refs.get(lab, 0) + 1

    def _unref(self, lab):
        self.refs[lab] -= 1
        if self.refs[lab] == 0:
            del self.refs[lab]

    def submit(self, rid, prompt, new, parent=None, shared_tokens=0):
        pages = pages_for(prompt + new)
        sp = shared_tokens // PAGE if parent is not None else 0
        if pages > self.stride or self.L * (pages - sp) > self.P:
            return "capacity"
        shared = [[self.req[parent]["rows"][l][j] for j in range(sp)] for l in range(self.L)] if sp else []
        for row in shared:
            for lab in row:
                self._ref(lab)
        self.req[rid] = dict(prompt=prompt, new=new, pages=pages, sp=sp, shared=shared, state="queued",
                             slot=-1, ctx=0, rows=None)
        self.queue.append(rid)
        return "ok"

    def admit(self):
        out = []
        if self.static and any(s is not None for s in self.slots):
            return out
        while self.queue:
            r = self.req[self.queue[0]]
            need = self.L * (r["pages"] - r["sp"])
            if need > self.free() or all(s is not None for s in self.slots):
                break
            rid = self.queue.pop(0)
            slot = self.slots.index(None)
            self.slots[slot] = rid
            rows = []
            for l in range(self.L):
                row = list(r["shared"][l]) if r["sp"] else []
                for _ in range(r["pages"] - r["sp"]):
                    lab = self.next_label
                    self.next_label += 1
                    self._ref(lab)
                    row.append(lab)
                rows.append(row)
            r.update(state="running", slot=slot, ctx=r["sp"] * PAGE, rows=rows, shared=[])
            out.append(rid)
        return out

    def finish(self, rid):
        r = self.req.pop(rid)
        if r["state"] == "queued":
            self.queue.remove(rid)
            for row in r["shared"]:
                for lab in row:
                    self._unref(lab)
        else:
            for row in r["rows"]:
                for lab in row:
                    self._unref(lab)
            self.slots[r["slot"]] = None


def check_consistent(s, m):
    st = s.stats()
    assert st["free_pages"] == m.free()
    assert st["queued"] == len(m.queue)
    assert st["running"] == sum(x is not None for x in m.slots)
    bt, ctx = s.block_tables, s.context_lens
    lab2page, page2lab = {}, {}
    for slot, rid in enumerate(m.slots):
        if rid is None:
            assert (bt[:, slot, :] == -1).all() and ctx[slot] == 0
            continue
        r = m.req[rid]
        assert s.slot(rid) == slot and ctx[slot] == r["ctx"]
        for l in range(m.L):
            row = bt[l, slot]
            assert (row[r["pages"]:] == -1).all()
            for j, lab in enumerate(r["rows"][l]):
                p = int(row[j])
                assert 0 <= p < m.P
                assert lab2page.setdefault(lab, p) == p, "one model page maps to two library pages"
                assert page2lab.setdefault(p, lab) == lab, "one library page holds two model pages"
    for rid in m.queue:
        assert s.slot(rid) == -1


@pytest.mark.parametrize("static", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_operations_match_the_model(static, seed):
    rng = np.random.default_rng(100 + seed)
    P, L, MB, STRIDE = 60, 2, 4, 8
    mode = B.PA_BATCH_STATIC if static else B.PA_BATCH_CONTINUOUS
    s = B.Scheduler(P, L, MB, STRIDE, mode)
    m = Model(P, L, MB, STRIDE, static)
    live = []
    for _ in range(600):
        op = rng.choice(["submit", "shared", "admit", "advance", "finish"], p=[0.3, 0.1, 0.25, 0.2, 0.15])
        if op == "submit":
            prompt, new = int(rng.integers(0, 120)), int(rng.integers(0, 40))
            if prompt + new == 0:
                continue
            try:
                rid = s.submit(prompt, new)
                res = "ok"
            except B.PakvError as e:
                assert e.status == B.PA_ERR_CAPACITY
                res, rid = "capacity", None
            assert res == m.submit(rid if rid else -1, prompt, new)
            if rid:
                live.append(rid)
        elif op == "shared":
            running = [r for r in live if m.req[r]["state"] == "running"]
            if not running:
                continue
            parent = int(rng.choice(running))
            sh = int(rng.integers(0, m.req[parent]["ctx"] + 1))
            prompt, new = sh + int(rng.integers(0, 40)), int(rng.integers(1, 30))
            try:
                rid = s.submit_shared(parent, sh, prompt, new)
                res = "ok"
            except B.PakvError as e:
                assert e.status == B.PA_ERR_CAPACITY
                res, rid = "capacity", None
            assert res == m.submit(rid if rid else -1, prompt, new, parent, sh)
            if rid:
                live.append(rid)
        elif op == "admit":
            assert s.admit() == m.admit()
        elif op == "advance":
            running = [r for r in live if m.req[r]["state"] == "running"]
            if not running:
                continue
            rid = int(rng.choice(running))
            r = m.req[rid]
            room = r["prompt"] + r["new"] - r["ctx"]
            n = int(rng.integers(0, room + 3))
            if n > room:
                with pytest.raises(B.PakvError) as ei:
                    s.advance(rid, n)
                assert ei.value.status == B.PA_ERR_INVALID
            else:
                s.advance(rid, n)
                r["ctx"] += n
        elif op == "finish" and live:
            rid = int(live.pop(int(rng.integers(len(live)))))
            s.finish(rid)
            m.finish(rid)
        check_consistent(s, m)
    for rid in live:
        s.finish(rid)
        m.finish(rid)
    check_consistent(s, m)
    assert s.stats() == {"free_pages": P, "queued": 0, "running": 0}


def test_first_in_first_out_blocks_later_requests():
    s = B.Scheduler(10, 1, 8, 16)
    a = s.submit(8 * PAGE, 0)        # 8 pages
    b = s.submit(4 * PAGE - 3, 3)    # 4 pages
    c = s.submit(1, 0)               # 1 page: fits, but must not overtake b
    assert s.admit() == [a]
    assert s.admit() == []
    assert s.slot(b) == -1 and s.slot(c) == -1
    s.finish(a)
    assert s.admit() == [b, c]
    assert s.stats() == {"free_pages": 5, "queued": 0, "running": 2}


def test_static_batching_waits_for_the_whole_group():
    s = B.Scheduler(100, 2, 8, 16, B.PA_BATCH_STATIC)
    a, b, c = s.submit(16, 16), s.submit(40, 8), s.submit(5, 5)
    assert s.admit() == [a, b, c]
    d = s.submit(1, 1)
    s.finish(a)
    s.finish(b)
    assert s.admit() == []            # c still runs
    s.finish(c)
    assert s.admit() == [d]


def test_batch_slots_limit_admission():
    s = B.Scheduler(100, 1, 2, 16)
    ids = [s.submit(10, 10) for _ in range(3)]
    assert s.admit() == ids[:2]
    assert s.admit() == []
    s.finish(ids[0])
    assert s.admit() == [ids[2]]
    assert s.slot(ids[2]) == 0        # the lowest empty slot


def test_oversize_requests_are_rejected():
    s = B.Scheduler(20, 4, 4, 16)
    with pytest.raises(B.PakvError) as ei:
        s.submit(5 * PAGE + 1, 0)      # 6 pages x 4 layers = 24 > 20
    assert ei.value.status == B.PA_ERR_CAPACITY
    with pytest.raises(B.PakvError) as ei:
        B.Scheduler(1000, 1, 4, 16).submit(16 * PAGE, 1)   # 17 pages > a row of 16
    assert ei.value.status == B.PA_ERR_CAPACITY
    rid = s.submit(5 * PAGE, 0)        # exactly the pool
    assert s.admit() == [rid] and s.stats()["free_pages"] == 0


def test_block_tables_rows_and_context():
    s = B.Scheduler(64, 3, 4, 8)
    a = s.submit(20, 30)              # 50 tokens -> 4 pages per layer
    b = s.submit(1, 0)
    assert s.admit() == [a, b]
    bt = s.block_tables
    sa, sb = s.slot(a), s.slot(b)
    assert (bt[:, sa, :4] >= 0).all() and (bt[:, sa, 4:] == -1).all()
    assert (bt[:, sb, :1] >= 0).all() and (bt[:, sb, 1:] == -1).all()
    used = np.concatenate([bt[:, sa, :4].ravel(), bt[:, sb, :1].ravel()])
    assert len(set(used.tolist())) == used.size == 15
    assert s.context_lens[sa] == 0
    s.advance(a, 20)
    assert s.context_lens[sa] == 20
    s.advance(a, 30)
    with pytest.raises(B.PakvError):
        s.advance(a, 1)               # past prompt + max_new
    s.finish(a)
    assert (bt[:, sa, :] == -1).all() and s.context_lens[sa] == 0


def test_shared_prefix_pages_outlive_the_parent():
    s = B.Scheduler(40, 2, 4, 8)
    parent = s.submit(40, 8)           # 3 pages per layer
    assert s.admit() == [parent]
    s.advance(parent, 40)
    child = s.submit_shared(parent, 35, 50, 10)    # shares 2 full pages per layer
    assert s.stats()["free_pages"] == 40 - 6
    assert s.admit() == [child]
    bt, sp, sc = s.block_tables, s.slot(parent), s.slot(child)
    assert (bt[:, sc, :2] == bt[:, sp, :2]).all()
    assert not set(bt[:, sc, 2:4].ravel()) & set(bt[:, sp, :3].ravel())
    assert s.context_lens[sc] == 32                 # the shared full pages are in the cache
    assert s.stats()["free_pages"] == 40 - 6 - 2 * 2
    s.finish(parent)
    assert s.stats()["free_pages"] == 40 - 2 * 4    # the child's 4 pages per layer stay
    s.finish(child)
    assert s.stats()["free_pages"] == 40


def test_state_errors():
    L = B.lib()
    s = B.Scheduler(16, 1, 2, 4)
    q = s.submit(10, 1)
    with pytest.raises(B.PakvError) as ei:
        s.advance(q, 1)                # still queued
    assert ei.value.status == B.PA_ERR_STATE
    with pytest.raises(B.PakvError) as ei:
        s.submit_shared(q, 0, 5, 1)    # parent not running
    assert ei.value.status == B.PA_ERR_STATE
    s.finish(q)                        # cancel a queued request
    with pytest.raises(B.PakvError) as ei:
        s.finish(q)
    assert ei.value.status == B.PA_ERR_INVALID
    h = ctypes.c_void_p()
    assert L.pa_sched_create(ctypes.byref(h), 0, 1, 1, 1, 0) == B.PA_ERR_INVALID
    assert L.pa_sched_create(ctypes.byref(h), 4, 1, 1, 1, 7) == B.PA_ERR_INVALID
    assert L.pa_sched_create(None, 4, 1, 1, 1, 0) == 1
    with pytest.raises(B.PakvError):
        s.submit(0, 0)
