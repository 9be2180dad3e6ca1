"""Seeded synthetic workloads for paged decode attention.

This module draws the inputs and nothing else: context lengths, the placement
of every sequence's pages in the shared pool, and BF16 values for queries,
cached keys/values and new-token keys/values. It holds no attention arithmetic.
The oracle and the HIP library both consume what it produces, and neither is
imported here.

Values come from a counter-based generator, so the same element can be made
on the host (numpy) or on the GPU (torch) with identical bits, and any page of
a pool too large for the host can be regenerated there on its own:

* ``h = mix(lo32(i) ^ mix(hi32(i) ^ key(seed, stream)))`` for flat element
  index ``i``, where ``mix`` is the 32-bit "lowbias32" integer hash from
  C. Wellons, "Prospecting for Hash Functions" (2018);
* the BF16 value is ``table[h >> 16]``, a 65536-entry table of the normal
  quantiles ``sigma * Phi^-1((j + 0.5) / 65536)`` rounded to BF16 (nearest
  even). Drawing a uniform 16-bit index and reading the quantile table is
  inverse-transform sampling of N(0, sigma^2), discretised to 2^16 levels.

Pool layout (shared with the library's header): K is
``[num_pages][Hkv][d/32][16][32]`` (head dims in slabs of 32, each slab
holding all 16 slots), V is ``[num_pages][Hkv][d][16]``, BF16.
Slots that hold no token (tails of last pages, pages nobody references, and in
append workloads the slot the new token will fill) are set to BF16 NaN
(0x7FC0), so that reading them by mistake shows up in the output.

The five named workloads follow the configurations the project is measured
on (seeds 1001..1005); ``custom`` builds small ones for tests.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

PAGE = 16
K_SLAB = 32          # head dims per K slab: K pool [page][kv_head][d/32][16][32]
NAN_BITS = 0x7FC0
MASK32 = 0xFFFFFFFF

STREAM_K_POOL = 1
STREAM_V_POOL = 2
STREAM_Q = 3
STREAM_K_NEW = 4
STREAM_V_NEW = 5

_C1 = 0x7FEB352D
_C2 = 0x846CA68B


# ------------------------------------------------------------ hash generator
def _mul32(x, c: int):
    """(x * c) mod 2^32 for x in [0, 2^32) held in int64, without overflow:
    the 16-bit halves of x times a 32-bit constant stay below 2^48."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & MASK32


def _mix32(x):
    x = x ^ (x >> 16)
    x = _mul32(x, _C1)
    x = x ^ (x >> 15)
    x = _mul32(x, _C2)
    return x ^ (x >> 16)


def _mix32_int(x: int) -> int:
    x &= MASK32
    x ^= x >> 16
    x = (x * _C1) & MASK32
    x ^= x >> 15
    x = (x * _C2) & MASK32
    return x ^ (x >> 16)


def stream_key(seed: int, stream: int) -> int:
    return _mix32_int(seed * 0x9E3779B1 + stream * 0x85EBCA77 + 0x165667B1)


def hash32(seed: int, stream: int, idx):
    """32-bit hash of flat indices ``idx`` (int64 numpy array or torch tensor)."""
    key = stream_key(seed, stream)
    inner = _mix32((idx >> 32) ^ key)
    return _mix32((idx & MASK32) ^ inner)


def normal_table_bits(sigma: float) -> np.ndarray:
    """BF16 bits of sigma * Phi^-1((j + 0.5) / 2^16), j = 0..65535."""
    from scipy.special import ndtri
    p = (np.arange(1 << 16, dtype=np.float64) + 0.5) / float(1 << 16)
    vals = (ndtri(p) * float(sigma)).astype(np.float32)
    u = vals.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _mix32_u32(x: np.ndarray) -> np.ndarray:
    """_mix32 on a uint32 numpy array, in place: uint32 products wrap modulo
    2^32 by themselves, which is the arithmetic the hash is defined with."""
    x ^= x >> np.uint32(16)
    x *= np.uint32(_C1)
    x ^= x >> np.uint32(15)
    x *= np.uint32(_C2)
    x ^= x >> np.uint32(16)
    return x


def hash32_np(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """hash32 of non-negative int64 indices with uint32 numpy arithmetic (the
    same function; faster on the host than the int64 form torch needs)."""
    idx = np.asarray(idx, dtype=np.int64)
    key = np.uint32(stream_key(seed, stream))
    inner = _mix32_u32((idx >> 32).astype(np.uint32) ^ key)
    lo = idx.astype(np.uint32)
    lo ^= inner
    return _mix32_u32(lo)


def values_np(seed: int, stream: int, idx: np.ndarray, table: np.ndarray) -> np.ndarray:
    h = hash32_np(seed, stream, idx)
    return table[h >> np.uint32(16)]


# ------------------------------------------------------------------ workload
@dataclass
class Workload:
    name: str
    seed: int
    num_layers: int
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    sigma: float
    ctx_lens: np.ndarray            # int32 [B], tokens attended (incl. the new one when appending)
    block_tables: np.ndarray        # int32 [L][B][stride]
    num_pages: int
    page_valid: np.ndarray          # int32 [num_pages], valid slot prefix before any append
    append: bool                    # new token written at ctx_len - 1 before decoding
    pool_note: str = ""
    _table: Optional[np.ndarray] = field(default=None, repr=False)

    # -- shapes and counts
    @property
    def stride(self) -> int:
        return int(self.block_tables.shape[2])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> np.float32:
        return np.float32(1.0 / math.sqrt(self.head_dim))

    @property
    def page_elems(self) -> int:
        return self.num_kv_heads * PAGE * self.head_dim

    @property
    def positions(self) -> Optional[np.ndarray]:
        if not self.append:
            return None
        return (self.ctx_lens.astype(np.int64) - 1).astype(np.int32)

    def kv_bytes_per_layer(self) -> int:
        """Algorithmic K+V bytes one decode pass reads: every cached token once."""
        return int(self.ctx_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * 2

    def kv_bytes_per_step(self) -> int:
        return self.kv_bytes_per_layer() * self.num_layers

    def pool_bytes(self) -> int:
        return 2 * self.num_pages * self.page_elems * 2

    def table(self) -> np.ndarray:
        if self._table is None:
            self._table = normal_table_bits(self.sigma)
        return self._table

    # -- small per-sequence arrays (host)
    def q_bits(self) -> np.ndarray:
        n = self.num_layers * self.num_seqs * self.num_q_heads * self.head_dim
        v = values_np(self.seed, STREAM_Q, np.arange(n, dtype=np.int64), self.table())
        return v.reshape(self.num_layers, self.num_seqs, self.num_q_heads, self.head_dim)

    def new_kv_bits(self, which: str) -> np.ndarray:
        stream = STREAM_K_NEW if which == "k" else STREAM_V_NEW
        n = self.num_layers * self.num_seqs * self.num_kv_heads * self.head_dim
        v = values_np(self.seed, stream, np.arange(n, dtype=np.int64), self.table())
        return v.reshape(self.num_layers, self.num_seqs, self.num_kv_heads, self.head_dim)

    # -- pool contents
    def _slot_of(self, which: str, elem_in_page):
        if which == "k":        # [Hkv][d/32][16][32]
            return (elem_in_page // K_SLAB) % PAGE
        return elem_in_page % PAGE  # [Hkv][d][16]

    def _pool_shape(self, which: str, pages: int):
        if which == "k":
            return (pages, self.num_kv_heads, self.head_dim // K_SLAB, PAGE, K_SLAB)
        return (pages, self.num_kv_heads, self.head_dim, PAGE)

    def pool_pages_bits(self, which: str, page_ids) -> np.ndarray:
        """Host copy of the listed physical pages, shaped like the pool."""
        page_ids = np.asarray(page_ids, dtype=np.int64).reshape(-1)
        e = self.page_elems
        stream = STREAM_K_POOL if which == "k" else STREAM_V_POOL
        local = np.arange(e, dtype=np.int64)
        out = np.empty((page_ids.size, e), dtype=np.uint16)
        slot = self._slot_of(which, local)
        for i0 in range(0, page_ids.size, 256):
            ids = page_ids[i0:i0 + 256]
            idx = ids[:, None] * e + local[None, :]
            v = values_np(self.seed, stream, idx, self.table())
            poison = slot[None, :] >= self.page_valid[ids][:, None]
            out[i0:i0 + ids.size] = np.where(poison, np.uint16(NAN_BITS), v)
        return out.reshape(self._pool_shape(which, page_ids.size))

    def pool_bits(self, which: str) -> np.ndarray:
        return self.pool_pages_bits(which, np.arange(self.num_pages))

    def pool_device(self, which: str, device, chunk_elems: int = 1 << 26):
        """The whole pool made on ``device`` with torch integer ops, bit-identical
        to ``pool_bits``. Returns an int16 tensor shaped like the pool."""
        import torch
        e = self.page_elems
        total = self.num_pages * e
        stream = STREAM_K_POOL if which == "k" else STREAM_V_POOL
        table = torch.from_numpy(self.table().view(np.int16)).to(device)
        valid = torch.from_numpy(self.page_valid.astype(np.int64)).to(device)
        pool = torch.empty(total, dtype=torch.int16, device=device)
        nan = torch.tensor(NAN_BITS, dtype=torch.int16, device=device)
        for start in range(0, total, chunk_elems):
            end = min(total, start + chunk_elems)
            idx = torch.arange(start, end, dtype=torch.int64, device=device)
            h = hash32(self.seed, stream, idx)
            v = table[h >> 16]
            local = idx % e
            slot = self._slot_of(which, local)
            poison = slot >= valid[idx // e]
            pool[start:end] = torch.where(poison, nan, v)
            del idx, h, v, local, slot, poison
        return pool.view(self._pool_shape(which, self.num_pages))

    def sequence_pages(self, layer: int, b: int) -> np.ndarray:
        n = int(self.ctx_lens[b])
        return self.block_tables[layer, b, :-(-n // PAGE)] if n > 0 else self.block_tables[layer, b, :0]


# --------------------------------------------------------------- construction
def _deal_pages(rng, need: np.ndarray, num_pages: int, stride: int,
                interleave: bool, filler: Optional[int] = None):
    """Assign physical pages from a shuffled free list.

    ``need`` is ``[L][B]`` pages per (layer, sequence). With ``interleave`` the
    free list is dealt round-robin over all (layer, sequence) units by logical
    page index; otherwise sequence by sequence. Unused table entries get
    ``filler`` (an unreferenced page) so they never point outside the pool.
    """
    num_layers, num_seqs = need.shape
    total = int(need.sum())
    assert total <= num_pages, "pool too small for the demand"
    order = rng.permutation(num_pages).astype(np.int32)
    used = order[:total]
    if filler is None:
        filler = int(order[total]) if total < num_pages else int(order[0])
    bt = np.full((num_layers, num_seqs, stride), filler, dtype=np.int32)
    if interleave:
        nxt = 0
        flat_need = need.reshape(-1)
        flat_bt = bt.reshape(num_layers * num_seqs, stride)
        for j in range(int(flat_need.max()) if flat_need.size else 0):
            sel = np.nonzero(flat_need > j)[0]
            flat_bt[sel, j] = used[nxt:nxt + sel.size]
            nxt += sel.size
    else:
        nxt = 0
        for layer in range(num_layers):
            for b in range(num_seqs):
                k = int(need[layer, b])
                bt[layer, b, :k] = used[nxt:nxt + k]
                nxt += k
    return bt


def _page_valid(bt, ctx_valid: np.ndarray, num_pages: int) -> np.ndarray:
    """Valid slot prefix of every physical page given tokens present per sequence."""
    valid = np.zeros(num_pages, dtype=np.int32)
    num_layers, num_seqs, _ = bt.shape
    for layer in range(num_layers):
        for b in range(num_seqs):
            n = int(ctx_valid[b])
            full, rem = divmod(n, PAGE)
            pages = bt[layer, b]
            if full:
                valid[pages[:full]] = PAGE
            if rem:
                valid[pages[full]] = rem
    return valid


def _finish(name, seed, num_layers, hq, hkv, d, sigma, ctx, bt, num_pages, append, note):
    ctx = np.asarray(ctx, dtype=np.int32)
    present = ctx - 1 if append else ctx
    valid = _page_valid(bt, np.maximum(present, 0), num_pages)
    return Workload(name=name, seed=seed, num_layers=num_layers, num_seqs=len(ctx),
                    num_q_heads=hq, num_kv_heads=hkv, head_dim=d, sigma=sigma,
                    ctx_lens=ctx, block_tables=bt, num_pages=num_pages,
                    page_valid=valid, append=append, pool_note=note)


def _pages(n) -> np.ndarray:
    return -(-np.asarray(n, dtype=np.int64) // PAGE)


def make_workload(name: str) -> Workload:
    """The five measured configurations, by name: tiny, c2, c3, c4, c5."""
    if name == "tiny":
        seed = 1001
        rng = np.random.default_rng(seed)
        ctx = np.array([128], np.int32)
        bt = rng.permutation(64)[:8].astype(np.int32).reshape(1, 1, 8)
        return _finish(name, seed, 1, 32, 8, 64, 1.0, ctx, bt, 64, False,
                       "64 pages; 8 of them, in random order, hold the sequence")
    if name == "c2":
        seed = 1002
        rng = np.random.default_rng(seed)
        ctx = rng.integers(1, 513, 8).astype(np.int32)
        need = _pages(ctx).reshape(1, -1)
        bt = _deal_pages(rng, need, 256, 32, interleave=False)
        return _finish(name, seed, 1, 32, 8, 64, 1.0, ctx, bt, 256, False,
                       "256 pages from a shuffled free list, sequence by sequence")
    if name == "c3":
        seed = 1003
        rng = np.random.default_rng(seed)
        ctx = rng.integers(256, 2049, 64).astype(np.int32)
        need = _pages(ctx).reshape(1, -1)
        budget = (128 << 20) // (32 << 10)          # 128 MiB at 32 KiB per page = 4096
        if int(need.sum()) <= budget:
            num_pages, note = budget, "128 MiB budget (4096 pages)"
        else:
            num_pages, note = 2 * budget, ("demand exceeds the 128 MiB default, pool raised "
                                           "to 256 MiB (8192 pages, the 64 x 128 worst case)")
        bt = _deal_pages(rng, need, num_pages, 128, interleave=True)
        return _finish(name, seed, 1, 32, 8, 64, 1.0, ctx, bt, num_pages, False, note)
    if name == "c4":
        seed = 1004
        rng = np.random.default_rng(seed)
        raw = rng.lognormal(math.log(1024.0), 1.0, 256)
        ctx = np.clip(np.rint(raw), 16, 8192).astype(np.int32)
        need = np.broadcast_to(_pages(ctx), (16, 256)).copy()
        demand = int(need.sum())
        num_pages = demand + -(-demand // 100) + 1
        bt = _deal_pages(rng, need, num_pages, 512, interleave=True)
        return _finish(name, seed, 16, 32, 8, 64, 0.5, ctx, bt, num_pages, True,
                       f"demand {demand} pages + 1% slack, dealt round-robin over (layer, seq)")
    if name == "c5":
        seed = 1005
        rng = np.random.default_rng(seed)
        ctx = rng.integers(4096, 16385, 64).astype(np.int32)
        need = _pages(ctx).reshape(1, -1)
        demand = int(need.sum())
        num_pages = demand + -(-demand // 100) + 1
        bt = _deal_pages(rng, need, num_pages, 1024, interleave=True)
        return _finish(name, seed, 1, 28, 4, 128, 1.0, ctx, bt, num_pages, False,
                       f"demand {demand} pages + 1% slack, interleaved")
    raise ValueError(f"unknown workload {name!r}")


WORKLOADS = ["tiny", "c2", "c3", "c4", "c5"]


# ------------------------------------------------------------------ prefill
@dataclass
class PrefillWorkload:
    """A chunk of new tokens per sequence on top of ``ctx_before`` cached ones.

    ``base`` carries the pool and block tables; its ``ctx_lens`` are the
    lengths after the chunk, and only the ``ctx_before`` tokens are valid in
    the pool (the chunk's slots are NaN until the chunk is written). Row
    arrays are layer-major: q ``[L][N][Hq][d]``, k/v ``[L][N][Hkv][d]``, with
    sequence ``b`` owning rows ``query_start[b] ..``.
    """
    base: Workload
    ctx_before: np.ndarray   # int32 [B]
    chunks: np.ndarray       # int32 [B]

    @property
    def name(self) -> str:
        return self.base.name

    @property
    def query_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.chunks)]).astype(np.int32)

    @property
    def num_rows(self) -> int:
        return int(self.chunks.sum())

    def _heads(self, which: str) -> int:
        return self.base.num_q_heads if which == "q" else self.base.num_kv_heads

    def _stream(self, which: str) -> int:
        return {"q": STREAM_Q, "k": STREAM_K_NEW, "v": STREAM_V_NEW}[which]

    def rows_bits(self, which: str, layer: int, rows) -> np.ndarray:
        """Host copy of the listed rows of one layer: ``[len(rows)][H][d]``."""
        w = self.base
        per_row = self._heads(which) * w.head_dim
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        idx = (layer * self.num_rows + rows)[:, None] * per_row + np.arange(per_row, dtype=np.int64)[None, :]
        v = values_np(w.seed, self._stream(which), idx, w.table())
        return v.reshape(rows.size, self._heads(which), w.head_dim)

    def rows_device(self, which: str, device):
        """All layers' rows made on ``device``, bit-identical to ``rows_bits``
        (int16 ``[L][N][H][d]``)."""
        import torch
        w = self.base
        shape = (w.num_layers, self.num_rows, self._heads(which), w.head_dim)
        total = int(np.prod(shape))
        table = torch.from_numpy(w.table().view(np.int16)).to(device)
        out = torch.empty(total, dtype=torch.int16, device=device)
        for start in range(0, total, 1 << 26):
            end = min(total, start + (1 << 26))
            idx = torch.arange(start, end, dtype=torch.int64, device=device)
            out[start:end] = table[hash32(w.seed, self._stream(which), idx) >> 16]
            del idx
        return out.view(shape)

    def attended_pairs(self) -> int:
        """(query token, key) pairs of one layer and one query head: token i of
        sequence b sees ctx_before[b] + i + 1 keys."""
        c = self.ctx_before.astype(np.int64)
        n = self.chunks.astype(np.int64)
        return int((n * c + n * (n + 1) // 2).sum())

    def flops_per_layer(self) -> int:
        """2 d flops for the score and 2 d for the weighted value, per query
        head and attended pair."""
        w = self.base
        return 4 * w.head_dim * w.num_q_heads * self.attended_pairs()

    def write_bytes_per_layer(self) -> int:
        w = self.base
        return self.num_rows * w.num_kv_heads * w.head_dim * 2 * 2


def make_prefill_workload(name: str) -> PrefillWorkload:
    """Prefill configurations: ``prefill`` is the 16-layer prefill of 8 prompts
    of 2048 tokens (the context limit of the samir-vllm engine) at the
    Llama-3.2-1B attention shape; ``prefill_d128`` is 4 prompts of 4096 tokens
    at the 28q/4kv, d=128 shape, one layer; ``prefill_chunked`` continues 8
    caches of U[0, 4096] tokens with 512-token chunks (one layer, d=64)."""
    if name == "prefill":
        seed, layers, hq, hkv, d = 1006, 16, 32, 8, 64
        before = np.zeros(8, np.int32)
        chunks = np.full(8, 2048, np.int32)
        stride = 128
    elif name == "prefill_d128":
        seed, layers, hq, hkv, d = 1007, 1, 28, 4, 128
        before = np.zeros(4, np.int32)
        chunks = np.full(4, 4096, np.int32)
        stride = 256
    elif name == "prefill_chunked":
        seed, layers, hq, hkv, d = 1008, 1, 32, 8, 64
        rng0 = np.random.default_rng(seed)
        before = rng0.integers(0, 4097, 8).astype(np.int32)
        chunks = np.full(8, 512, np.int32)
        stride = 288
    else:
        raise ValueError(f"unknown prefill workload {name!r}")
    rng = np.random.default_rng(seed + 100)
    total = before + chunks
    need = np.broadcast_to(_pages(total), (layers, total.size)).copy()
    demand = int(need.sum())
    num_pages = demand + -(-demand // 100) + 1
    bt = _deal_pages(rng, need, num_pages, stride, interleave=True)
    base = _finish(name, seed, layers, hq, hkv, d, 1.0, total, bt, num_pages, False,
                   f"demand {demand} pages + 1% slack, interleaved; chunk slots NaN until written")
    base.page_valid = _page_valid(bt, before, num_pages)
    return PrefillWorkload(base=base, ctx_before=before, chunks=chunks)


PREFILL_WORKLOADS = ["prefill", "prefill_d128", "prefill_chunked"]


def custom(seed: int, ctx_lens: List[int], num_q_heads: int = 32, num_kv_heads: int = 8,
           head_dim: int = 64, num_layers: int = 1, sigma: float = 1.0,
           append: bool = False, stride: Optional[int] = None, extra_pages: int = 3,
           interleave: bool = True, name: str = "custom") -> Workload:
    """A small seeded workload with the given context lengths."""
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    need = np.broadcast_to(_pages(ctx), (num_layers, ctx.size)).copy()
    if stride is None:
        stride = max(1, int(need.max()) if need.size else 1)
    num_pages = int(need.sum()) + extra_pages
    bt = _deal_pages(rng, need, num_pages, stride, interleave=interleave)
    return _finish(name, seed, num_layers, num_q_heads, num_kv_heads, head_dim, sigma,
                   ctx, bt, num_pages, append, "custom")
