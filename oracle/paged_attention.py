"""Plain FP64 CPU oracle for paged decode attention, the paged KV append, and
paged prefill attention (a chunk of prompt tokens written into the pages, then
causal attention over them).

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library; it reads the documented
pool layout and nothing else.

Sources (web pages, cited by title and section):

* [samir-course] "Curso gratuito recorre la inferencia de LLM con videos, notas
  y un motor funcional en C++" (news-factory.app), section "¿Cómo administra
  el motor la memoria de la caché KV?": one shared pool of BF16 pages, each
  physical page holding the keys and values of 16 tokens; a block table per
  sequence and per layer; decode attention reads each sequence's cached pages
  where they lie instead of first gathering a contiguous prefix, with an FP32
  online softmax.
* [samir-review] comrad404.com review of the samir-vllm README, section
  "Что README говорит о KV-кэше и пакетном декодировании": prefill fills a
  request's pages, decode adds the new token's K/V.
* [tiny-vllm] ... section "Prefill vs. Decode": prefill processes all the
  input tokens at once (compute-bound); decode produces one token at a time
  (bound by fetching the cached K/V).
* [tiny-vllm] "Construye tu propio motor de inferencia LLM de alto rendimiento
  en C++ y CUDA" (aibit.im), section "Atención de Consulta Agrupada (GQA)":
  contiguous grouping, q head i uses KV head i / (q heads per KV head), and a
  token-major contiguous KV cache ([token][kv_head][head_dim]).

Readings taken where the pages are silent:

* The attention is the standard scaled dot-product softmax attention
  (the pages name self-attention but never print the formula); the scale is an
  argument (1/sqrt(head_dim) in every workload).
* Online softmax reaches the two-pass softmax exactly up to rounding order, so
  the oracle is the plain definition: gather, scores, two-pass softmax,
  weighted sum of V, all in float64.
* Pool layout inside a page (the pages give none): K is
  ``[num_pages][num_kv_heads][head_dim / 32][16][32]`` (the head dimensions
  in slabs of 32, each slab holding all 16 slots) and V is
  ``[num_pages][num_kv_heads][head_dim][16]`` (V stores the 16 slots of each
  dimension together). One physical page id indexes both. The oracle takes
  the K pool as that 5-D array and V as the 4-D one.
* ``ctx_len == 0`` gives an all-zero output. Slots at or beyond ``ctx_len``
  and pages a sequence does not reference may hold any bits, NaN included;
  they never contribute.

Arrays of BF16 values are passed as ``uint16`` bit patterns.
"""

from __future__ import annotations

import numpy as np

PAGE_SIZE = 16  # tokens per physical page [samir-course]
K_SLAB = 32     # head dimensions per K slab (pool layout reading above)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns exactly to float64.

    A BF16 value is the upper 16 bits of an IEEE binary32 value, so shifting
    the bits up by 16 and reinterpreting as float32 is exact; float32 to
    float64 is exact too.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns stay NaN
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def k_slot_row(k_pool: np.ndarray, physical: int, slot: int) -> np.ndarray:
    """The K values of one slot of one page, all KV heads: ``[Hkv][d]`` bits.

    Dimension ``i`` of the row lies in slab ``i // 32`` at column ``i % 32``,
    so concatenating the slabs in order gives the row.
    """
    num_kv_heads, slabs = k_pool.shape[1], k_pool.shape[2]
    return k_pool[physical, :, :, slot, :].reshape(num_kv_heads, slabs * K_SLAB)


def set_k_slot_row(k_pool: np.ndarray, physical: int, slot: int, rows: np.ndarray) -> None:
    """Store ``rows`` (``[Hkv][d]`` bits) into one slot of one page, slab by
    slab (the inverse of ``k_slot_row``)."""
    rows = np.asarray(rows, dtype=np.uint16)
    k_pool[physical, :, :, slot, :] = rows.reshape(rows.shape[0], -1, K_SLAB)


def gather_sequence(k_pool: np.ndarray, v_pool: np.ndarray,
                    block_table_row: np.ndarray, ctx_len: int):
    """Copy one sequence's cached tokens out of the pages into contiguous
    token-major arrays ``Kc[t][kv_head][d]`` and ``Vc[t][kv_head][d]`` (FP64).

    Token ``t`` lives in logical page ``t // 16`` at slot ``t % 16``; the block
    table row maps that logical page to a physical page [samir-course]. The
    contiguous result has the token-major layout of [tiny-vllm]'s
    pre-paging cache.
    """
    n = int(ctx_len)
    num_pages, num_kv_heads, slabs, page, width = k_pool.shape
    head_dim = slabs * width
    assert page == PAGE_SIZE and width == K_SLAB
    assert v_pool.shape == (num_pages, num_kv_heads, head_dim, PAGE_SIZE)
    kc = np.empty((n, num_kv_heads, head_dim), dtype=np.float64)
    vc = np.empty((n, num_kv_heads, head_dim), dtype=np.float64)
    for t in range(n):
        logical_page = t // PAGE_SIZE
        slot = t % PAGE_SIZE
        physical = int(block_table_row[logical_page])
        assert 0 <= physical < num_pages, "block table names a page outside the pool"
        kc[t] = bf16_bits_to_f64(k_slot_row(k_pool, physical, slot))
        vc[t] = bf16_bits_to_f64(v_pool[physical, :, :, slot])
    return kc, vc


def attend_one_head(q_vec: np.ndarray, keys: np.ndarray, values: np.ndarray,
                    scale: float) -> np.ndarray:
    """Standard softmax attention of one query vector over ``n`` keys/values.

    ``s_t = scale * <q, k_t>``; two-pass softmax (max, then exponentials and
    their sum); output ``sum_t e_t v_t / sum_t e_t``.
    """
    scores = scale * (keys @ q_vec)          # [n]
    m = np.max(scores)
    e = np.exp(scores - m)                   # [n]
    z = np.sum(e)
    return (e @ values) / z                  # [d]


def decode_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                     block_tables: np.ndarray, ctx_lens: np.ndarray,
                     scale: float) -> np.ndarray:
    """Decode-step grouped-query attention over paged K/V, in float64.

    q            uint16 (BF16 bits) ``[B][Hq][d]``, one new query per sequence
    k_pool       uint16 ``[P][Hkv][d/32][16][32]``
    v_pool       uint16 ``[P][Hkv][d][16]``
    block_tables int ``[B][stride]`` physical page of each logical page
    ctx_lens     int ``[B]`` cached tokens to attend over (0 gives zeros)
    scale        softmax scale; a float32 value is widened exactly
    returns      float64 ``[B][Hq][d]``

    Query head ``h`` reads KV head ``h // (Hq // Hkv)`` (contiguous grouping,
    [tiny-vllm] "Atención de Consulta Agrupada (GQA)").
    """
    num_seqs, num_q_heads, head_dim = q.shape
    num_kv_heads = k_pool.shape[1]
    assert num_q_heads % num_kv_heads == 0
    group = num_q_heads // num_kv_heads
    scale = float(np.float64(scale))
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for b in range(num_seqs):
        n = int(ctx_lens[b])
        if n == 0:
            continue
        kc, vc = gather_sequence(k_pool, v_pool, block_tables[b], n)
        qb = bf16_bits_to_f64(q[b])
        for h in range(num_q_heads):
            g = h // group
            out[b, h] = attend_one_head(qb[h], kc[:, g, :], vc[:, g, :], scale)
    return out


def kv_append(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray,
              v_new: np.ndarray, block_tables: np.ndarray,
              positions: np.ndarray):
    """Write each sequence's new-token K/V row into its page slot.

    Decode adds the new token to the cache ([samir-review]); token ``pos``
    goes to slot ``pos % 16`` of physical page ``block_table[pos // 16]``.
    ``k_new``/``v_new`` are uint16 ``[B][Hkv][d]`` (one projection row of
    ``Hkv * d`` values per sequence). A negative position skips the sequence.
    Returns new pools; the inputs are not modified. A bit copy: the result is
    exact.
    """
    k_out = np.array(k_pool, dtype=np.uint16, copy=True)
    v_out = np.array(v_pool, dtype=np.uint16, copy=True)
    for b in range(k_new.shape[0]):
        pos = int(positions[b])
        if pos < 0:
            continue
        physical = int(block_tables[b][pos // PAGE_SIZE])
        slot = pos % PAGE_SIZE
        set_k_slot_row(k_out, physical, slot, k_new[b])
        v_out[physical, :, :, slot] = v_new[b]
    return k_out, v_out


def kv_write(k_pool: np.ndarray, v_pool: np.ndarray, k_rows: np.ndarray,
             v_rows: np.ndarray, query_start: np.ndarray, block_tables: np.ndarray,
             ctx_before: np.ndarray):
    """Write each sequence's chunk of new tokens into its pages.

    Prefill fills a request's pages ([samir-review]). Sequence ``b`` owns rows
    ``query_start[b] .. query_start[b+1]-1`` of ``k_rows``/``v_rows`` (uint16
    ``[N][Hkv][d]``); its row ``i`` is the token at position
    ``ctx_before[b] + i``, stored by the same rule as a single appended token
    (slot ``pos % 16`` of page ``block_table[pos // 16]``). Returns new pools.
    """
    k_out = np.array(k_pool, dtype=np.uint16, copy=True)
    v_out = np.array(v_pool, dtype=np.uint16, copy=True)
    for b in range(len(query_start) - 1):
        for row in range(int(query_start[b]), int(query_start[b + 1])):
            pos = int(ctx_before[b]) + row - int(query_start[b])
            physical = int(block_tables[b][pos // PAGE_SIZE])
            slot = pos % PAGE_SIZE
            set_k_slot_row(k_out, physical, slot, k_rows[row])
            v_out[physical, :, :, slot] = v_rows[row]
    return k_out, v_out


def prefill_attention(q: np.ndarray, k_pool: np.ndarray, v_pool: np.ndarray,
                      k_rows: np.ndarray, v_rows: np.ndarray, query_start: np.ndarray,
                      block_tables: np.ndarray, ctx_before: np.ndarray, scale: float):
    """Prefill of a chunk of new tokens per sequence, in float64.

    Prefill processes all input tokens of a request at once ([tiny-vllm],
    "Prefill vs. Decode") and fills the request's pages ([samir-review]).
    Readings: attention is causal (the token at position ``p`` attends over
    positions ``0 .. p`` of its own sequence, as in any decoder-only model;
    the pages do not print the mask), and a chunk may continue a cache that
    already holds ``ctx_before[b]`` tokens (a shared prefix, or an earlier
    chunk).

    q            uint16 ``[N][Hq][d]``, row ``query_start[b] + i`` is token ``i``
                 of sequence ``b``'s chunk
    k_rows/v_rows uint16 ``[N][Hkv][d]``, the chunk's keys and values
    query_start  int ``[B + 1]``, nondecreasing row offsets
    ctx_before   int ``[B]``, tokens already in each sequence's cache
    returns      (out float64 ``[N][Hq][d]``, k_pool', v_pool') with the chunk
                 written into the pools
    """
    k_new_pool, v_new_pool = kv_write(k_pool, v_pool, k_rows, v_rows, query_start,
                                      block_tables, ctx_before)
    num_rows, num_q_heads, head_dim = q.shape
    group = num_q_heads // k_pool.shape[1]
    scale = float(np.float64(scale))
    out = np.zeros((num_rows, num_q_heads, head_dim), dtype=np.float64)
    for b in range(len(query_start) - 1):
        first, last = int(query_start[b]), int(query_start[b + 1])
        if last == first:
            continue
        before = int(ctx_before[b])
        kc, vc = gather_sequence(k_new_pool, v_new_pool, block_tables[b], before + last - first)
        for row in range(first, last):
            p = before + row - first                 # the query token's position
            qr = bf16_bits_to_f64(q[row])
            for h in range(num_q_heads):
                g = h // group
                out[row, h] = attend_one_head(qr[h], kc[:p + 1, g, :], vc[:p + 1, g, :], scale)
    return out, k_new_pool, v_new_pool
