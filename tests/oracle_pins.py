"""Pins for the FP64 oracle: checks against facts fixed by the pages and by
mathematics, not by the oracle itself.

Every pin is a plain function ``pin_xxx(o)`` taking an oracle module ``o``
(``decode_attention``, ``kv_append``, ``gather_sequence``,
``bf16_bits_to_f64``) and raising ``AssertionError`` on failure. The pins are
run against the real oracle (test_oracle_pins.py) and against copies of it
with planted mistakes (test_oracle_mutations.py), which each must trip at
least one pin.

Inputs are built here from contiguous token-major K/V with this module's own
scatter into pages, independently of the oracle's gather.
"""

from __future__ import annotations

import math

import numpy as np

PAGE = 16
NAN_BF16 = np.uint16(0x7FC0)


# ----------------------------------------------------------------- helpers
def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to BF16 bit patterns, round-to-nearest-even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bits_to_f64_ref(bits) -> np.ndarray:
    """Independent BF16 decode from the IEEE fields (sign, exponent, mantissa)."""
    b = np.asarray(bits, dtype=np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    exp = (b >> 7) & 0xFF
    man = (b & 0x7F).astype(np.float64)
    normal = sign * (1.0 + man / 128.0) * np.power(2.0, exp.astype(np.float64) - 127.0)
    sub = sign * (man / 128.0) * 2.0 ** -126
    out = np.where(exp == 0, sub, normal)
    out = np.where((exp == 0xFF) & (man == 0), sign * np.inf, out)
    out = np.where((exp == 0xFF) & (man != 0), np.nan, out)
    return out


def random_bf16(rng, shape, sigma=1.0) -> np.ndarray:
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(sigma))


def to_k_slabs(k_by_slot_pool: np.ndarray) -> np.ndarray:
    """``[P][Hkv][16][d]`` (one row per slot) to the pool's K layout
    ``[P][Hkv][d/32][16][32]``: dimension i of slot t goes to slab i // 32,
    row t, column i % 32."""
    p, h, page, d = k_by_slot_pool.shape
    assert d % 32 == 0
    return np.ascontiguousarray(k_by_slot_pool.reshape(p, h, page, d // 32, 32).transpose(0, 1, 3, 2, 4))


def k_by_slot(k_pool: np.ndarray) -> np.ndarray:
    """The inverse of ``to_k_slabs``: the K pool as ``[P][Hkv][16][d]``."""
    p, h, slabs, page, width = k_pool.shape
    return np.ascontiguousarray(k_pool.transpose(0, 1, 3, 2, 4)).reshape(p, h, page, slabs * width)


def scatter_pages(kc_bits, vc_bits, ctx_lens, num_pages, rng, fill=NAN_BF16,
                  stride=None, pages_per_seq=None):
    """Place contiguous per-sequence K/V (``[B][n][Hkv][d]`` lists of uint16)
    into a pool at random physical pages. Unused slots and pages get ``fill``.

    K pool ``[P][Hkv][d/32][16][32]``; V pool ``[P][Hkv][d][16]``.
    Returns (k_pool, v_pool, block_tables).
    """
    num_seqs = len(ctx_lens)
    hkv, d = kc_bits[0].shape[1], kc_bits[0].shape[2]
    need = [max(1, -(-int(n) // PAGE)) for n in ctx_lens]
    if pages_per_seq is not None:
        need = [max(a, int(b)) for a, b in zip(need, pages_per_seq)]
    if stride is None:
        stride = max(need)
    assert sum(need) <= num_pages
    k_pool = np.full((num_pages, hkv, PAGE, d), fill, dtype=np.uint16)
    v_pool = np.full((num_pages, hkv, d, PAGE), fill, dtype=np.uint16)
    order = rng.permutation(num_pages)
    bt = np.zeros((num_seqs, stride), dtype=np.int32)
    nxt = 0
    for b in range(num_seqs):
        for j in range(need[b]):
            bt[b, j] = order[nxt]
            nxt += 1
        for t in range(int(ctx_lens[b])):
            p = bt[b, t // PAGE]
            k_pool[p, :, t % PAGE, :] = kc_bits[b][t]
            v_pool[p, :, :, t % PAGE] = vc_bits[b][t]
    return to_k_slabs(k_pool), v_pool, bt


def make_case(rng, num_seqs, hq, hkv, d, ctx_lens, extra_pages=5, sigma=1.0):
    kc = [random_bf16(rng, (int(n), hkv, d), sigma) for n in ctx_lens]
    vc = [random_bf16(rng, (int(n), hkv, d), sigma) for n in ctx_lens]
    q = random_bf16(rng, (num_seqs, hq, d), sigma)
    pages = sum(max(1, -(-int(n) // PAGE)) for n in ctx_lens) + extra_pages
    k_pool, v_pool, bt = scatter_pages(kc, vc, ctx_lens, pages, rng)
    return q, kc, vc, k_pool, v_pool, bt, np.asarray(ctx_lens, dtype=np.int32)


def _assert_close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# -------------------------------------------------------------------- pins
def pin_bf16_widening(o):
    """BF16 widening against the IEEE-754 field definition, every pattern."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = o.bf16_bits_to_f64(bits)
    ref = bits_to_f64_ref(bits)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite]), "finite BF16 patterns widen wrongly"
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN patterns widen wrongly"
    inf = np.isinf(ref)
    assert np.array_equal(got[inf], ref[inf]), "infinite BF16 patterns widen wrongly"
    assert o.bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert o.bf16_bits_to_f64(np.array([0xC040], np.uint16))[0] == -3.0


def pin_sdpa_library(o):
    """Equals torch's scaled_dot_product_attention in float64 on CPU with the
    KV heads repeated G times each (contiguous grouping, so repeat_interleave)."""
    import torch
    rng = np.random.default_rng(11)
    for (hq, hkv, d, lens) in [(8, 2, 64, [1, 15, 16, 17, 40]),
                               (6, 3, 32, [33, 2, 64]),
                               (7, 1, 32, [5, 48]),
                               (4, 4, 32, [31])]:
        q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, len(lens), hq, hkv, d, lens)
        scale = np.float32(1.0 / math.sqrt(d)) * np.float32(1.5)
        out = o.decode_attention(q, k_pool, v_pool, bt, ctx, scale)
        g = hq // hkv
        for b, n in enumerate(lens):
            qt = torch.from_numpy(bits_to_f64_ref(q[b])).reshape(1, hq, 1, d)
            kt = torch.from_numpy(bits_to_f64_ref(kc[b])).permute(1, 0, 2)  # [hkv][n][d]
            vt = torch.from_numpy(bits_to_f64_ref(vc[b])).permute(1, 0, 2)
            kt = kt.repeat_interleave(g, dim=0).unsqueeze(0).contiguous()
            vt = vt.repeat_interleave(g, dim=0).unsqueeze(0).contiguous()
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, scale=float(scale)).reshape(hq, d).numpy()
            _assert_close(out[b], ref, 1e-12, f"sdpa b={b} n={n}")


def pin_ctx_one_returns_value(o):
    """A single cached token gets softmax weight 1: the output is that V row."""
    rng = np.random.default_rng(12)
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 3, 8, 2, 32, [1, 1, 1])
    out = o.decode_attention(q, k_pool, v_pool, bt, ctx, np.float32(0.25))
    for b in range(3):
        for h in range(8):
            ref = bits_to_f64_ref(vc[b][0, h // 4])
            assert np.array_equal(out[b, h], ref), f"ctx=1 b={b} h={h}"


def pin_ctx_two_sigmoid(o):
    """Two tokens: the weight of token 0 is the logistic function of s0 - s1."""
    rng = np.random.default_rng(13)
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 2, 4, 2, 32, [2, 2])
    scale = np.float32(0.3)
    out = o.decode_attention(q, k_pool, v_pool, bt, ctx, scale)
    for b in range(2):
        for h in range(4):
            g = h // 2
            qv = bits_to_f64_ref(q[b, h])
            k0 = bits_to_f64_ref(kc[b][0, g])
            k1 = bits_to_f64_ref(kc[b][1, g])
            x = float(scale) * (float(np.dot(qv, k0)) - float(np.dot(qv, k1)))
            w0 = 1.0 / (1.0 + math.exp(-x))
            ref = w0 * bits_to_f64_ref(vc[b][0, g]) + (1.0 - w0) * bits_to_f64_ref(vc[b][1, g])
            _assert_close(out[b, h], ref, 1e-13, f"ctx=2 b={b} h={h}")


def pin_identical_keys_mean(o):
    """All keys equal: equal weights, the output is the mean of the V rows."""
    rng = np.random.default_rng(14)
    n = 37
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 1, 4, 1, 32, [n])
    row = random_bf16(rng, (1, 32))
    kc_same = [np.broadcast_to(row, (n, 1, 32)).copy()]
    k_pool, v_pool, bt = scatter_pages(kc_same, vc, [n], 6, rng)
    out = o.decode_attention(q, k_pool, v_pool, bt, ctx, np.float32(0.7))
    ref = bits_to_f64_ref(vc[0][:, 0, :]).mean(axis=0)
    for h in range(4):
        _assert_close(out[0, h], ref, 1e-13, f"identical keys h={h}")


def pin_zero_query_or_scale_mean(o):
    """q = 0 or scale = 0 makes every score 0: output is the mean of V."""
    rng = np.random.default_rng(15)
    lens = [20, 3]
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 2, 6, 3, 32, lens)
    zero_q = np.zeros_like(q)
    for qq, sc in [(zero_q, np.float32(0.5)), (q, np.float32(0.0))]:
        out = o.decode_attention(qq, k_pool, v_pool, bt, ctx, sc)
        for b, n in enumerate(lens):
            for h in range(6):
                ref = bits_to_f64_ref(vc[b][:, h // 2, :]).mean(axis=0)
                _assert_close(out[b, h], ref, 1e-13, f"mean V b={b} h={h}")


def pin_value_ones_convex(o):
    """Softmax weights sum to one: all-ones V gives exactly 1 (to rounding)."""
    rng = np.random.default_rng(16)
    lens = [1, 16, 50]
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 3, 4, 2, 32, lens)
    ones = [np.full((n, 2, 32), 0x3F80, dtype=np.uint16) for n in lens]
    k_pool, v_pool, bt = scatter_pages(kc, ones, lens, 10, rng)
    out = o.decode_attention(q, k_pool, v_pool, bt, ctx, np.float32(0.4))
    _assert_close(out, np.ones_like(out), 1e-14, "V = 1")


def pin_hard_max(o):
    """With a huge scale one token dominates: exp of the others underflows to
    exactly 0 and the output equals that token's V row (needs the max shift)."""
    rng = np.random.default_rng(17)
    n, d = 12, 32
    q = f32_to_bf16_bits(np.ones((1, 1, d), np.float32))
    kc_f = np.full((n, 1, d), -1.0, np.float32)
    kc_f[5] = 1.0
    kc = [f32_to_bf16_bits(kc_f)]
    vc = [random_bf16(rng, (n, 1, d))]
    k_pool, v_pool, bt = scatter_pages(kc, vc, [n], 3, rng)
    out = o.decode_attention(q, k_pool, v_pool, bt, np.array([n], np.int32), np.float32(1.0e4))
    assert np.array_equal(out[0, 0], bits_to_f64_ref(vc[0][5, 0])), "hard max"


def pin_ctx_zero_gives_zeros(o):
    rng = np.random.default_rng(18)
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 2, 4, 2, 32, [0, 5])
    out = o.decode_attention(q, k_pool, v_pool, bt, ctx, np.float32(0.5))
    assert np.array_equal(out[0], np.zeros((4, 32))), "ctx=0 must give zeros"
    assert np.all(np.isfinite(out[1]))


def pin_page_permutation_invariant(o):
    """Moving pages to other physical slots (and rewriting the block tables)
    leaves the output bitwise unchanged."""
    rng = np.random.default_rng(19)
    lens = [35, 16, 1, 64]
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 4, 8, 2, 64, lens, extra_pages=7)
    out1 = o.decode_attention(q, k_pool, v_pool, bt, ctx, np.float32(0.25))
    perm = rng.permutation(k_pool.shape[0])       # new position of each page
    k2 = np.empty_like(k_pool)
    v2 = np.empty_like(v_pool)
    k2[perm] = k_pool
    v2[perm] = v_pool
    bt2 = perm[bt].astype(np.int32)
    out2 = o.decode_attention(q, k2, v2, bt2, ctx, np.float32(0.25))
    assert np.array_equal(out1, out2), "page placement changed the output"


def pin_tail_and_free_pages_ignored(o):
    """Slots past ctx_len and pages no sequence references never contribute:
    NaN, +1e30-like and zero fills give bitwise equal outputs."""
    rng = np.random.default_rng(20)
    lens = [17, 30, 5]
    kc = [random_bf16(rng, (n, 2, 32)) for n in lens]
    vc = [random_bf16(rng, (n, 2, 32)) for n in lens]
    q = random_bf16(rng, (3, 4, 32))
    outs = []
    for fill in (NAN_BF16, np.uint16(0x7149), np.uint16(0xF149), np.uint16(0)):
        r = np.random.default_rng(99)                     # same placement each time
        k_pool, v_pool, bt = scatter_pages(kc, vc, lens, 12, r, fill=fill)
        outs.append(o.decode_attention(q, k_pool, v_pool, bt, np.array(lens, np.int32),
                                       np.float32(0.35)))
    for x in outs[1:]:
        assert np.array_equal(outs[0], x), "tail/free-page contents leaked into the output"
    assert np.all(np.isfinite(outs[0]))


def pin_power_of_two_scale(o):
    """(q * 2^k, scale * 2^-k) gives the same scores exactly, so the same output."""
    rng = np.random.default_rng(21)
    lens = [40, 9]
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 2, 4, 2, 32, lens, sigma=0.5)
    out1 = o.decode_attention(q, k_pool, v_pool, bt, ctx, np.float32(0.25))
    q4 = f32_to_bf16_bits(bits_to_f64_ref(q).astype(np.float32) * np.float32(4.0))
    assert np.array_equal(bits_to_f64_ref(q4), 4.0 * bits_to_f64_ref(q))   # exact
    out2 = o.decode_attention(q4, k_pool, v_pool, bt, ctx, np.float32(0.0625))
    assert np.array_equal(out1, out2), "power-of-two rescaling changed the output"
    out3 = o.decode_attention(q, k_pool, v_pool, bt, ctx, np.float32(0.5))
    assert not np.array_equal(out1, out3), "the scale has no effect"


def pin_kv_head_locality(o):
    """Changing the V of KV head j changes exactly q heads [jG, (j+1)G)."""
    rng = np.random.default_rng(22)
    lens = [23]
    hq, hkv, d = 12, 3, 32
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 1, hq, hkv, d, lens)
    base = o.decode_attention(q, k_pool, v_pool, bt, ctx, np.float32(0.3))
    g = hq // hkv
    for j in range(hkv):
        vc2 = [vc[0].copy()]
        vc2[0][:, j, :] = random_bf16(rng, (lens[0], d))
        r = np.random.default_rng(5)
        kp, vp, bt2 = scatter_pages(kc, vc2, lens, 4, r)
        kp0, vp0, bt0 = scatter_pages(kc, vc, lens, 4, np.random.default_rng(5))
        ref = o.decode_attention(q, kp0, vp0, bt0, ctx, np.float32(0.3))
        out = o.decode_attention(q, kp, vp, bt2, ctx, np.float32(0.3))
        assert np.array_equal(ref, base)
        for h in range(hq):
            changed = not np.array_equal(out[0, h], ref[0, h])
            assert changed == (j * g <= h < (j + 1) * g), f"kv head {j} -> q head {h}"


def pin_gather_roundtrip(o):
    """gather_sequence inverts this module's scatter bit for bit."""
    rng = np.random.default_rng(23)
    lens = [1, 16, 33]
    q, kc, vc, k_pool, v_pool, bt, ctx = make_case(rng, 3, 4, 2, 64, lens)
    for b, n in enumerate(lens):
        kg, vg = o.gather_sequence(k_pool, v_pool, bt[b], n)
        assert np.array_equal(kg, bits_to_f64_ref(kc[b])), f"K gather b={b}"
        assert np.array_equal(vg, bits_to_f64_ref(vc[b])), f"V gather b={b}"


def pin_append_then_gather(o):
    """Appending token n-1 then gathering n tokens gives the contiguous cache
    with the new row at the end, and no other pool bit changes."""
    rng = np.random.default_rng(24)
    lens = [16, 1, 20, 47, 17]              # new token positions 15, 0, 19, 46, 16
    hkv, d = 2, 64
    kc = [random_bf16(rng, (n, hkv, d)) for n in lens]
    vc = [random_bf16(rng, (n, hkv, d)) for n in lens]
    old = [n - 1 for n in lens]
    # allocate pages for all n tokens, store only the first n-1
    need = [-(-n // PAGE) for n in lens]
    k_pool, v_pool, bt = scatter_pages([k[:n - 1] for k, n in zip(kc, lens)],
                                       [v[:n - 1] for v, n in zip(vc, lens)],
                                       old, sum(need) + 4, rng, stride=max(need),
                                       pages_per_seq=need)
    k_new = np.stack([k[-1] for k in kc])
    v_new = np.stack([v[-1] for v in vc])
    pos = np.array(old, np.int32)
    k2, v2 = o.kv_append(k_pool, v_pool, k_new, v_new, bt, pos)
    for b, n in enumerate(lens):
        kg, vg = o.gather_sequence(k2, v2, bt[b], n)
        assert np.array_equal(kg, bits_to_f64_ref(kc[b])), f"append K b={b}"
        assert np.array_equal(vg, bits_to_f64_ref(vc[b])), f"append V b={b}"
    kd = k_by_slot(k2) != k_by_slot(k_pool)
    vd = v2 != v_pool
    written_k = np.zeros_like(kd)
    written_v = np.zeros_like(vd)
    for b, p in enumerate(old):
        written_k[bt[b][p // PAGE], :, p % PAGE, :] = True
        written_v[bt[b][p // PAGE], :, :, p % PAGE] = True
    assert not np.any(kd & ~written_k), "append touched K bits outside the new slots"
    assert not np.any(vd & ~written_v), "append touched V bits outside the new slots"
    assert np.all(k_by_slot(k2)[written_k] != NAN_BF16) and np.all(v2[written_v] != NAN_BF16)
    # a negative position skips the sequence
    pos_skip = pos.copy()
    pos_skip[2] = -1
    k3, v3 = o.kv_append(k_pool, v_pool, k_new, v_new, bt, pos_skip)
    keep_k = written_k.copy()
    keep_v = written_v.copy()
    keep_k[bt[2][old[2] // PAGE], :, old[2] % PAGE, :] = False
    keep_v[bt[2][old[2] // PAGE], :, :, old[2] % PAGE] = False
    assert np.array_equal(k_by_slot(k3) != k_by_slot(k_pool), keep_k), "skipped sequence: K bits changed"
    assert np.array_equal(v3 != v_pool, keep_v), "skipped sequence: V bits changed"


# ------------------------------------------------------------ prefill pins
def make_prefill_case(rng, hq, hkv, d, befores, chunks, extra_pages=4, sigma=1.0):
    """Contiguous K/V for ``before + chunk`` tokens per sequence: the first
    ``before`` tokens already in pages, the chunk's rows passed separately."""
    tot = [int(a) + int(c) for a, c in zip(befores, chunks)]
    kc = [random_bf16(rng, (n, hkv, d), sigma) for n in tot]
    vc = [random_bf16(rng, (n, hkv, d), sigma) for n in tot]
    q = random_bf16(rng, (int(sum(chunks)), hq, d), sigma)
    per_seq = [max(1, -(-n // PAGE)) for n in tot]
    k_pool, v_pool, bt = scatter_pages([k[:a] for k, a in zip(kc, befores)],
                                       [v[:a] for v, a in zip(vc, befores)], befores,
                                       sum(per_seq) + extra_pages, rng, pages_per_seq=per_seq)
    qs = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    k_rows = np.concatenate([k[a:] for k, a in zip(kc, befores)]).astype(np.uint16)
    v_rows = np.concatenate([v[a:] for v, a in zip(vc, befores)]).astype(np.uint16)
    return q, kc, vc, k_pool, v_pool, bt, qs, np.asarray(befores, np.int64), k_rows, v_rows


def pin_prefill_sdpa_library(o):
    """Causal prefill equals torch's scaled_dot_product_attention in float64
    on contiguous K/V: is_causal=True for an empty cache, and an explicit
    mask (key j visible to chunk token i iff j <= before + i) otherwise."""
    import torch
    rng = np.random.default_rng(41)
    for hq, hkv, d, befores, chunks in [(8, 2, 64, [0, 0], [1, 37]),
                                        (6, 3, 32, [5, 16, 40], [20, 3, 17]),
                                        (7, 1, 32, [0, 31], [33, 1])]:
        q, kc, vc, k_pool, v_pool, bt, qs, bef, k_rows, v_rows = make_prefill_case(
            rng, hq, hkv, d, befores, chunks)
        scale = np.float32(1.0 / math.sqrt(d))
        out, _, _ = o.prefill_attention(q, k_pool, v_pool, k_rows, v_rows, qs, bt, bef, scale)
        g = hq // hkv
        for b, (a, c) in enumerate(zip(befores, chunks)):
            rows = slice(int(qs[b]), int(qs[b + 1]))
            qt = torch.from_numpy(bits_to_f64_ref(q[rows])).permute(1, 0, 2).unsqueeze(0)   # [1][hq][c][d]
            kt = torch.from_numpy(bits_to_f64_ref(kc[b])).permute(1, 0, 2).repeat_interleave(g, 0)
            vt = torch.from_numpy(bits_to_f64_ref(vc[b])).permute(1, 0, 2).repeat_interleave(g, 0)
            kt, vt = kt.unsqueeze(0).contiguous(), vt.unsqueeze(0).contiguous()
            if a == 0:
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qt.contiguous(), kt, vt, is_causal=True, scale=float(scale))
            else:
                mask = torch.arange(a + c)[None, :] <= (a + torch.arange(c))[:, None]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qt.contiguous(), kt, vt, attn_mask=mask, scale=float(scale))
            _assert_close(out[rows], ref[0].permute(1, 0, 2).numpy(), 1e-12, f"prefill sdpa b={b}")


def pin_prefill_last_row_is_decode(o):
    """The last chunk token of every sequence sees the whole cache: its row is
    decode attention over before + chunk tokens of the written pool."""
    rng = np.random.default_rng(42)
    q, kc, vc, k_pool, v_pool, bt, qs, bef, k_rows, v_rows = make_prefill_case(
        rng, 8, 4, 32, [0, 9, 32], [5, 30, 1])
    out, k2, v2 = o.prefill_attention(q, k_pool, v_pool, k_rows, v_rows, qs, bt, bef, 0.25)
    last = qs[1:] - 1
    ref = o.decode_attention(q[last], k2, v2, bt, bef + np.diff(qs), 0.25)
    _assert_close(out[last], ref, 1e-12, "last prefill row vs decode")


def pin_prefill_causality(o):
    """Changing chunk token j's key and value changes rows j.. only; rows
    before it keep every bit."""
    rng = np.random.default_rng(43)
    q, kc, vc, k_pool, v_pool, bt, qs, bef, k_rows, v_rows = make_prefill_case(
        rng, 4, 2, 32, [7], [12])
    base, _, _ = o.prefill_attention(q, k_pool, v_pool, k_rows, v_rows, qs, bt, bef, 0.5)
    for j in (0, 5, 11):
        k2, v2 = k_rows.copy(), v_rows.copy()
        k2[j] = random_bf16(rng, k2[j].shape)
        v2[j] = random_bf16(rng, v2[j].shape)
        out, _, _ = o.prefill_attention(q, k_pool, v_pool, k2, v2, qs, bt, bef, 0.5)
        assert np.array_equal(out[:j], base[:j]), f"rows before {j} changed"
        assert not np.allclose(out[j:], base[j:]), f"rows from {j} did not change"


def pin_prefill_write_matches_appends(o):
    """Writing a chunk equals appending its tokens one position at a time, bit
    for bit; nothing else in the pools changes."""
    rng = np.random.default_rng(44)
    q, kc, vc, k_pool, v_pool, bt, qs, bef, k_rows, v_rows = make_prefill_case(
        rng, 4, 2, 64, [0, 14, 3], [20, 2, 0])
    k_w, v_w = o.kv_write(k_pool, v_pool, k_rows, v_rows, qs, bt, bef)
    k_a, v_a = k_pool.copy(), v_pool.copy()
    chunks = np.diff(qs)
    for i in range(int(chunks.max())):
        pos = np.where(i < chunks, bef + i, -1).astype(np.int32)
        rows = np.minimum(qs[:-1] + i, len(k_rows) - 1)
        k_a, v_a = o.kv_append(k_a, v_a, k_rows[rows], v_rows[rows], bt, pos)
    assert np.array_equal(k_w, k_a) and np.array_equal(v_w, v_a), "chunk write != appends"
    written = 0
    for b in range(len(chunks)):
        for i in range(int(chunks[b])):
            pos = int(bef[b]) + i
            page = bt[b][pos // PAGE]
            assert np.array_equal(k_by_slot(k_w)[page, :, pos % PAGE, :], k_rows[qs[b] + i])
            assert np.array_equal(v_w[page, :, :, pos % PAGE], v_rows[qs[b] + i])
            written += 1
    changed = int(np.count_nonzero(np.any(k_by_slot(k_w) != k_by_slot(k_pool), axis=-1)))
    assert changed <= written * k_pool.shape[1], "bits outside the written slots changed"


def pin_prefill_one_token_is_decode(o):
    """A one-token chunk is one append then one decode step."""
    rng = np.random.default_rng(45)
    q, kc, vc, k_pool, v_pool, bt, qs, bef, k_rows, v_rows = make_prefill_case(
        rng, 6, 2, 32, [0, 1, 16, 47], [1, 1, 1, 1])
    out, k2, v2 = o.prefill_attention(q, k_pool, v_pool, k_rows, v_rows, qs, bt, bef, 0.3)
    k3, v3 = o.kv_append(k_pool, v_pool, k_rows, v_rows, bt, bef.astype(np.int32))
    assert np.array_equal(k2, k3) and np.array_equal(v2, v3)
    _assert_close(out, o.decode_attention(q, k3, v3, bt, bef + 1, 0.3), 1e-12, "one-token prefill")


ALL_PINS = [pin_bf16_widening, pin_sdpa_library, pin_ctx_one_returns_value,
            pin_ctx_two_sigmoid, pin_identical_keys_mean,
            pin_zero_query_or_scale_mean, pin_value_ones_convex, pin_hard_max,
            pin_ctx_zero_gives_zeros, pin_page_permutation_invariant,
            pin_tail_and_free_pages_ignored, pin_power_of_two_scale,
            pin_kv_head_locality, pin_gather_roundtrip, pin_append_then_gather,
            pin_prefill_sdpa_library, pin_prefill_last_row_is_decode, pin_prefill_causality,
            pin_prefill_write_matches_appends, pin_prefill_one_token_is_decode]
