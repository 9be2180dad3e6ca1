"""GPU parity at the edges of the softmax, through the C ABI, against the FP64
oracle.

Contexts reach past three splits at both head shapes (d = 64 with 4 query
heads per KV head, d = 128 with 7), so the log-sum-exp merge sees partials
whose maxima lie far apart. Cases:

* scale 0 (every weight equal: the mean of V), a negative scale, a large scale
  (4.0) and one so large that one key takes all the weight in each head
  (exp2 underflows to zero for every other key);
* identical keys (every weight equal whatever the scale: the mean of V),
  compared with both the oracle and that closed form;
* keys rising along the sequence (the running maximum moves at every page
  pair) and falling (it never moves after the first pair);
* finite key and value magnitudes far outside the generator's range (values
  scaled by powers of two up to 2^12, per token).

The bar is the parity bar of every decode test: |gpu - ref| <= 2e-3 and
|gpu - ref| / |ref| <= 1e-2 where |ref| >= 1e-2. Where values are scaled by a
power of two 2^k, the exact output scales by 2^k too (a convex combination of
the values), so that case applies the bar to both outputs divided by the
largest |V| the sequence attends to, rounded up to a power of two: an exact
division that leaves the comparison's relative accuracy unchanged.
"""

import numpy as np
import pytest

import oracle
from gpu_helpers import check_parity, device, log
from paged_kv_decode_02_amd import binding as B
from paged_kv_decode_02_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = [(64, 32, 8), (128, 28, 4)]          # (d, Hq, Hkv): G = 4 and G = 7
CTX = [1, 2, 33, 700, 2500, 6500]             # 6500 tokens: >= 3 splits at any split size <= 2048


def _bits_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _f32_to_bits(x):
    """float32 -> BF16 bits, round to nearest even (exact for the values used
    here, which are BF16 values times powers of two)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


class HostCase:
    """A workload whose pools are taken from host arrays (possibly edited)."""

    def __init__(self, w, k_bits, v_bits, dev):
        import torch
        self.w = w
        self.k_bits, self.v_bits = k_bits, v_bits
        self.k = torch.from_numpy(k_bits.view(np.int16)).to(dev)
        self.v = torch.from_numpy(v_bits.view(np.int16)).to(dev)
        self.pool = B.Pool(self.k, self.v)
        self.bt = torch.from_numpy(np.ascontiguousarray(w.block_tables[0])).to(dev)
        self.ctx = torch.from_numpy(w.ctx_lens).to(dev)
        self.q_bits = w.q_bits()[0]
        self.q = torch.from_numpy(self.q_bits.view(np.int16)).to(dev)

    def run(self, scale, q_bits=None):
        import torch
        q = self.q if q_bits is None else torch.from_numpy(q_bits.view(np.int16)).to(self.q.device)
        out = B.decode(self.pool, q, self.bt, self.ctx, float(scale)).cpu().numpy()
        # the planned launch must give the same bits
        plan = torch.from_numpy(B.decode_plan(self.pool, self.w.ctx_lens, self.w.num_q_heads, self.w.stride)).to(self.q.device)
        planned = B.decode_planned(self.pool, q, self.bt, self.ctx, float(scale), plan).cpu().numpy()
        assert np.array_equal(out, planned), "pa_decode_planned differs from pa_decode"
        return out

    def oracle(self, scale, q_bits=None):
        q = self.q_bits if q_bits is None else q_bits
        return oracle.decode_attention(q, self.k_bits, self.v_bits, self.w.block_tables[0],
                                       self.w.ctx_lens, np.float32(scale))


def _case(d, hq, hkv, seed, dev, edit=None):
    w = W.custom(seed=seed, ctx_lens=CTX, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 name=f"edges-d{d}")
    k, v = w.pool_bits("k"), w.pool_bits("v")
    if edit is not None:
        k, v = edit(w, k, v)
    return HostCase(w, k, v, dev)


def _token_slots(w, b):
    """(page, slot) of every attended token of sequence b."""
    n = int(w.ctx_lens[b])
    t = np.arange(n)
    return w.block_tables[0, b, t // 16], t % 16


@pytest.mark.parametrize("d,hq,hkv", SHAPES, ids=["d64_g4", "d128_g7"])
def test_scales(d, hq, hkv):
    dev = device()
    case = _case(d, hq, hkv, 500 + d, dev)
    for scale in (0.0, -0.125, 4.0, 1.0e4):
        log(f"softmax edges d={d} G={hq // hkv} ctx={CTX} scale={scale} entry=pa_decode")
        out = case.run(scale)
        ref = case.oracle(scale)
        a, r = check_parity(out, ref, f"d={d} scale={scale}")
        log(f"  max abs {a:.2e} max rel {r:.2e}")
        if scale == 0.0:
            # every weight equal: the mean of the attended V rows
            g = hq // hkv
            for b, n in enumerate(CTX):
                pg, sl = _token_slots(case.w, b)
                vrows = _bits_to_f32(case.v_bits[pg, :, :, sl]).astype(np.float64)   # [n][Hkv][d]
                mean = vrows.mean(axis=0)
                check_parity(out[b], np.repeat(mean, g, axis=0), f"d={d} scale 0 seq {b}: mean of V")


@pytest.mark.parametrize("d,hq,hkv", SHAPES, ids=["d64_g4", "d128_g7"])
def test_one_hot_weights(d, hq, hkv):
    """A scale of 1e4 on unit-variance data: the top score of a head leads the
    next by ~1e2 or more, so every other weight is exp2 of a large negative
    number (zero in FP32): the output is the V row of the best key."""
    dev = device()
    case = _case(d, hq, hkv, 600 + d, dev)
    scale = 1.0e4
    out = case.run(scale)
    ref = case.oracle(scale)
    check_parity(out, ref, f"one-hot d={d}")
    g = hq // hkv
    kf = _bits_to_f32(case.k_bits).astype(np.float64)
    qf = _bits_to_f32(case.q_bits).astype(np.float64)
    exact = 0
    for b, n in enumerate(CTX):
        pg, sl = _token_slots(case.w, b)
        keys = kf[pg, :, :, sl, :].reshape(n, hkv, d)   # [n][Hkv][d]
        for h in range(hq):
            s = keys[:, h // g, :] @ qf[b, h]
            top = np.sort(s)[-2:] if n > 1 else s
            if n == 1 or (top[1] - top[0]) * scale > 200.0:
                best = int(np.argmax(s))
                vrow = _bits_to_f32(case.v_bits[pg[best], h // g, :, sl[best]]).astype(np.float64)
                assert np.array_equal(out[b, h].astype(np.float64), vrow), f"seq {b} head {h}: not V of argmax"
                exact += 1
    log(f"one-hot d={d}: {exact} heads equal V of their best key exactly")
    assert exact > 0


@pytest.mark.parametrize("d,hq,hkv", SHAPES, ids=["d64_g4", "d128_g7"])
def test_identical_keys_give_mean_of_v(d, hq, hkv):
    def edit(w, k, v):
        k = k.copy()
        for b in range(w.num_seqs):
            pg, sl = _token_slots(w, b)
            for i in range(pg.size):
                oracle.set_k_slot_row(k, int(pg[i]), int(sl[i]), oracle.k_slot_row(k, int(pg[0]), int(sl[0])))
        return k, v

    dev = device()
    case = _case(d, hq, hkv, 700 + d, dev, edit)
    g = hq // hkv
    for scale in (float(case.w.scale), 4.0, -3.0):
        out = case.run(scale)
        a, r = check_parity(out, case.oracle(scale), f"identical keys d={d} scale={scale}")
        for b, n in enumerate(CTX):
            pg, sl = _token_slots(case.w, b)
            mean = _bits_to_f32(case.v_bits[pg, :, :, sl]).astype(np.float64).mean(axis=0)
            check_parity(out[b], np.repeat(mean, g, axis=0), f"identical keys d={d} seq {b}: mean of V")
        log(f"identical keys d={d} scale={scale}: max abs {a:.2e} max rel {r:.2e}")


@pytest.mark.parametrize("d,hq,hkv", SHAPES, ids=["d64_g4", "d128_g7"])
@pytest.mark.parametrize("direction", ["rising", "falling"])
def test_monotone_scores(d, hq, hkv, direction):
    """Keys scaled along the sequence so every head's scores rise (the running
    maximum moves at each page pair: every rescale taken) or fall (it never
    moves after the first pair: every rescale skipped). Queries are made
    positive so that a larger key scale gives a larger score."""
    def edit(w, k, v):
        k = k.copy()
        kf = _bits_to_f32(k)
        for b in range(w.num_seqs):
            pg, sl = _token_slots(w, b)
            n = pg.size
            for i in range(n):
                frac = i / max(n - 1, 1)
                e = int(round(6 * (frac if direction == "rising" else 1 - frac)))   # 2^0 .. 2^6
                row = np.abs(kf[pg[i], :, :, sl[i], :]) * np.float32(2.0 ** e)
                k[pg[i], :, :, sl[i], :] = _f32_to_bits(row)
        return k, v

    dev = device()
    case = _case(d, hq, hkv, 800 + d, dev, edit)
    qpos = _f32_to_bits(np.abs(_bits_to_f32(case.q_bits)))
    scale = float(case.w.scale) * 0.05
    out = case.run(scale, qpos)
    a, r = check_parity(out, case.oracle(scale, qpos), f"{direction} scores d={d}")
    log(f"{direction} scores d={d}: max abs {a:.2e} max rel {r:.2e}")


@pytest.mark.parametrize("d,hq,hkv", SHAPES, ids=["d64_g4", "d128_g7"])
def test_large_magnitudes(d, hq, hkv):
    """Keys and values of each token scaled by 2^e, e drawn from 0..12 (values
    up to ~2e4 against the generator's ~4.3): exact in BF16. The scores then
    span a wide range and the outputs reach thousands."""
    rng = np.random.default_rng(99 + d)

    def edit(w, k, v):
        k, v = k.copy(), v.copy()
        kf, vf = _bits_to_f32(k), _bits_to_f32(v)
        for b in range(w.num_seqs):
            pg, sl = _token_slots(w, b)
            for i in range(pg.size):
                ek, ev = rng.integers(0, 13, 2)
                k[pg[i], :, :, sl[i], :] = _f32_to_bits(kf[pg[i], :, :, sl[i], :] * np.float32(2.0 ** (int(ek) - 6)))
                v[pg[i], :, :, sl[i]] = _f32_to_bits(vf[pg[i], :, :, sl[i]] * np.float32(2.0 ** int(ev)))
        return k, v

    dev = device()
    case = _case(d, hq, hkv, 900 + d, dev, edit)
    scale = float(case.w.scale)
    out = case.run(scale)
    ref = case.oracle(scale)
    worst_a = worst_r = 0.0
    for b in range(case.w.num_seqs):
        pg, sl = _token_slots(case.w, b)
        vmax = float(np.abs(_bits_to_f32(case.v_bits[pg, :, :, sl])).max()) if pg.size else 1.0
        div = 2.0 ** np.ceil(np.log2(max(vmax, 1.0)))
        a, r = check_parity(out[b] / div, ref[b] / div, f"large magnitudes d={d} seq {b} (/ {div:g})")
        worst_a, worst_r = max(worst_a, a), max(worst_r, r)
    log(f"large magnitudes d={d}: max |ref| {np.abs(ref).max():.3g}; normalised max abs {worst_a:.2e} "
        f"max rel {worst_r:.2e}")
