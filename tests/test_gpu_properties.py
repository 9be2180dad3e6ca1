"""GPU properties of the HIP path that hold at any size: bitwise determinism,
batch invariance, placement invariance, shared pages, exact one-token output,
bit-exact append that touches nothing else, the generator on the GPU, and the
error paths of the C ABI."""

import numpy as np
import pytest

import oracle
from gpu_helpers import Uploaded, check_parity, device, log
from paged_kv_decode_02_amd import binding as B
from paged_kv_decode_02_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_generator_on_gpu_matches_host():
    import torch
    dev = device()
    w = W.custom(seed=2, ctx_lens=[5, 40, 100], num_q_heads=28, num_kv_heads=4, head_dim=128)
    log("generator k/v pools on cuda:0 vs host")
    for which in "kv":
        g = w.pool_device(which, dev, chunk_elems=1 << 14).cpu().numpy().view(np.uint16)
        assert np.array_equal(g, w.pool_bits(which))
    torch.cuda.synchronize()


def test_determinism_ten_runs():
    dev = device()
    w = W.make_workload("c3")
    log("determinism: c3 x10, entry=pa_decode")
    up = Uploaded(w, dev)
    first = up.step().clone()
    for _ in range(9):
        again = up.step()
        assert bool((again == first).all()), "decode output changed between identical runs"


def test_batch_invariance_bitwise():
    """A sequence's output bits do not depend on the batch around it, with or
    without a launch plan (which packs different sequences into one
    workgroup depending on the batch): one-split, whole-in-workgroup
    (2..4 splits) and merge-kernel (5+ splits) sequences."""
    import torch
    dev = device()
    ctx = [700, 5, 1500, 33, 0, 260, 5000, 9000, 2049]
    w = W.custom(seed=8, ctx_lens=ctx)
    log(f"batch invariance ctx={ctx}")
    up = Uploaded(w, dev)
    full = up.step()[0].clone()
    planned = up.step(fused=False, planned=True)[0].clone()
    assert bool((planned == full).all()), "planned batch differs from the plain batch"

    def run(idx, plan):
        ix = torch.tensor(idx, device=dev)
        q, bt, c = up.q[0][ix].contiguous(), up.bt[0][ix].contiguous(), up.ctx[ix].contiguous()
        if not plan:
            return B.decode(up.pool, q, bt, c, float(w.scale))
        p = torch.from_numpy(B.decode_plan(up.pool, w.ctx_lens[idx], w.num_q_heads, w.stride)).to(dev)
        return B.decode_planned(up.pool, q, bt, c, float(w.scale), p)

    for plan in (False, True):
        for b in range(len(ctx)):
            out = run([b], plan)
            assert bool((out[0] == full[b]).all()), f"sequence {b} differs alone vs in the batch (plan={plan})"
        # and inside bigger, different batches
        for idx in ([3, 2, 2, 0], [7, 1, 6, 6, 3, 8, 0, 5], [8, 7, 6, 5, 4, 3, 2, 1, 0, 7, 2]):
            out = run(idx, plan)
            assert bool((out == full[torch.tensor(idx, device=dev)]).all()), f"batch {idx} (plan={plan})"


def test_page_permutation_invariance_bitwise():
    import torch
    dev = device()
    w = W.custom(seed=9, ctx_lens=[900, 17, 1200], num_q_heads=28, num_kv_heads=4, head_dim=128)
    log("page permutation invariance d=128")
    up = Uploaded(w, dev)
    base = up.step()[0].clone()
    perm = torch.from_numpy(np.random.default_rng(1).permutation(w.num_pages)).to(dev)
    k2 = torch.empty_like(up.k_pool)
    v2 = torch.empty_like(up.v_pool)
    k2[perm] = up.k_pool
    v2[perm] = up.v_pool
    pool2 = B.Pool(k2, v2)
    bt2 = perm.to(torch.int32)[up.bt[0].long()].contiguous()
    out = B.decode(pool2, up.q[0], bt2, up.ctx, float(w.scale))
    assert bool((out == base).all()), "moving pages changed the output"


def test_shared_pages_across_sequences():
    """Two block tables naming the same pages (a shared prefix) read them read-only."""
    import torch
    dev = device()
    w = W.custom(seed=10, ctx_lens=[640, 640], num_q_heads=32, num_kv_heads=8, head_dim=64)
    log("shared pages")
    up = Uploaded(w, dev)
    bt = up.bt[0].clone()
    bt[1, :20] = bt[0, :20]                  # first 320 tokens shared
    q = up.q[0].clone()
    out = B.decode(up.pool, q, bt, up.ctx, float(w.scale)).cpu().numpy()
    ref = oracle.decode_attention(up.q_host[0], w.pool_bits("k"), w.pool_bits("v"),
                                  bt.cpu().numpy(), w.ctx_lens, w.scale)
    check_parity(out, ref, "shared pages")


def test_one_token_returns_value_row_exactly():
    dev = device()
    for d, hq, hkv in [(64, 32, 8), (128, 28, 4)]:
        w = W.custom(seed=11, ctx_lens=[1, 1, 1], num_q_heads=hq, num_kv_heads=hkv, head_dim=d)
        log(f"ctx=1 exact d={d}")
        up = Uploaded(w, dev)
        out = up.step()[0].cpu().numpy()
        v = w.pool_bits("v")
        for b in range(3):
            p = int(w.block_tables[0, b, 0])
            for h in range(hq):
                row = oracle.bf16_bits_to_f64(v[p, h // (hq // hkv), :, 0])
                assert np.array_equal(out[b, h].astype(np.float64), row), (d, b, h)


def test_append_bit_exact_and_nothing_else_changes():
    import torch
    dev = device()
    for d, hq, hkv in [(64, 32, 8), (128, 28, 4)]:
        ctx = [1, 16, 17, 40, 300, 33]
        w = W.custom(seed=12, ctx_lens=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                     append=True, extra_pages=5)
        log(f"append d={d} positions={list(w.positions)} entry=pa_kv_append")
        up = Uploaded(w, dev)
        k0, v0 = w.pool_bits("k"), w.pool_bits("v")
        pos = w.positions.copy()
        pos[2] = -1                                     # skipped
        pos_t = torch.from_numpy(pos).to(dev)
        B.kv_append(up.pool, up.k_new[0], up.v_new[0], up.bt[0], pos_t)
        k1 = up.k_pool.cpu().numpy().view(np.uint16)
        v1 = up.v_pool.cpu().numpy().view(np.uint16)
        ek, ev = oracle.kv_append(k0, v0, up.k_new_host[0], up.v_new_host[0], w.block_tables[0], pos)
        assert np.array_equal(k1, ek), "K pool differs from the oracle's append"
        assert np.array_equal(v1, ev), "V pool differs from the oracle's append"
        # decode after append matches the oracle over ctx tokens (skipped seq: ctx - 1)
        ctx_eff = w.ctx_lens.copy()
        ctx_eff[2] -= 1
        ctx_t = torch.from_numpy(ctx_eff).to(dev)
        out = B.decode(up.pool, up.q[0], up.bt[0], ctx_t, float(w.scale)).cpu().numpy()
        ref = oracle.decode_attention(up.q_host[0], ek, ev, w.block_tables[0], ctx_eff, w.scale)
        check_parity(out, ref, f"decode after append d={d}")


def test_fused_append_equals_separate_calls():
    """pa_decode_append leaves the same pool bits and the same output bits as
    pa_kv_append followed by pa_decode, for positions inside and past the
    decoded context and for skipped sequences."""
    import torch
    dev = device()
    for d, hq, hkv in [(64, 32, 8), (128, 28, 4)]:
        ctx = [1, 16, 17, 1024, 1025, 2100, 40, 1000, 70]
        w = W.custom(seed=15, ctx_lens=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                     append=True, extra_pages=6)
        log(f"fused vs separate d={d} ctx={ctx} entry=pa_decode_append")
        pos = w.positions.copy()
        pos[6] = -1                      # skipped
        pos[2] = 3                       # rewrites a token inside the context
        pos[7] = 5                       # early in a long context (not the last pair of its wave)
        pos[8] = 90                      # past the decoded context (written, not attended)
        pos_t = torch.from_numpy(pos).to(dev)
        ctx_eff = w.ctx_lens.copy()
        ctx_eff[6] -= 1                  # its last slot is never written
        ctx_eff[2] = 16                  # its slot 16 is never written; token 3 is rewritten
        ctx_eff[7] = 999                 # slot 999 never written
        ctx_eff[8] = 69                  # slot 69 never written; 90 is written but not read
        ctx_t = torch.from_numpy(ctx_eff).to(dev)
        a = Uploaded(w, dev)
        B.kv_append(a.pool, a.k_new[0], a.v_new[0], a.bt[0], pos_t)
        out_a = B.decode(a.pool, a.q[0], a.bt[0], ctx_t, float(w.scale))
        b = Uploaded(w, dev)
        out_b = B.decode_append(b.pool, b.q[0], b.k_new[0], b.v_new[0], pos_t, b.bt[0], ctx_t,
                                float(w.scale))
        assert bool((a.k_pool == b.k_pool).all()) and bool((a.v_pool == b.v_pool).all())
        assert bool((out_a.view(torch.int32) == out_b.view(torch.int32)).all()), \
            "fused output differs from the two-call output"
        ek, ev = oracle.kv_append(w.pool_bits("k"), w.pool_bits("v"), b.k_new_host[0], b.v_new_host[0],
                                  w.block_tables[0], pos)
        assert np.array_equal(b.k_pool.cpu().numpy().view(np.uint16), ek)
        assert np.array_equal(b.v_pool.cpu().numpy().view(np.uint16), ev)
        ref = oracle.decode_attention(b.q_host[0], ek, ev, w.block_tables[0], ctx_eff, w.scale)
        check_parity(out_b.cpu().numpy(), ref, f"fused d={d}")


def test_out_of_range_inputs_stay_in_bounds():
    """Page ids outside the pool and over-long contexts are clamped (no fault);
    a position past the table or a bad page id makes the append skip."""
    import torch
    dev = device()
    w = W.custom(seed=13, ctx_lens=[40, 20], num_q_heads=32, num_kv_heads=8, head_dim=64,
                 append=True)
    up = Uploaded(w, dev)
    log("clamped inputs")
    bt = up.bt[0].clone()
    bt[0, 1] = w.num_pages + 1000
    bt[1, 0] = -5
    ctx = torch.tensor([10**6, 20], dtype=torch.int32, device=dev)
    out = B.decode(up.pool, up.q[0], bt, ctx, float(w.scale))
    torch.cuda.synchronize()
    assert out.shape == (2, 32, 64)
    k_before = up.k_pool.clone()
    pos = torch.tensor([w.stride * 16, 0], dtype=torch.int32, device=dev)
    B.kv_append(up.pool, up.k_new[0], up.v_new[0], bt, pos)     # seq 0: past the table; seq 1: page -5
    torch.cuda.synchronize()
    assert bool((up.k_pool == k_before).all())


def test_error_paths_on_gpu():
    import torch
    dev = device()
    w = W.custom(seed=14, ctx_lens=[9000, 700])         # 5 splits of 2048: needs the workspace
    up = Uploaded(w, dev)
    log("error paths")
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(B.PakvError) as e:
        B.decode(up.pool, up.q[0], up.bt[0], up.ctx, 0.125, workspace=small)
    assert e.value.status == 5
    # the C ABI itself refuses a query-head count that is not a multiple of the KV heads
    q12 = up.q[0][:, :12].contiguous()
    st = B.lib().pa_decode(up.pool.handle, q12.data_ptr(), 2, 12, up.bt[0].data_ptr(), w.stride,
                           up.ctx.data_ptr(), 0.125, up.out[0].data_ptr(), up.workspace.data_ptr(),
                           up.workspace.numel(), None)
    assert st == 2
    # and a scale whose log2(e) multiple is not finite in FP32
    st = B.lib().pa_decode(up.pool.handle, up.q[0].data_ptr(), 2, 32, up.bt[0].data_ptr(), w.stride,
                           up.ctx.data_ptr(), 3.0e38, up.out[0].data_ptr(), up.workspace.data_ptr(),
                           up.workspace.numel(), None)
    assert st == 2


def test_binding_rejects_mismatched_shapes():
    """Every tensor is checked against the pool and the batch before anything
    is queued: a wrong shape raises ValueError and leaves the pool and the
    output untouched."""
    import torch
    dev = device()
    w = W.custom(seed=16, ctx_lens=[300, 40, 9], append=True)
    up = Uploaded(w, dev)
    log("binding shape checks")
    q, bt, ctx, kn, vn, pos = up.q[0], up.bt[0], up.ctx, up.k_new[0], up.v_new[0], up.pos
    out = torch.full((3, 32, 64), 7.0, device=dev)
    k0, v0 = up.k_pool.clone(), up.v_pool.clone()
    bad_decode = [
        dict(q=q[:2].contiguous()),                                   # 2 queries, 3 table rows
        dict(bt=bt[:2].contiguous()),                                 # 2 table rows
        dict(ctx=ctx[:2].contiguous()),                               # 2 context lengths
        dict(out=torch.empty((3, 32, 32), device=dev)),               # wrong output shape
        dict(q=torch.zeros((3, 32, 128), dtype=torch.int16, device=dev)),   # head_dim 128 on a d=64 pool
        dict(q=torch.zeros((3, 12, 64), dtype=torch.int16, device=dev)),    # 12 heads over 8 KV heads
    ]
    for bad in bad_decode:
        args = dict(q=q, bt=bt, ctx=ctx, out=out)
        args.update(bad)
        with pytest.raises(ValueError):
            B.decode(up.pool, args["q"], args["bt"], args["ctx"], 0.125, out=args["out"])
        plan = torch.from_numpy(B.decode_plan(up.pool, w.ctx_lens, w.num_q_heads, w.stride)).to(dev)
        with pytest.raises(ValueError):
            B.decode_planned(up.pool, args["q"], args["bt"], args["ctx"], 0.125, plan, out=args["out"])
        with pytest.raises(ValueError):
            B.decode_planned_host(up.pool, args["q"], args["bt"], args["ctx"], 0.125, plan.cpu().numpy(),
                                  out=args["out"])
    bad_rows = [
        dict(kn=kn[:2].contiguous()),
        dict(vn=torch.zeros((3, 8, 32), dtype=torch.int16, device=dev)),
        dict(pos=pos[:1].contiguous()),
        dict(kn=torch.zeros((3, 4, 64), dtype=torch.int16, device=dev)),
    ]
    for bad in bad_rows:
        args = dict(kn=kn, vn=vn, pos=pos)
        args.update(bad)
        with pytest.raises(ValueError):
            B.kv_append(up.pool, args["kn"], args["vn"], bt, args["pos"])
        with pytest.raises(ValueError):
            B.decode_append(up.pool, q, args["kn"], args["vn"], args["pos"], bt, ctx, 0.125, out=out)
    # chunk rows for prefill / chunk write
    qs = torch.tensor([0, 2, 3, 3], dtype=torch.int32, device=dev)
    rows_k = torch.zeros((3, 8, 64), dtype=torch.int16, device=dev)
    with pytest.raises(ValueError):
        B.kv_write(up.pool, rows_k[:2].contiguous(), rows_k, qs, bt, ctx, 2)
    with pytest.raises(ValueError):
        B.prefill(up.pool, torch.zeros((3, 32, 64), dtype=torch.int16, device=dev), rows_k,
                  torch.zeros((3, 8, 128), dtype=torch.int16, device=dev), qs, bt, ctx, 0.125, 2)
    with pytest.raises(ValueError):
        B.prefill(up.pool, torch.zeros((3, 32, 64), dtype=torch.int16, device=dev), rows_k, rows_k,
                  qs, bt, ctx, 0.125, 2, out=torch.empty((3, 32, 32), device=dev))
    torch.cuda.synchronize()
    assert bool((up.k_pool == k0).all()) and bool((up.v_pool == v0).all())
    assert bool((out == 7.0).all())


def test_stream_read_helper():
    import torch
    dev = device()
    buf = torch.ones(1 << 20, dtype=torch.int32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    B.stream_read(buf, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0


@pytest.mark.parametrize("case", ["custom", "c3", "c5"])
def test_planned_decode_is_bitwise_plain_decode(case):
    import torch
    dev = device()
    if case == "custom":
        ctx = [0, 1, 16, 17, 1024, 1025, 3000, 40, 2049, 0, 777]
        w = W.custom(seed=21, ctx_lens=ctx, stride=200)
    else:
        w = W.make_workload(case)
    log(f"planned decode vs pa_decode: {case}, {w.num_seqs} seqs, d={w.head_dim}")
    up = Uploaded(w, dev)
    plain = up.step().clone()
    stride = w.block_tables.shape[-1]
    plan_host = B.decode_plan(up.pool, w.ctx_lens, w.num_q_heads, stride)
    # units out of range are skipped on the device: an item naming a sequence
    # past the batch and a split past the grid
    s_max = -(-stride // (B.split_tokens(w.head_dim) // 16))
    bogus = np.array([w.num_seqs + 5, (s_max << 20) | 0, -1, -1, 0, 0, 0, 0], dtype=np.int32)
    for extra in (np.zeros(0, np.int32), bogus):
        p = np.concatenate([plan_host, extra])
        if p.size > B.lib().pa_decode_plan_capacity(up.pool.handle, w.num_seqs, stride):
            continue
        plan = torch.from_numpy(p).to(dev)
        out = torch.full_like(plain[0], float("nan"))
        B.decode_planned(up.pool, up.q[0], up.bt[0], up.ctx, float(w.scale), plan, out=out,
                         workspace=up.workspace)
        torch.cuda.synchronize()
        assert bool((out == plain[0]).all()), f"{case}: planned decode differs from pa_decode"
        if p.size <= 2048:      # the same plan in the kernel's arguments
            out2 = torch.full_like(plain[0], float("nan"))
            B.decode_planned_host(up.pool, up.q[0], up.bt[0], up.ctx, float(w.scale), p, out=out2,
                                  workspace=up.workspace)
            torch.cuda.synchronize()
            assert bool((out2 == plain[0]).all()), f"{case}: host-planned decode differs from pa_decode"
    if case == "custom":
        ref = oracle.decode_attention(up.q_host[0], w.pool_bits("k"), w.pool_bits("v"),
                                      w.block_tables[0], w.ctx_lens, w.scale)
        check_parity(out.cpu().numpy(), ref, "planned decode vs oracle")


def test_plan_chains_guarded():
    """A plan whose items chain behind the bins' first items (300 sequences of
    at most 4 splits each, so every sequence is one item): with every chain
    link broken (pointing back at its own item, or backwards, or past the
    plan) each workgroup runs only its bin's first item and stops. The
    sequences of the first items then match pa_decode bit for bit and every
    other output row is left as it was (NaN)."""
    import torch
    dev = device()
    rng = np.random.default_rng(404)
    ctx = rng.integers(1, 4 * 2048 + 1, 300).astype(np.int32)
    w = W.custom(seed=31, ctx_lens=ctx.tolist(), stride=512)
    up = Uploaded(w, dev)
    plain = up.step().clone()[0]
    plan = B.decode_plan(up.pool, w.ctx_lens, w.num_q_heads, w.stride)
    items = plan.reshape(-1, 8)
    nb = min(len(items), 256 // w.num_kv_heads)
    assert len(items) > nb, "the plan must chain items"
    heads = set()
    for i in range(nb):
        heads.update(int(x) & 0xFFFFF for x in items[i, :4] if x >= 0)
    for how in ("self", "back", "past"):
        bad = items.copy()
        idx = np.arange(len(items))
        bad[:, 5] = {"self": idx, "back": np.maximum(idx - 1, 0), "past": len(items) + idx}[how]
        log(f"broken chain links ({how}): {len(items)} items, {nb} bins")
        for host in (False, True):
            out = torch.full_like(plain, float("nan"))
            if host:
                B.decode_planned_host(up.pool, up.q[0], up.bt[0], up.ctx, float(w.scale), bad.reshape(-1),
                                      out=out, workspace=up.workspace)
            else:
                B.decode_planned(up.pool, up.q[0], up.bt[0], up.ctx, float(w.scale),
                                 torch.from_numpy(bad.reshape(-1).copy()).to(dev), out=out,
                                 workspace=up.workspace)
            torch.cuda.synchronize()
            o, p = out.cpu().numpy(), plain.cpu().numpy()
            for b in range(w.num_seqs):
                if b in heads:
                    assert np.array_equal(o[b], p[b]), f"{how}: sequence {b} of a first item"
                else:
                    assert np.isnan(o[b]).all(), f"{how}: sequence {b} written past a broken link"
