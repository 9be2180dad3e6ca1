"""pa_decode_static (the allocation-free decode: split partials in the
library's static device scratch) against pa_decode, through the C ABI.

Two calls in a row, the second with a smaller input, both with sequences of
more splits than a workgroup merges itself, so that the scratch is written
and read: the outputs must equal pa_decode's bit for bit (the same kernels
and reduction order), and pass the decode parity bar against the FP64
oracle. A call whose partials would not fit the scratch is refused with
PA_ERR_WORKSPACE and writes nothing."""

import ctypes

import numpy as np
import pytest

import oracle
from gpu_helpers import Uploaded, check_parity, device, log
from paged_kv_decode_02_amd import binding as B
from paged_kv_decode_02_amd import workloads as W

pytestmark = pytest.mark.gpu


def _static(up, w, out):
    import torch
    st = B.lib().pa_decode_static(up.pool.handle, up.q[0].data_ptr(), w.num_seqs, w.num_q_heads,
                                  up.bt[0].data_ptr(), w.stride, up.ctx.data_ptr(), ctypes.c_float(float(w.scale)),
                                  out.data_ptr(), None)
    torch.cuda.synchronize()
    return st


def test_static_scratch_matches_pa_decode_twice():
    import torch
    dev = device()
    cases = [
        # d = 128, G = 7: splits of 1024 tokens, more than 4 per sequence
        dict(seed=71, ctx_lens=[16384, 9000, 4097, 1, 12000, 700, 15000, 5000], num_q_heads=28,
             num_kv_heads=4, head_dim=128),
        # then smaller: d = 64, G = 4, splits of 2048 tokens
        dict(seed=72, ctx_lens=[9000, 700, 12000], num_q_heads=32, num_kv_heads=8, head_dim=64),
    ]
    for k, c in enumerate(cases):
        w = W.custom(name=f"static-{k}", **c)
        up = Uploaded(w, dev)
        need = B.decode_workspace_bytes(up.pool, w.num_seqs, w.num_q_heads, w.stride)
        log(f"pa_decode_static call {k}: ctx={c['ctx_lens']} d={w.head_dim} scratch need {need} bytes")
        assert need > 0, "the case must use the scratch"
        ref = B.decode(up.pool, up.q[0], up.bt[0], up.ctx, float(w.scale))
        out = torch.full_like(ref, float("nan"))
        assert _static(up, w, out) == B.PA_OK
        assert bool((out.view(torch.int32) == ref.view(torch.int32)).all()), f"call {k}: differs from pa_decode"
        exp = oracle.decode_attention(up.q_host[0], w.pool_bits("k"), w.pool_bits("v"), w.block_tables[0],
                                      w.ctx_lens, w.scale)
        a, r = check_parity(out.cpu().numpy(), exp, f"pa_decode_static call {k}")
        log(f"  bit-identical to pa_decode; vs oracle max abs {a:.2e} max rel {r:.2e}")


def test_static_scratch_refuses_oversize():
    import torch
    dev = device()
    w = W.custom(seed=73, ctx_lens=[1, 2], num_q_heads=32, num_kv_heads=8, head_dim=64)
    up = Uploaded(w, dev)
    L = B.lib()
    out = torch.full((600, 32, 64), 7.0, device=dev)
    # 600 sequences x 32 heads x 40 splits x (64 + 2) floats: ~200 MB of partials
    st = L.pa_decode_static(up.pool.handle, up.q[0].data_ptr(), 600, 32, up.bt[0].data_ptr(), 40 * 128,
                            up.ctx.data_ptr(), ctypes.c_float(0.125), out.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == B.PA_ERR_WORKSPACE
    assert bool((out == 7.0).all())
