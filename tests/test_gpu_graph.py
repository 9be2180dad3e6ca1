"""The decode step captured into a HIP graph (through torch) and replayed:
every replay, with the program's own eager work and synchronisations between
replays, matches the FP64 oracle within the parity bar, and gives the eager
step's output and pool bit for bit."""

import numpy as np
import pytest

from gpu_helpers import Uploaded, check_parity, device, full_oracle, log
from paged_kv_decode_02_amd import binding as B
from paged_kv_decode_02_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,hq,hkv", [(64, 32, 8), (128, 28, 4)])
def test_graph_replay_matches_eager(d, hq, hkv):
    import torch
    dev = device()
    ctx = [1, 17, 700, 1024, 1025, 2600, 90, 4100]
    w = W.custom(seed=31 + d, ctx_lens=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                 num_layers=3, append=True, stride=300)
    log(f"graph replay: d={d} layers=3 ctx={ctx} entry=pa_kv_append+pa_decode_planned")
    up = Uploaded(w, dev)
    eager = up.step(fused=False, planned=True).clone()
    k_eager, v_eager = up.k_pool.clone(), up.v_pool.clone()
    plan = torch.from_numpy(B.decode_plan(up.pool, w.ctx_lens, w.num_q_heads, w.stride)).to(dev)
    stream = torch.cuda.Stream()

    def layers(s):
        for layer in range(w.num_layers):
            B.kv_append(up.pool, up.k_new[layer], up.v_new[layer], up.bt[layer], up.pos, stream=s)
            B.decode_planned(up.pool, up.q[layer], up.bt[layer], up.ctx, float(w.scale), plan,
                             out=up.out[layer], workspace=up.workspace, stream=s)

    with torch.cuda.stream(stream):          # warm up on the capture stream
        layers(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        layers(stream)
    torch.cuda.synchronize()
    ref = full_oracle(w, up)
    scratch = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        up.out.fill_(float("nan"))
        scratch.mul_(1.0001).add_(0.5)        # eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        a, r = check_parity(up.out.cpu().numpy(), ref, f"graph replay {rep} vs oracle")
        assert bool((up.out == eager).all()), f"replay {rep}: output differs from the eager step"
        assert bool((up.k_pool == k_eager).all()) and bool((up.v_pool == v_eager).all()), \
            f"replay {rep}: pool differs from the eager step"
    log(f"graph replay d={d}: 4 replays within the bar of the oracle (last: max abs {a:.2e} "
        f"max rel {r:.2e}) and bitwise equal to eager")
