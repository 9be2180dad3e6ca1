"""The C ABI from a plain C program (tests/c_client/pakv_client.c): the
scheduler admits three requests over a page pool, their prompts are
prefilled, then five decode steps append a token per request and attend
(layer 0 through a host launch plan, layer 1 through pa_decode), all without
Python or torch in the loop. Every output, and the final pool bit for bit,
is checked against the oracle replaying the same sequence of operations on
the block tables the program used."""

import os
import subprocess

import numpy as np
import pytest

import oracle
from gpu_helpers import check_parity, log
from oracle_pins import random_bf16

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "pakv_client")
NAN = 0x7FC0


@pytest.mark.parametrize("d,hq,hkv", [(64, 32, 8), (128, 28, 4)])
def test_c_client_serving_run(tmp_path, d, hq, hkv):
    assert os.path.exists(CLIENT), f"{CLIENT} is not built (run __graft_entry__.build())"
    P, L, MB, stride, steps = 96, 2, 4, 24, 5
    reqs = [(37, 8), (70, 6), (5, 9)]                  # (prompt, max new tokens), slots 0, 1, 2
    rng = np.random.default_rng(4321 + d)
    scale = float(np.float32(1.0) / np.sqrt(np.float32(d)))
    k_pool = np.full((P, hkv, d // 32, 16, 32), NAN, np.uint16)
    v_pool = np.full((P, hkv, d, 16), NAN, np.uint16)
    out_dir = str(tmp_path)
    put = lambda name, a: np.ascontiguousarray(a).tofile(os.path.join(out_dir, name))
    get = lambda name, dt, shape: np.fromfile(os.path.join(out_dir, name), dtype=dt).reshape(shape)
    with open(os.path.join(out_dir, "config.txt"), "w") as f:
        f.write(f"{P} {hkv} {hq} {d} {L} {MB} {stride} {steps} {len(reqs)}\n")
        for p, n in reqs:
            f.write(f"{p} {n}\n")
    put("k_pool.bin", k_pool)
    put("v_pool.bin", v_pool)
    N = sum(p for p, _ in reqs)
    pre = {}
    for l in range(L):
        pre[l] = (random_bf16(rng, (N, hq, d)), random_bf16(rng, (N, hkv, d)), random_bf16(rng, (N, hkv, d)))
        for name, a in zip(("q", "k", "v"), pre[l]):
            put(f"prefill_{name}_{l}.bin", a)
    dec = {}
    for s in range(steps):
        for l in range(L):
            dec[s, l] = (random_bf16(rng, (MB, hq, d)), random_bf16(rng, (MB, hkv, d)),
                         random_bf16(rng, (MB, hkv, d)))
            for name, a in zip(("q", "k", "v"), dec[s, l]):
                put(f"step{s}_{name}_{l}.bin", a)

    log(f"c client: d={d} Hq={hq} Hkv={hkv} requests={reqs} steps={steps}")
    res = subprocess.run([CLIENT, out_dir], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"pakv_client failed ({res.returncode}): {res.stderr}{res.stdout}"
    log(res.stdout.strip())

    # the oracle replays the run on the block tables the program used
    qs = np.concatenate([[0], np.cumsum([p for p, _ in reqs] + [0] * (MB - len(reqs)))]).astype(np.int64)
    bt_all = get("bt_prefill.bin", np.int32, (L, MB, stride))
    before = get("ctx_prefill.bin", np.int32, (MB,))
    assert not before.any()
    k_host, v_host = k_pool, v_pool
    checked = 0
    for l in range(L):
        q, kr, vr = pre[l]
        bt = np.where(bt_all[l] < 0, 0, bt_all[l])
        ref, k_host, v_host = oracle.prefill_attention(q, k_host, v_host, kr, vr, qs, bt, before, scale)
        check_parity(get(f"prefill_out_{l}.bin", np.float32, (N, hq, d)), ref, f"c client prefill layer {l}")
        checked += 1
    for s in range(steps):
        bt_all = get(f"bt_step{s}.bin", np.int32, (L, MB, stride))
        pos = get(f"pos_step{s}.bin", np.int32, (MB,))
        ctx = get(f"ctx_step{s}.bin", np.int32, (MB,))
        for l in range(L):
            _, kn, vn = dec[s, l]
            k_host, v_host = oracle.kv_append(k_host, v_host, kn, vn, np.where(bt_all[l] < 0, 0, bt_all[l]), pos)
        for l in range(L):
            ref = oracle.decode_attention(dec[s, l][0], k_host, v_host, np.where(bt_all[l] < 0, 0, bt_all[l]),
                                          ctx, scale)
            check_parity(get(f"step{s}_out_{l}.bin", np.float32, (MB, hq, d)), ref, f"c client step {s} layer {l}")
            checked += 1
    assert np.array_equal(get("k_final.bin", np.uint16, k_pool.shape), k_host), "K pool differs"
    assert np.array_equal(get("v_final.bin", np.uint16, v_pool.shape), v_host), "V pool differs"
    log(f"c client d={d}: {checked} launches checked, pools bit-exact")
