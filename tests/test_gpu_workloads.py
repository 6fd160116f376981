"""GPU parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (one dms_decode_step per token over all layers): sampled decode
steps checked against the oracle on every layer and q head, every live set and
count checked exactly at the end."""
import numpy as np
import pytest

import oracle
import synth
from dms_case import assert_close

pytestmark = pytest.mark.gpu


def bf(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def run_workload(name, steps, check_steps, per_layer_steps=()):
    import torch
    import compact_decode_attention_amd as dms
    wl = synth.WORKLOADS[name]
    inp = synth.SynthInputs(wl)
    L, Hq, H, D, w = wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    ctx = int(inp.ctx_lens()[0])
    total = ctx + steps
    dev = torch.device("cuda:0")
    K, V, LG = [], [], []
    for l in range(L):
        K.append(inp.k(0, l, 0, total))
        V.append(inp.v(0, l, 0, total))
        LG.append(inp.logits(0, l, 0, total))
    Q = np.stack([inp.q(0, l, ctx, steps) for l in range(L)], axis=1)   # [steps][L][Hq][D]
    pool = dms.Pool(n_layers=L, n_q_heads=Hq, n_kv_heads=H, head_dim=D, window=w, max_seqs=1,
                    max_positions=total, max_pages=L * H * ((total + 63) // 64), device=dev)
    for l in range(L):
        pool.prefill(0, l, bf(K[l][:ctx], torch).to(dev), bf(V[l][:ctx], torch).to(dev),
                     torch.from_numpy(LG[l][:ctx]).to(dev))
    marks = [oracle.marks(LG[l]) for l in range(L)]
    worst = 0.0
    for i in range(steps):
        t = ctx + i
        q = bf(Q[i], torch).to(dev).view(L, 1, Hq, D)
        k = bf(np.stack([K[l][t] for l in range(L)]), torch).to(dev).view(L, 1, H, D)
        v = bf(np.stack([V[l][t] for l in range(L)]), torch).to(dev).view(L, 1, H, D)
        lg = torch.from_numpy(np.stack([LG[l][t] for l in range(L)])).to(dev).view(L, 1, H)
        out = torch.empty((L, 1, Hq, D), dtype=torch.bfloat16, device=dev)
        if i in per_layer_steps:
            for l in range(L):
                pool.decode_step([0], l, q[l:l + 1], k[l:l + 1], v[l:l + 1], lg[l:l + 1], out[l:l + 1])
        else:
            pool.decode_step([0], 0, q, k, v, lg, out)
        if i in check_steps:
            got = out.view(torch.int16).cpu().numpy().view(np.uint16)
            for l in range(L):
                ref = oracle.attend(Q[i, l][None], [t], K[l][:t + 1], V[l][:t + 1], marks[l][:t + 1], w)[0]
                e = assert_close(got[l, 0], ref, "%s step %d layer %d" % (name, i, l))
                worst = max(worst, e[0])
    st, live = pool.stats(0, per_head=True)
    assert st.position == total and st.device_error == 0
    for l in range(L):
        for h in range(H):
            ref = oracle.live_positions(total - 1, w, marks[l][:, h])
            assert live[l, h] == len(ref)
            assert np.array_equal(pool.export_live(0, l, h), ref), (l, h)
    assert st.live_slots == sum(len(oracle.live_positions(total - 1, w, marks[l][:, h]))
                                for l in range(L) for h in range(H))
    assert st.kv_bytes_live == st.live_slots * 2 * D * 2
    pool.close()
    return worst


def test_qwen3_8b_ctx8192_full_size():
    """36 layers, 32 q / 8 kv heads, D=128, ctx 8192, 128 steps, w=512."""
    run_workload("qwen3-8b_ctx8192", steps=128, check_steps={0, 1, 2, 63, 64, 126, 127},
                 per_layer_steps={5, 6})


def test_llama32_1b_ctx8192_full_size():
    """16 layers, 32 q / 8 kv heads, D=64, ctx 8192, 128 steps, w=512."""
    run_workload("llama3.2-1b_ctx8192", steps=128, check_steps={0, 1, 50, 127}, per_layer_steps={7})


def test_tiny_workload_every_step():
    """1 layer, D=64, ctx 1024, 16 steps, w=256: every step checked."""
    run_workload("tiny_d64_ctx1024", steps=16, check_steps=set(range(16)))
