"""GPU parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times (one dms_decode_step per token over all layers): sampled decode
steps checked against the oracle on every layer and q head, every live set and
count checked exactly at the end."""
import numpy as np
import pytest

import oracle
import synth
from dms_case import ATOL, assert_close

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
                e = assert_close(got[l, 0], ref, "%s step %d layer %d" % (name, i, l), record=name, max_abs=ATOL)
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
    ref = np.sum([oracle.kv_bytes(total - 1, w, marks[l], D) for l in range(L)], axis=0)
    assert (st.kv_bytes_live, st.kv_bytes_allocated, st.kv_bytes_dense_equiv) == tuple(ref)
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


def test_qwen3_8b_batch32_ragged_full_size():
    """32 sequences with prompts U{4096..32768} in one shared page pool, 36 layers,
    64 decode steps, every step one call over all sequences and layers (split
    into several launches).  Eviction logits of every head come from the
    counter-based generator; K/V/q of 36 sampled (sequence, layer) pairs too
    (the shortest and longest prompt at the first and last layer, and one pair
    of every sequence at a layer spread over the stack), and their outputs are
    checked against the oracle at four steps; the other pairs take K/V/q
    from torch's seeded device generator.  Live counts of every head checked
    exactly, live sets on a sample."""
    import torch
    import compact_decode_attention_amd as dms
    wl = synth.WORKLOADS["qwen3-8b_batch32_ragged"]
    inp = synth.SynthInputs(wl)
    L, Hq, H, D, w, B, S = (wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window, wl.n_seqs,
                            wl.gen_len)
    ctx = [int(c) for c in inp.ctx_lens()]
    s_short, s_long = int(np.argmin(ctx)), int(np.argmax(ctx))
    sampled = [(s_short, 0), (s_short, L - 1), (s_long, 0), (s_long, L - 1)]
    sampled += [(s, (7 * s + 3) % L) for s in range(B) if (s, (7 * s + 3) % L) not in sampled]
    dev = torch.device("cuda:0")
    marks, pages = {}, 0
    for s in range(B):
        for l in range(L):
            mk = oracle.marks(inp.logits(s, l, 0, ctx[s] + S))
            marks[(s, l)] = mk
            pages += sum((oracle.live_count(ctx[s] + S - 1, w, mk[:, h]) + 63) // 64 for h in range(H))
    pool = dms.Pool(n_layers=L, n_q_heads=Hq, n_kv_heads=H, head_dim=D, window=w, max_seqs=B,
                    max_positions=max(ctx) + S, max_pages=pages, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    host = {}
    for s in range(B):
        for l in range(L):
            T = ctx[s]
            if (s, l) in sampled:
                K, V = inp.k(s, l, 0, T + S), inp.v(s, l, 0, T + S)
                host[(s, l)] = (K, V, inp.q(s, l, T, S))
                k, v = bf(K[:T], torch).to(dev), bf(V[:T], torch).to(dev)
            else:
                k = torch.randn((T, H, D), generator=gen, device=dev).to(torch.bfloat16)
                v = torch.randn((T, H, D), generator=gen, device=dev).to(torch.bfloat16)
            pool.prefill(s, l, k, v, torch.from_numpy(inp.logits(s, l, 0, T)).to(dev))
    seqs = list(range(B))
    check_steps = {0, S // 3, 2 * S // 3, S - 1}
    for i in range(S):
        q = torch.randn((L, B, Hq, D), generator=gen, device=dev).to(torch.bfloat16)
        k = torch.randn((L, B, H, D), generator=gen, device=dev).to(torch.bfloat16)
        v = torch.randn((L, B, H, D), generator=gen, device=dev).to(torch.bfloat16)
        for (s, l) in sampled:
            K, V, Q = host[(s, l)]
            t = ctx[s] + i
            q[l, s] = bf(Q[i], torch).to(dev)
            k[l, s] = bf(K[t], torch).to(dev)
            v[l, s] = bf(V[t], torch).to(dev)
        lg = torch.from_numpy(np.stack([np.stack([inp.logits(s, l, ctx[s] + i, 1)[0] for s in range(B)])
                                        for l in range(L)])).to(dev)
        out = torch.empty((L, B, Hq, D), dtype=torch.bfloat16, device=dev)
        pool.decode_step(seqs, 0, q, k, v, lg, out)
        if i in check_steps:
            got = out.view(torch.int16).cpu().numpy().view(np.uint16)
            for (s, l) in sampled:
                K, V, Q = host[(s, l)]
                t = ctx[s] + i
                ref = oracle.attend(Q[i][None], [t], K[:t + 1], V[:t + 1], marks[(s, l)][:t + 1], w)[0]
                assert_close(got[l, s], ref, "ragged step %d seq %d layer %d" % (i, s, l),
                             record="qwen3-8b_batch32_ragged (sampled)", max_abs=ATOL)
    st_all, _ = pool.stats()
    assert st_all.device_error == 0
    total_live = 0
    for s in range(B):
        t = ctx[s] + S - 1
        st, live = pool.stats(s, per_head=True)
        assert st.position == t + 1
        for l in range(L):
            ref = [oracle.live_count(t, w, marks[(s, l)][:t + 1, h]) for h in range(H)]
            assert np.array_equal(live[l], ref), (s, l)
            total_live += sum(ref)
    assert st_all.live_slots == total_live
    ref = np.sum([oracle.kv_bytes(ctx[s] + S - 1, w, marks[(s, l)], D) for s in range(B) for l in range(L)], axis=0)
    assert (st_all.kv_bytes_live, st_all.kv_bytes_allocated, st_all.kv_bytes_dense_equiv) == tuple(ref)
    rng = np.random.default_rng(3)
    heads = [(s, l, h) for (s, l) in sampled for h in range(H)]
    heads += [(int(rng.integers(B)), int(rng.integers(L)), int(rng.integers(H))) for _ in range(16)]
    for (s, l, h) in heads:
        t = ctx[s] + S - 1
        assert np.array_equal(pool.export_live(s, l, h), oracle.live_positions(t, w, marks[(s, l)][:t + 1, h]))
    pool.close()
