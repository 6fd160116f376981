"""Decode steps captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every replay advances the positions in the device's head records while the
host's copy stays where the capture left it.  Checked here, against the oracle:
every replay's outputs (with eager work and synchronisations between replays);
an extend call and eager decode steps made after the replays, which must take
their positions from the device; and replays or an extend that run past
max_positions, which the kernels must catch (sticky DMS_E_STATE, tokens
dropped, the store unchanged)."""
import numpy as np
import pytest

import oracle
from dms_case import Case, Runner, assert_close, from_dev_bf16, to_dev

pytestmark = pytest.mark.gpu


def capture_step(r, layer0, n_layers):
    """A graph of one dms_decode_step over layers layer0 .. layer0+n_layers-1 of
    sequence 0, reading static input buffers; returns (graph, buffers)."""
    torch, c = r.torch, r.case
    q, k, v, lg = r.step_inputs(0, [0], list(range(layer0, layer0 + n_layers)))
    bufs = {"q": q.clone(), "k": k.clone(), "v": v.clone(), "lg": lg.clone(),
            "out": torch.empty((n_layers, 1, c.n_q_heads, c.head_dim), dtype=torch.bfloat16, device="cuda")}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            r.pool.decode_step([0], layer0, bufs["q"], bufs["k"], bufs["v"], bufs["lg"], bufs["out"])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g, bufs


def replay(r, g, bufs, i, layer0, n_layers):
    q, k, v, lg = r.step_inputs(i, [0], list(range(layer0, layer0 + n_layers)))
    bufs["q"].copy_(q)
    bufs["k"].copy_(k)
    bufs["v"].copy_(v)
    bufs["lg"].copy_(lg)
    g.replay()
    r.torch.cuda.synchronize()
    return from_dev_bf16(bufs["out"])


@pytest.mark.parametrize("kv_format", [0, 1])
def test_graph_replays_then_extend_and_decode(kv_format):
    """Layer 0 is stepped by replays of a captured one-layer step, then extended
    by a chunk; layer 1 by eager steps.  Every output and live set matches."""
    n_rep, chunk = 9, 37
    case = Case(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, window=16, ctx_lens=[150],
                steps=n_rep + chunk + 3, seed=77, kv_format=kv_format)
    case.gen()
    r = Runner(case)
    torch = r.torch
    try:
        r.prefill_all()
        ctx = case.ctx_lens[0]
        g, bufs = capture_step(r, 0, 1)  # nothing runs during capture
        for i in range(n_rep):
            out = replay(r, g, bufs, i, 0, 1)
            r.check_outputs(out, i, layer0=0, record="decode graph replays")
            torch.zeros(1024, device="cuda").sum().item()  # eager work between replays
            e1 = r.decode(i, layer0=1, n_layers=1)
            r.check_outputs(e1, i, layer0=1)
        # layer 0: a chunk at the device's position ctx + n_rep (the host's copy is behind)
        d = case.data[(0, 0)]
        t0 = ctx + n_rep
        rows = slice(t0, t0 + chunk)
        out = torch.empty((chunk, case.n_q_heads, case.head_dim), dtype=torch.bfloat16, device="cuda")
        r.pool.extend(0, 0, to_dev(d.k[rows], torch, torch.bfloat16), to_dev(d.v[rows], torch, torch.bfloat16),
                      to_dev(d.logits[rows], torch, torch.float32), q=to_dev(d.q[rows], torch, torch.bfloat16),
                      out=out)
        ref = np.stack([case.oracle_out(0, 0, t) for t in range(t0, t0 + chunk)])
        assert_close(from_dev_bf16(out), ref, "extend after graph replays", record="extend after graph replays")
        for h in range(case.n_kv_heads):
            assert np.array_equal(r.pool.export_live(0, 0, h), case.oracle_live(0, 0, h, t0 + chunk - 1)), h
            assert np.array_equal(r.pool.export_live(0, 1, h), case.oracle_live(0, 1, h, ctx + n_rep - 1)), h
        st, _ = r.pool.stats(0)
        assert st.device_error == 0 and st.position == t0 + chunk
        # eager decode of layer 0 after the chunk (host copy refreshed by stats)
        i = n_rep + chunk
        o = r.decode(i, layer0=0, n_layers=1)
        r.check_outputs(o, i, layer0=0)
        for h in range(case.n_kv_heads):
            pos, k, v, ks, vs = r.pool.export_kv(0, 0, h)
            assert np.array_equal(pos, case.oracle_live(0, 0, h, ctx + i)), h
            if kv_format:
                k8, kss, v8, vss = case.quantized(0, 0)
                assert np.array_equal(k, k8[pos, h]) and np.array_equal(v, v8[pos, h])
                assert np.array_equal(ks, kss[pos, h]) and np.array_equal(vs, vss[pos, h])
            else:
                assert np.array_equal(k, d.k[pos, h]) and np.array_equal(v, d.v[pos, h])
    finally:
        r.close()


def test_replays_past_max_positions_are_dropped_on_the_device():
    """max_positions = prompt + 4: of 7 replays the last 3 find the record at the
    limit; their tokens are dropped and the sticky flag reports DMS_E_STATE."""
    import compact_decode_attention_amd as dms
    case = Case(n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=64, window=8, ctx_lens=[100], steps=7, seed=5,
                max_positions=104)
    case.gen()
    r = Runner(case)
    try:
        r.prefill_all()
        g, bufs = capture_step(r, 0, 1)
        for i in range(4):
            r.check_outputs(replay(r, g, bufs, i, 0, 1), i)
        for i in range(4, 7):
            replay(r, g, bufs, i, 0, 1)
        st, _ = r.pool.stats(0, raise_on_error=False)
        assert st.device_error == dms.DMS_E_STATE
        assert st.position == 104
        for h in range(2):
            assert np.array_equal(r.pool.export_live(0, 0, h), case.oracle_live(0, 0, h, 103))
        with pytest.raises(dms.DMSError) as e:
            r.pool.stats(0)
        assert e.value.status == dms.DMS_E_STATE
    finally:
        r.close()


def test_extend_past_max_positions_after_replays_is_dropped_on_the_device():
    """After 6 replays the host still counts the prompt only, so an 8-token
    extend passes its check; the device finds 100 + 6 + 8 > 110 and stores
    nothing."""
    import compact_decode_attention_amd as dms
    case = Case(n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=64, window=8, ctx_lens=[100], steps=14, seed=6,
                max_positions=110)
    case.gen()
    r = Runner(case)
    torch = r.torch
    try:
        r.prefill_all()
        g, bufs = capture_step(r, 0, 1)
        for i in range(6):
            r.check_outputs(replay(r, g, bufs, i, 0, 1), i)
        d = case.data[(0, 0)]
        rows = slice(106, 114)
        r.pool.extend(0, 0, to_dev(d.k[rows], torch, torch.bfloat16), to_dev(d.v[rows], torch, torch.bfloat16),
                      to_dev(d.logits[rows], torch, torch.float32))
        st, _ = r.pool.stats(0, raise_on_error=False)
        assert st.device_error == dms.DMS_E_STATE and st.position == 106
        for h in range(2):
            pos, k, v, _, _ = r.pool.export_kv(0, 0, h)
            ref = case.oracle_live(0, 0, h, 105)
            assert np.array_equal(pos, ref)
            assert np.array_equal(k, d.k[ref, h]) and np.array_equal(v, d.v[ref, h])
    finally:
        r.close()
