"""GPU parity of dms_extend (several new tokens of one (seq, layer) appended in
one call) against the oracle, through the C ABI.

After a prefill of ctx tokens, chunks of n tokens are appended.  Each chunk's
outputs (query t attends over the live set at t) are compared with the oracle's
masked attention at positions t .. t+n-1 over the full uncompressed K/V; after
each chunk the live sets and the stored rows are compared exactly; decode steps
after the chunks check that the window ring and the head record were left
right.  Chunk sizes around the window w make slots change hands several times
in one call (a token marked inside the chunk expiring inside it)."""
import numpy as np
import pytest

import oracle
import synth
from dms_case import assert_close

pytestmark = pytest.mark.gpu


def bf(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def make_inputs(T, Hq, Hkv, D, seed, marks):
    q = synth.normal_bf16(seed, synth.stream_id(synth.TAG_Q), 0, T * Hq * D).reshape(T, Hq, D)
    k = synth.normal_bf16(seed, synth.stream_id(synth.TAG_K), 0, T * Hkv * D).reshape(T, Hkv, D)
    v = synth.normal_bf16(seed, synth.stream_id(synth.TAG_V), 0, T * Hkv * D).reshape(T, Hkv, D)
    if marks == "all":
        lg = np.ones((T, Hkv), np.float32)
    elif marks == "none":
        lg = -np.ones((T, Hkv), np.float32)
    else:
        z = synth.normal_f32(seed, synth.stream_id(synth.TAG_SCORE), 0, T * Hkv).reshape(T, Hkv)
        lg = (-(-0.3 + z.astype(np.float64))).astype(np.float32)
    return q, k, v, lg


def run_extend(ctx, chunks, w, marks="random", G=4, D=128, Hkv=2, seed=5, kv_format=0, with_out=True,
               decode_steps=6, max_pages=None, softmax_scale=0.0):
    import torch
    import compact_decode_attention_amd as dms
    Hq = G * Hkv
    total = ctx + sum(chunks) + decode_steps
    q, k, v, lg = make_inputs(total, Hq, Hkv, D, seed, marks)
    mk = oracle.marks(lg)
    fp8 = kv_format == 1
    if fp8:
        k8, ks = oracle.quantize_rows(k)
        v8, vs = oracle.quantize_rows(v)

    def ref_out(t0, n):
        if fp8:
            return oracle.attend_fp8(q[t0:t0 + n], np.arange(t0, t0 + n), k8[:t0 + n], ks[:t0 + n], v8[:t0 + n],
                                     vs[:t0 + n], mk[:t0 + n], w, softmax_scale)
        return oracle.attend(q[t0:t0 + n], np.arange(t0, t0 + n), k[:t0 + n], v[:t0 + n], mk[:t0 + n], w,
                             softmax_scale)

    def check_store(t):
        for h in range(Hkv):
            pos, kc, vc, ksc, vsc = pool.export_kv(0, 0, h)
            assert np.array_equal(pos, oracle.live_positions(t, w, mk[:t + 1, h])), ("live set", t, h)
            if fp8:
                assert np.array_equal(kc, k8[pos, h]) and np.array_equal(vc, v8[pos, h])
                assert np.array_equal(ksc, ks[pos, h]) and np.array_equal(vsc, vs[pos, h])
            else:
                assert np.array_equal(kc, k[pos, h]) and np.array_equal(vc, v[pos, h]), ("stored rows", t, h)

    pool = dms.Pool(n_layers=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=total, max_pages=max_pages or Hkv * ((total + 63) // 64), kv_format=kv_format,
                    softmax_scale=softmax_scale)
    dev = "cuda"
    try:
        pool.prefill(0, 0, bf(k[:ctx], torch).to(dev), bf(v[:ctx], torch).to(dev), torch.from_numpy(lg[:ctx]).to(dev))
        t = ctx
        for n in chunks:
            out = torch.empty((n, Hq, D), dtype=torch.bfloat16, device=dev) if with_out else None
            pool.extend(0, 0, bf(k[t:t + n], torch).to(dev), bf(v[t:t + n], torch).to(dev),
                        torch.from_numpy(lg[t:t + n]).to(dev), q=bf(q[t:t + n], torch).to(dev) if with_out else None,
                        out=out)
            if with_out:
                got = out.view(torch.int16).cpu().numpy().view(np.uint16)
                assert_close(got, ref_out(t, n), "extend t0=%d n=%d w=%d marks=%s" % (t, n, w, marks),
                             record="extend (fp8 pool)" if fp8 else "extend")
            t += n
            check_store(t - 1)
        for i in range(decode_steps):
            o = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
            pool.decode_step([0], 0, bf(q[t], torch).to(dev).view(1, 1, Hq, D), bf(k[t], torch).to(dev).view(1, 1, Hkv, D),
                             bf(v[t], torch).to(dev).view(1, 1, Hkv, D), torch.from_numpy(lg[t]).to(dev).view(1, 1, Hkv), o)
            assert_close(o.view(torch.int16).cpu().numpy().view(np.uint16)[0, 0], ref_out(t, 1)[0],
                         "decode after extend t=%d" % t)
            t += 1
        check_store(t - 1)
        st, _ = pool.stats(0)
        assert st.position == t
    finally:
        pool.close()


@pytest.mark.parametrize("marks", ["random", "all", "none"])
@pytest.mark.parametrize("w", [1, 2, 16, 64])
@pytest.mark.parametrize("chunks", [[1], [2, 3], [15, 16, 17], [100], [200, 1, 64]])
def test_extend_chunks(chunks, w, marks):
    run_extend(150, chunks, w, marks, seed=len(chunks) * 7 + w)


@pytest.mark.parametrize("kv_format", [0, 1])
@pytest.mark.parametrize("scale", [0.02, 0.3])
def test_extend_softmax_scale(scale, kv_format):
    """A softmax scale other than 1/sqrt(head_dim) from the pool config, in the
    chunks' attention and the decode steps after them, on bf16 and FP8 pools."""
    run_extend(130, [40, 97], 24, seed=int(scale * 100) + 3, kv_format=kv_format, softmax_scale=scale)


def test_extend_eviction_disabled():
    run_extend(300, [70, 129], 1 << 20)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_extend_group_sizes(G, D):
    run_extend(257, [33, 96], 40, G=G, D=D, seed=G * 10 + D)


@pytest.mark.parametrize("w", [1, 8, 64])
def test_extend_fp8(w):
    run_extend(190, [1, 70, 130], w, kv_format=1, seed=w + 3)


@pytest.mark.parametrize("w", [2, 32])
def test_extend_without_output(w):
    """Appending only (no attention): the store and later decode steps are right."""
    run_extend(100, [50, 7, 90], w, with_out=False, seed=w)


def test_extend_long_chunk_small_window():
    """A 2000-token chunk with w = 3 and every token marked: chains of ~660
    reuses per slot, resolved by pointer jumping."""
    run_extend(64, [2000], 3, marks="all", Hkv=1, G=2, seed=12)


def test_extend_from_a_one_token_prompt():
    run_extend(1, [63, 1, 64, 65], 16, seed=2)


def test_extend_with_logits_from_k_channel():
    """Eviction logits read from K channel 3 (no logits input) in an extend call."""
    import torch
    import compact_decode_attention_amd as dms
    T0, n, Hkv, G, D, w = 120, 90, 2, 4, 64, 10
    q, k, v, lg = make_inputs(T0 + n, G * Hkv, Hkv, D, 31, "random")
    u = lg.view(np.uint32).astype(np.uint64)
    k[:, :, 3] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    mk = oracle.marks(oracle.k_channel_logits(k, 3))
    pool = dms.Pool(n_layers=1, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=T0 + n, max_pages=Hkv * 4, logit_channel=3)
    try:
        pool.prefill(0, 0, bf(k[:T0], torch).cuda(), bf(v[:T0], torch).cuda(), None)
        out = torch.empty((n, G * Hkv, D), dtype=torch.bfloat16, device="cuda")
        pool.extend(0, 0, bf(k[T0:], torch).cuda(), bf(v[T0:], torch).cuda(), None, q=bf(q[T0:], torch).cuda(),
                    out=out)
        ref = oracle.attend(q[T0:], np.arange(T0, T0 + n), k, v, mk, w)
        assert_close(out.view(torch.int16).cpu().numpy().view(np.uint16), ref, "extend, logits from K")
        for h in range(Hkv):
            assert np.array_equal(pool.export_live(0, 0, h), oracle.live_positions(T0 + n - 1, w, mk[:, h]))
    finally:
        pool.close()


def test_extend_errors():
    import torch
    import compact_decode_attention_amd as dms
    pool = dms.Pool(n_layers=1, n_q_heads=4, n_kv_heads=1, head_dim=64, window=4, max_seqs=1,
                    max_positions=40, max_pages=4)
    try:
        k = torch.zeros((30, 1, 64), dtype=torch.bfloat16, device="cuda")
        lg = torch.zeros((30, 1), dtype=torch.float32, device="cuda")
        with pytest.raises(dms.DMSError) as e:
            pool.extend(0, 0, k, k, lg)  # not prefilled
        assert e.value.status == dms.DMS_E_STATE
        pool.prefill(0, 0, k[:20], k[:20], lg[:20])
        with pytest.raises(dms.DMSError) as e:
            pool.extend(0, 0, k, k, lg)  # 20 + 30 > max_positions
        assert e.value.status == dms.DMS_E_STATE
        pool.extend(0, 0, k[:20], k[:20], lg[:20])
        st, _ = pool.stats(0)
        assert st.position == 40 and st.live_slots == 40
    finally:
        pool.close()


def test_extend_32k_chunked_prefill_sampled_rows():
    """The Qwen3-8B-shaped 32K prompt (32 q / 8 kv heads, D 128, w 512, keep
    score N(-1.2, 1)) as the bench times it: 8192 tokens prefilled, then 12
    chunks of 2048 appended with output; sampled rows of every chunk against the
    oracle, and every head's live set at the end."""
    import torch
    import compact_decode_attention_amd as dms
    wl = synth.WORKLOADS["qwen3-8b_prefill32k"]
    inp = synth.SynthInputs(wl)
    T, Hq, Hkv, D, w = wl.ctx_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    P0, C = 8192, 2048
    q, k, v, lg = inp.q(0, 0, 0, T), inp.k(0, 0, 0, T), inp.v(0, 0, 0, T), inp.logits(0, 0, 0, T)
    pool = dms.Pool(n_layers=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=T, max_pages=Hkv * (T // 64))
    try:
        dq, dk, dv = bf(q, torch).cuda(), bf(k, torch).cuda(), bf(v, torch).cuda()
        dl = torch.from_numpy(lg).cuda()
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
        pool.prefill(0, 0, dk[:P0], dv[:P0], dl[:P0])
        for t0 in range(P0, T, C):
            pool.extend(0, 0, dk[t0:t0 + C], dv[t0:t0 + C], dl[t0:t0 + C], q=dq[t0:t0 + C], out=out[t0:t0 + C])
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        rng = np.random.default_rng(1)
        rows = sorted(set([P0, P0 + 1, P0 + C - 1, P0 + C, P0 + C + 511, P0 + C + 512, T - 1] +
                          [int(t0 + rng.integers(0, C)) for t0 in range(P0, T, C)]))
        mk = oracle.marks(lg)
        ref = oracle.attend(q[rows], np.array(rows), k, v, mk, w)
        assert_close(got[rows], ref, "chunked 32K rows")
        for h in range(Hkv):
            assert np.array_equal(pool.export_live(0, 0, h), oracle.live_positions(T - 1, w, mk[:, h]))
    finally:
        pool.close()


def test_extend_after_a_decode_step_stored_a_wide_v():
    """A decode step appends a V row with values of magnitude 2^20 (no fp16
    counterpart); the extend that follows reads it from the store and must
    take the two-part bf16 weights: outputs match the oracle."""
    import torch
    import compact_decode_attention_amd as dms
    T0, n, G, Hkv, D, w = 130, 70, 4, 2, 64, 1 << 20
    total = T0 + 1 + n
    q, k, v, lg = make_inputs(total, G * Hkv, Hkv, D, 17, "random")
    v = v.copy()
    f = (v[T0].astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** 20)
    v[T0] = (f.view(np.uint32) >> 16).astype(np.uint16)
    mk = oracle.marks(lg)
    pool = dms.Pool(n_layers=1, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=total, max_pages=Hkv * 4)
    try:
        pool.prefill(0, 0, bf(k[:T0], torch).cuda(), bf(v[:T0], torch).cuda(), torch.from_numpy(lg[:T0]).cuda())
        o = torch.empty((1, 1, G * Hkv, D), dtype=torch.bfloat16, device="cuda")
        pool.decode_step([0], 0, bf(q[T0], torch).cuda().view(1, 1, -1, D), bf(k[T0], torch).cuda().view(1, 1, Hkv, D),
                         bf(v[T0], torch).cuda().view(1, 1, Hkv, D), torch.from_numpy(lg[T0]).cuda().view(1, 1, Hkv), o)
        t0 = T0 + 1
        out = torch.empty((n, G * Hkv, D), dtype=torch.bfloat16, device="cuda")
        pool.extend(0, 0, bf(k[t0:], torch).cuda(), bf(v[t0:], torch).cuda(), torch.from_numpy(lg[t0:]).cuda(),
                    q=bf(q[t0:], torch).cuda(), out=out)
        ref = oracle.attend(q[t0:], np.arange(t0, total), k, v, mk, w)
        assert_close(out.view(torch.int16).cpu().numpy().view(np.uint16), ref, "extend after a wide V was stored")
    finally:
        pool.close()


def test_extend_chunk_beyond_the_lds_rows():
    """A 5000-token chunk (more rows than the slot assignment keeps in LDS, so
    its chain arrays live in the scratch), w = 7 with random marks: chains of
    ~700 reuses, outputs and the store against the oracle."""
    run_extend(64, [5000], 7, marks="random", Hkv=1, G=2, D=64, seed=21)


@pytest.mark.parametrize("kv_format", [0, 1])
def test_extend_gathered_rows_span_several_scratch_pages(kv_format):
    """Unmarked chunk rows at least w rows before a query block are read from
    the kv head's scratch pages they were gathered into.  With no token marked
    and w = 16, a 700-row chunk gathers up to ~680 rows per kv head (11 pages,
    a partial last tile), for both kv heads; a second chunk reuses the same
    scratch pages with a shorter gather.  bf16 and FP8 pools."""
    run_extend(40, [700, 90], 16, marks="none", kv_format=kv_format, seed=31 + kv_format)


def test_extend_gathered_rows_with_mixed_marks_and_long_window():
    """w = 128 and random marks: the gathered segment holds the unmarked rows at
    or below each block's first row - w, the band the 160 rows after; chunk
    sizes that are not multiples of 32 or 64."""
    run_extend(300, [517, 3, 250], 128, marks="random", seed=41)
