"""GPU parity of dms_prefill with output (masked causal attention on MFMA plus
compaction) against the oracle: every query row within tolerance, live sets
after the prefill exact, and decode continuing correctly from the compacted
store."""
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


def run_prefill(T, w, marks, G=4, D=128, Hkv=2, seed=5, extra_positions=0, decode_steps=0, softmax_scale=0.0,
                kv_format=0):
    import torch
    import compact_decode_attention_amd as dms
    Hq = G * Hkv
    total = T + decode_steps
    q, k, v, lg = make_inputs(total, Hq, Hkv, D, seed, marks)
    maxpos = total + extra_positions
    pool = dms.Pool(n_layers=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=maxpos, max_pages=Hkv * ((maxpos + 63) // 64), softmax_scale=softmax_scale,
                    kv_format=kv_format)
    mk = oracle.marks(lg)
    if kv_format:
        k8, ks = oracle.quantize_rows(k)
        v8, vs = oracle.quantize_rows(v)

    def ref_out(t0, n):
        if kv_format:
            return oracle.attend_fp8(q[t0:t0 + n], np.arange(t0, t0 + n), k8[:t0 + n], ks[:t0 + n], v8[:t0 + n],
                                     vs[:t0 + n], mk[:t0 + n], w, softmax_scale)
        return oracle.attend(q[t0:t0 + n], np.arange(t0, t0 + n), k[:t0 + n], v[:t0 + n], mk[:t0 + n], w,
                             softmax_scale)

    dev = "cuda"
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
    pool.prefill(0, 0, bf(k[:T], torch).to(dev), bf(v[:T], torch).to(dev), torch.from_numpy(lg[:T]).to(dev),
                 q=bf(q[:T], torch).to(dev), out=out)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_close(got, ref_out(0, T), "prefill T=%d w=%d marks=%s G=%d D=%d" % (T, w, marks, G, D),
                 record="prefill (fp8 pool)" if kv_format else "prefill")
    for h in range(Hkv):
        assert np.array_equal(pool.export_live(0, 0, h), oracle.live_positions(T - 1, w, mk[:T, h]))
    for i in range(decode_steps):
        t = T + i
        o = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
        pool.decode_step([0], 0, bf(q[t], torch).to(dev).view(1, 1, Hq, D), bf(k[t], torch).to(dev).view(1, 1, Hkv, D),
                         bf(v[t], torch).to(dev).view(1, 1, Hkv, D), torch.from_numpy(lg[t]).to(dev).view(1, 1, Hkv), o)
        assert_close(o.view(torch.int16).cpu().numpy().view(np.uint16)[0, 0], ref_out(t, 1)[0],
                     "decode after prefill t=%d" % t)
    pool.close()


@pytest.mark.parametrize("marks", ["random", "all", "none"])
@pytest.mark.parametrize("w", [1, 16, 64])
@pytest.mark.parametrize("T", [1, 31, 33, 130, 700])
def test_prefill_shapes(T, w, marks):
    run_prefill(T, w, marks)


@pytest.mark.parametrize("T", [64, 500])
def test_prefill_eviction_disabled(T):
    """Window beyond every position: plain causal attention."""
    run_prefill(T, 1 << 20, "random")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_prefill_group_sizes(G, D):
    run_prefill(300, 40, "random", G=G, D=D, seed=G * 10 + D)


def test_prefill_then_decode():
    run_prefill(257, 32, "random", decode_steps=40, seed=9)


@pytest.mark.parametrize("kv_format", [0, 1])
@pytest.mark.parametrize("scale", [0.02, 0.3])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_softmax_scale(scale, D, kv_format):
    """A softmax scale other than 1/sqrt(head_dim) from the pool config, in the
    prefill and in the decode steps after it, on bf16 and FP8 pools."""
    run_prefill(300, 48, "random", D=D, seed=int(scale * 100) + D, decode_steps=5, softmax_scale=scale,
                kv_format=kv_format)


def test_prefill_32k_sampled_rows():
    """Qwen3-8B-shaped prefill of one layer: 32768 tokens, 32 q / 8 kv heads,
    D=128, w=512, keep score N(-1.2, 1); sampled query rows vs the oracle."""
    import torch
    import compact_decode_attention_amd as dms
    wl = synth.WORKLOADS["qwen3-8b_prefill32k"]
    inp = synth.SynthInputs(wl)
    T, Hq, Hkv, D, w = wl.ctx_len, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.window
    q, k, v, lg = inp.q(0, 0, 0, T), inp.k(0, 0, 0, T), inp.v(0, 0, 0, T), inp.logits(0, 0, 0, T)
    pool = dms.Pool(n_layers=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=T, max_pages=Hkv * (T // 64))
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    pool.prefill(0, 0, bf(k, torch).cuda(), bf(v, torch).cuda(), torch.from_numpy(lg).cuda(),
                 q=bf(q, torch).cuda(), out=out)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    rng = np.random.default_rng(0)
    rows = sorted(set([0, 1, 31, 32, 511, 512, 513, 1000, T - 33, T - 32, T - 1] +
                      rng.integers(0, T, 24).tolist()))
    mk = oracle.marks(lg)
    ref = oracle.attend(q[rows], np.array(rows), k, v, mk, w)
    assert_close(got[rows], ref, "prefill 32k rows", record="qwen3-8b_prefill32k (sampled rows)")
    for h in range(Hkv):
        assert np.array_equal(pool.export_live(0, 0, h), oracle.live_positions(T - 1, w, mk[:, h]))
    pool.close()


def scaled_bf16(bits, factor):
    """bf16 bits of value * factor (factor a power of two: exact)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(factor)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def prefill_and_check(pool, layer, q, k, v, lg, w, what):
    import torch
    T, Hq, D = q.shape
    out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    pool.prefill(0, layer, bf(k, torch).cuda(), bf(v, torch).cuda(), torch.from_numpy(lg).cuda(),
                 q=bf(q, torch).cuda(), out=out)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_close(got, oracle.attend(q, np.arange(T), k, v, oracle.marks(lg), w), what)


def test_prefill_v_at_the_fp16_limit():
    """V values of 65280 (the largest bf16 value below 2^16, exact in fp16)
    keep the fp16 weights path: outputs match."""
    import compact_decode_attention_amd as dms
    T, G, Hkv, D, w = 200, 4, 2, 128, 24
    q, k, v, lg = make_inputs(T, G * Hkv, Hkv, D, 41, "random")
    v = v.copy()
    v[::13, :, ::5] = 0x477F  # positive: the outputs are dominated by them, no cancellation
    pool = dms.Pool(n_layers=1, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=T, max_pages=Hkv * 4)
    try:
        prefill_and_check(pool, 0, q, k, v, lg, w, "V at +-65280")
    finally:
        pool.close()


def test_prefill_v_beyond_fp16_range_switches_the_pool_to_bf16_weights():
    """A V value of magnitude 2^16 or more has no fp16 counterpart: the pool
    keeps its attention on the two-part bf16 weights from then on.  Layer 0's
    prompt holds values times 2^20, layer 1's is ordinary; both match."""
    import compact_decode_attention_amd as dms
    T, G, Hkv, D, w = 300, 4, 2, 128, 32
    pool = dms.Pool(n_layers=2, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=T, max_pages=2 * Hkv * 5)
    try:
        q, k, v, lg = make_inputs(T, G * Hkv, Hkv, D, 43, "random")
        vw = v.copy()
        vw[7::29] = scaled_bf16(v[7::29] & 0x7fff, 2.0 ** 20)  # magnitudes: no cancellation between them
        prefill_and_check(pool, 0, q, k, vw, lg, w, "V times 2^20 in some rows")
        q, k, v, lg = make_inputs(T, G * Hkv, Hkv, D, 44, "random")
        prefill_and_check(pool, 1, q, k, v, lg, w, "ordinary layer after a wide one")
    finally:
        pool.close()
