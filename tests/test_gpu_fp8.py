"""GPU parity of FP8 (OCP E4M3) pools against the oracle, through the C ABI.

Stored rows are checked bit for bit: dms_export_kv's codes and row scales must
equal the oracle's quantize_rows of the same bf16 inputs at the oracle's live
positions, after the prefill and after decode steps (which quantise the new
token on the GPU).  Outputs (prefill and decode) are compared with the oracle's
attend_fp8, i.e. attention over value(code) * scale in float64, within the same
tolerance as bf16 pools (the GPU reads the same dequantised values; only the
accumulation order and fp32 rounding differ)."""
import numpy as np
import pytest

import oracle
import synth
from dms_case import Case, Runner, assert_close

pytestmark = pytest.mark.gpu

FP8 = 1


def bf(a, torch):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def _rne_bf16(x):
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def make_inputs(T, Hq, Hkv, D, seed, marks, kv_range="normal"):
    q = synth.normal_bf16(seed, synth.stream_id(synth.TAG_Q), 0, T * Hq * D).reshape(T, Hq, D)
    k = synth.normal_bf16(seed, synth.stream_id(synth.TAG_K), 0, T * Hkv * D).reshape(T, Hkv, D)
    v = synth.normal_bf16(seed, synth.stream_id(synth.TAG_V), 0, T * Hkv * D).reshape(T, Hkv, D)
    if kv_range == "wide":
        # each element times 2^e, e uniform in [-14, 0], and every 7th row zero:
        # subnormal codes, rows of very different scales, all-zero rows (scale 1)
        e = np.floor(synth.uniform(seed, synth.stream_id(synth.TAG_SCORE, 1), 0, 2 * T * Hkv * D) * 15.0)
        e = e.reshape(2, T, Hkv, D)
        kf = synth.bf16_to_f32(k) * np.exp2(-e[0]).astype(np.float32)
        vf = synth.bf16_to_f32(v) * np.exp2(-e[1]).astype(np.float32)
        kf[::7] = 0.0
        vf[3::7] = 0.0
        k, v = _rne_bf16(kf), _rne_bf16(vf)
    if marks == "all":
        lg = np.ones((T, Hkv), np.float32)
    elif marks == "none":
        lg = -np.ones((T, Hkv), np.float32)
    else:
        z = synth.normal_f32(seed, synth.stream_id(synth.TAG_SCORE), 0, T * Hkv).reshape(T, Hkv)
        lg = (-(-0.3 + z.astype(np.float64))).astype(np.float32)
    return q, k, v, lg


def check_stored(pool, T, w, mk, k8, ks, v8, vs, Hkv):
    for h in range(Hkv):
        pos, kc, vc, ksc, vsc = pool.export_kv(0, 0, h)
        live = oracle.live_positions(T - 1, w, mk[:T, h])
        assert np.array_equal(pos, live)
        assert np.array_equal(kc, k8[pos, h]), "K codes, head %d" % h
        assert np.array_equal(vc, v8[pos, h]), "V codes, head %d" % h
        assert np.array_equal(ksc, ks[pos, h]), "K scales, head %d" % h
        assert np.array_equal(vsc, vs[pos, h]), "V scales, head %d" % h


def run_prefill8(T, w, marks, G=4, D=128, Hkv=2, seed=5, decode_steps=0, kv_range="normal"):
    import torch
    import compact_decode_attention_amd as dms
    Hq = G * Hkv
    total = T + decode_steps
    q, k, v, lg = make_inputs(total, Hq, Hkv, D, seed, marks, kv_range)
    k8, ks = oracle.quantize_rows(k)
    v8, vs = oracle.quantize_rows(v)
    pool = dms.Pool(n_layers=1, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, window=w, max_seqs=1,
                    max_positions=total, max_pages=Hkv * ((total + 63) // 64), kv_format=FP8)
    try:
        dev = "cuda"
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
        pool.prefill(0, 0, bf(k[:T], torch).to(dev), bf(v[:T], torch).to(dev), torch.from_numpy(lg[:T]).to(dev),
                     q=bf(q[:T], torch).to(dev), out=out)
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        mk = oracle.marks(lg)
        ref = oracle.attend_fp8(q[:T], np.arange(T), k8[:T], ks[:T], v8[:T], vs[:T], mk[:T], w)
        assert_close(got, ref, "fp8 prefill T=%d w=%d marks=%s G=%d D=%d" % (T, w, marks, G, D))
        check_stored(pool, T, w, mk, k8, ks, v8, vs, Hkv)
        for i in range(decode_steps):
            t = T + i
            o = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
            pool.decode_step([0], 0, bf(q[t], torch).to(dev).view(1, 1, Hq, D),
                             bf(k[t], torch).to(dev).view(1, 1, Hkv, D), bf(v[t], torch).to(dev).view(1, 1, Hkv, D),
                             torch.from_numpy(lg[t]).to(dev).view(1, 1, Hkv), o)
            r = oracle.attend_fp8(q[t:t + 1], [t], k8[:t + 1], ks[:t + 1], v8[:t + 1], vs[:t + 1], mk[:t + 1], w)[0]
            assert_close(o.view(torch.int16).cpu().numpy().view(np.uint16)[0, 0], r, "fp8 decode t=%d" % t)
        if decode_steps:
            check_stored(pool, total, w, mk, k8, ks, v8, vs, Hkv)
    finally:
        pool.close()


@pytest.mark.parametrize("marks", ["random", "all", "none"])
@pytest.mark.parametrize("w", [1, 16, 64])
@pytest.mark.parametrize("T", [1, 33, 130, 700])
def test_fp8_prefill_shapes(T, w, marks):
    run_prefill8(T, w, marks)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_fp8_prefill_group_sizes(G, D):
    run_prefill8(300, 40, "random", G=G, D=D, seed=G * 10 + D)


def test_fp8_prefill_eviction_disabled():
    run_prefill8(500, 1 << 20, "random")


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_wide_dynamic_range_and_zero_rows(D):
    """Elements spread over 15 binades, zero K and V rows: subnormal codes and
    the scale of an all-zero row, through prefill and decode."""
    run_prefill8(333, 24, "random", G=2, D=D, seed=71, decode_steps=70, kv_range="wide")


def test_fp8_prefill_then_decode():
    run_prefill8(257, 32, "random", decode_steps=40, seed=9)


def run_case8(case, check_every=1):
    case.gen()
    r = Runner(case)
    try:
        r.prefill_all()
        r.check_kv([case.ctx_lens[s] - 1 for s in range(case.n_seqs)])
        for i in range(case.steps):
            out = r.decode(i)
            r.check_outputs(out, i)
            if check_every and (i % check_every == 0 or i == case.steps - 1):
                r.check_live([case.ctx_lens[s] + i for s in range(case.n_seqs)])
        r.check_kv([case.ctx_lens[s] + case.steps - 1 for s in range(case.n_seqs)])
    finally:
        r.close()


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_fp8_decode_group_sizes(head_dim, group):
    run_case8(Case(n_layers=1, n_q_heads=2 * group, n_kv_heads=2, head_dim=head_dim, window=24,
                   ctx_lens=[200, 77], steps=30, seed=group * 100 + head_dim, kv_format=FP8), check_every=10)


@pytest.mark.parametrize("marks", ["all", "none", "random"])
@pytest.mark.parametrize("window", [1, 2, 64, 1 << 20])
def test_fp8_windows_and_mark_extremes(marks, window):
    H = 2
    if marks == "all":
        fn = lambda s, l, p: np.ones((len(p), H), np.float32)
    elif marks == "none":
        fn = lambda s, l, p: -np.ones((len(p), H), np.float32)
    else:
        fn = None
    run_case8(Case(n_layers=1, n_q_heads=8, n_kv_heads=H, head_dim=64, window=window,
                   ctx_lens=[63, 64, 65, 1], steps=70, seed=11, logits_fn=fn, keep_mu=0.0,
                   max_positions=200, kv_format=FP8), check_every=7)


def test_fp8_many_partials_and_layers():
    """Long live sets on several layers and sequences (tens of split-K partials
    per head), every step checked."""
    run_case8(Case(n_layers=3, n_q_heads=16, n_kv_heads=4, head_dim=128, window=100,
                   ctx_lens=[3000, 5000, 1500], steps=10, seed=31, keep_mu=0.5, kv_format=FP8), check_every=5)


def test_fp8_page_order_does_not_change_results():
    outs = []
    for seed in (0, 987654321):
        case = Case(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, window=40,
                    ctx_lens=[300, 170], steps=40, seed=5, page_order_seed=seed, kv_format=FP8)
        case.gen()
        r = Runner(case)
        r.prefill_all()
        o = [r.decode(i) for i in range(case.steps)]
        r.close()
        outs.append(np.stack(o))
    assert np.array_equal(outs[0], outs[1])


def test_fp8_pool_stats_count_fp8_bytes():
    case = Case(n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=128, window=16,
                ctx_lens=[500], steps=3, seed=4, kv_format=FP8)
    case.gen()
    r = Runner(case)
    try:
        r.prefill_all()
        for i in range(case.steps):
            r.decode(i)
        st, _ = r.pool.stats(0)
        t = case.ctx_lens[0] + case.steps - 1
        ref = oracle.kv_bytes(t, case.window, case.marks(0, 0), 128, fp8=True)
        assert (st.kv_bytes_live, st.kv_bytes_allocated, st.kv_bytes_dense_equiv) == ref
        assert st.kv_bytes_allocated == st.pages_used * 64 * 2 * oracle.row_bytes(128, fp8=True)
    finally:
        r.close()
