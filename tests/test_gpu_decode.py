"""GPU parity of the decode path (through the C ABI) against the oracle:
outputs within tolerance at every step, live sets and counts exactly."""
import numpy as np
import pytest

from dms_case import ATOL, RTOL, Case, Runner, bf16_bits_to_f64

pytestmark = pytest.mark.gpu


def run_case(case, check_live_every=1, layer_batched=True):
    case.gen()
    r = Runner(case)
    try:
        r.prefill_all()
        r.check_live([case.ctx_lens[s] - 1 for s in range(case.n_seqs)])
        worst = (0.0, 0.0)
        for i in range(case.steps):
            if layer_batched:
                out = r.decode(i)
            else:
                out = np.concatenate([r.decode(i, layer0=l, n_layers=1) for l in range(case.n_layers)])
            e = r.check_outputs(out, i, record="decode (fp8 pool)" if case.kv_format else "decode")
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
            if check_live_every and (i % check_live_every == 0 or i == case.steps - 1):
                r.check_live([case.ctx_lens[s] + i for s in range(case.n_seqs)])
        r.check_kv([case.ctx_lens[s] + case.steps - 1 for s in range(case.n_seqs)])
        return r, worst
    except Exception:
        r.close()
        raise


def test_tiny_d64_ctx1024_end_to_end():
    """One layer, 32 q / 8 kv heads, D=64, 1024-token prompt, 16 steps, w=256,
    keep score N(-1.2, 1) (about 1/8 kept)."""
    case = Case(n_layers=1, n_q_heads=32, n_kv_heads=8, head_dim=64, window=256,
                ctx_lens=[1024], steps=16, seed=20261203)
    r, worst = run_case(case)
    st, _ = r.pool.stats(0)
    assert st.position == 1024 + 16
    assert st.device_error == 0
    r.close()
    print("worst abs %.3g rel %.3g" % worst)


@pytest.mark.parametrize("kv_format", [0, 1])
@pytest.mark.parametrize("scale", [0.02, 0.3])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_softmax_scale(scale, D, kv_format):
    """A softmax scale other than 1/sqrt(head_dim) from the pool config: every
    step's outputs (layer-batched and per-layer calls), bf16 and FP8 pools."""
    case = Case(n_layers=2, n_q_heads=16, n_kv_heads=4, head_dim=D, window=30, ctx_lens=[333, 129], steps=12,
                seed=int(scale * 1000) + D, kv_format=kv_format, softmax_scale=scale)
    r, _ = run_case(case, check_live_every=6)
    r.close()
    r, _ = run_case(case, check_live_every=0, layer_batched=False)
    r.close()


def test_page_order_does_not_change_results():
    outs = []
    for seed in (0, 987654321):
        case = Case(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, window=40,
                    ctx_lens=[300, 170], steps=70, seed=5, page_order_seed=seed)
        case.gen()
        r = Runner(case)
        r.prefill_all()
        o = [r.decode(i) for i in range(case.steps)]
        r.close()
        outs.append(np.stack(o))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("marks", ["all", "none", "random"])
@pytest.mark.parametrize("window", [1, 2, 64, 1 << 20])
def test_windows_and_mark_extremes(marks, window):
    H = 2
    if marks == "all":
        fn = lambda s, l, p: np.ones((len(p), H), np.float32)
    elif marks == "none":
        fn = lambda s, l, p: -np.ones((len(p), H), np.float32)
    else:
        fn = None
    case = Case(n_layers=1, n_q_heads=8, n_kv_heads=H, head_dim=64, window=window,
                ctx_lens=[63, 64, 65, 1], steps=70, seed=11, logits_fn=fn, keep_mu=0.0,
                max_positions=200)
    r, _ = run_case(case, check_live_every=7)
    r.close()


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
def test_group_sizes(head_dim, group):
    case = Case(n_layers=1, n_q_heads=2 * group, n_kv_heads=2, head_dim=head_dim, window=24,
                ctx_lens=[200, 77], steps=30, seed=group * 100 + head_dim)
    r, _ = run_case(case, check_live_every=10)
    r.close()


def test_per_layer_calls_match_layer_batched():
    """One layer-batched call per step and one call per layer give the same
    results within the tolerance, and each matches the oracle.  The calls cut the
    page axis at different points (the batched call has more pages than the grid
    has waves), so the split-K rounding may differ in the last bits; repeating
    the same calls on a fresh pool reproduces every bit."""
    res = []
    for batched in (True, False, True):
        case = Case(n_layers=3, n_q_heads=16, n_kv_heads=4, head_dim=128, window=32,
                    ctx_lens=[9000, 7000], steps=4, seed=77, keep_mu=0.5)
        case.gen()
        r = Runner(case)
        r.prefill_all()
        outs = []
        for i in range(case.steps):
            if batched:
                o = r.decode(i)
            else:
                o = np.concatenate([r.decode(i, layer0=l, n_layers=1) for l in range(3)])
            if i in (0, case.steps - 1):
                r.check_outputs(o, i)
            outs.append(o)
        r.check_live([case.ctx_lens[s] + case.steps - 1 for s in range(2)])
        r.close()
        res.append(np.stack(outs))
    assert np.array_equal(res[0], res[2])
    a, b = bf16_bits_to_f64(res[0]), bf16_bits_to_f64(res[1])
    assert np.all(np.abs(a - b) <= ATOL + RTOL * np.abs(a))


def test_subset_of_sequences_per_call():
    """Sequences stepped by separate calls keep their own positions."""
    case = Case(n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=64, window=16,
                ctx_lens=[40, 90, 17], steps=12, seed=3)
    case.gen()
    r = Runner(case)
    r.prefill_all()
    for i in range(case.steps):
        o1 = r.decode(i, seqs=[2, 0])
        r.check_outputs(o1, i, seqs=[2, 0])
        o2 = r.decode(i, seqs=[1])
        r.check_outputs(o2, i, seqs=[1])
    r.check_live([case.ctx_lens[s] + case.steps - 1 for s in range(3)])
    r.close()


@pytest.mark.parametrize("kv_format", [0, 1])
def test_more_sequences_than_one_launch_takes(kv_format):
    """300 sequences in one call: more than the 256 a launch takes, so the call
    runs as two launches (256 + 44) that reuse the partials in stream order.
    Sequence ids in natural, reversed and shuffled order; every output, live set
    and stored row checked."""
    n = 300
    case = Case(n_layers=1, n_q_heads=4, n_kv_heads=1, head_dim=64, window=8,
                ctx_lens=[20 + (7 * s) % 53 for s in range(n)], steps=3, seed=41, kv_format=kv_format)
    case.gen()
    r = Runner(case)
    try:
        r.prefill_all()
        orders = [list(range(n)), list(range(n))[::-1], [int(x) for x in np.random.default_rng(5).permutation(n)]]
        for i, seqs in enumerate(orders):
            out = r.decode(i, seqs=seqs)
            r.check_outputs(out, i, seqs=seqs, record="decode (fp8 pool)" if kv_format else "decode")
        r.check_live([case.ctx_lens[s] + case.steps - 1 for s in range(n)])
        r.check_kv([case.ctx_lens[s] + case.steps - 1 for s in range(n)])
    finally:
        r.close()


def test_zero_query_gives_mean_of_live_values():
    case = Case(n_layers=1, n_q_heads=4, n_kv_heads=1, head_dim=128, window=10,
                ctx_lens=[150], steps=20, seed=9, zero_q=True)
    r, _ = run_case(case, check_live_every=5)
    r.close()


def test_release_and_reprefill_conserves_pages():
    case = Case(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=64, window=8,
                ctx_lens=[300, 200], steps=10, seed=21)
    case.gen()
    r = Runner(case)
    st0, _ = r.pool.stats()
    total_pages = st0.pages_free
    r.prefill_all()
    for i in range(case.steps):
        r.decode(i)
    st1, _ = r.pool.stats()
    assert st1.pages_used + st1.pages_free == total_pages
    r.pool.release(0)
    st2, _ = r.pool.stats()
    assert st2.pages_used + st2.pages_free == total_pages
    s0, _ = r.pool.stats(0)
    assert s0.live_slots == 0 and s0.position == -1
    # prefill seq 0 again and keep decoding both
    import compact_decode_attention_amd as dms
    case.steps_done = case.steps
    T = case.ctx_lens[0]
    for l in range(2):
        d = case.data[(0, l)]
        from dms_case import to_dev
        t = r.torch
        r.pool.prefill(0, l, to_dev(d.k[:T], t, t.bfloat16), to_dev(d.v[:T], t, t.bfloat16),
                       to_dev(d.logits[:T], t, t.float32))
    r.check_live([T - 1, case.ctx_lens[1] + case.steps - 1])
    st3, _ = r.pool.stats()
    assert st3.pages_used + st3.pages_free == total_pages
    r.close()


def test_reprefill_onto_other_pages_after_one_layer_calls():
    """Sequence 0 is stepped by one-layer calls, released, its freed pages are
    taken by sequence 1's prefill, and sequence 0 is prefilled again with the
    same prompt: the same page counts, so the calls' runs cover the same (head,
    page index) pairs as before the release, but on other pages.  Its next
    one-layer calls must read the new pages; sequence 1 must read its own."""
    case = Case(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=64, window=8,
                ctx_lens=[600, 600], steps=3, seed=23)
    case.gen()
    r = Runner(case)
    try:
        t = r.torch
        from dms_case import to_dev

        def prefill(s):
            T = case.ctx_lens[s]
            for l in range(case.n_layers):
                d = case.data[(s, l)]
                r.pool.prefill(s, l, to_dev(d.k[:T], t, t.bfloat16), to_dev(d.v[:T], t, t.bfloat16),
                               to_dev(d.logits[:T], t, t.float32))

        def one_layer_steps():
            for i in range(case.steps):
                for l in range(case.n_layers):
                    out = r.decode(i, seqs=[0], layer0=l, n_layers=1)
                    r.check_outputs(out, i, seqs=[0], layer0=l)

        prefill(0)
        one_layer_steps()
        r.pool.release(0)
        prefill(1)
        prefill(0)
        one_layer_steps()
        for i in range(case.steps):
            out = r.decode(i, seqs=[1])
            r.check_outputs(out, i, seqs=[1])
        r.check_live([case.ctx_lens[s] + case.steps - 1 for s in range(2)])
    finally:
        r.close()


@pytest.mark.parametrize("head_dim", [64, 128])
@pytest.mark.parametrize("kv_format", [0, 1])
def test_one_layer_calls_over_many_steps(head_dim, kv_format):
    """One sequence stepped by one-layer calls for 100 steps, every output
    checked.  About half the tokens are kept, so the heads keep growing into
    new pages: the page axis of later calls shifts, and a block's page from
    the call before it (which such calls read ahead of their plan) is often no
    longer its page."""
    case = Case(n_layers=2, n_q_heads=16, n_kv_heads=4, head_dim=head_dim, window=16,
                ctx_lens=[1500], steps=100, seed=31 + head_dim, keep_mu=0.0, kv_format=kv_format)
    case.gen()
    r = Runner(case)
    try:
        r.prefill_all()
        for i in range(case.steps):
            for l in range(case.n_layers):
                out = r.decode(i, seqs=[0], layer0=l, n_layers=1)
                r.check_outputs(out, i, seqs=[0], layer0=l,
                                record="decode (fp8 pool)" if kv_format else "decode")
        r.check_live([case.ctx_lens[0] + case.steps - 1])
        r.check_kv([case.ctx_lens[0] + case.steps - 1])
    finally:
        r.close()


def test_one_layer_calls_with_more_pages_than_blocks():
    """One-layer calls of about 260 pages (head_dim 128): more pages than the
    attention grid has blocks on a 256-CU part, so the second pair of waves of
    a block takes page b + grid; the layer-batched call of the same step (about
    520 pages) takes the general path.  Every output checked against the
    oracle."""
    case = Case(n_layers=2, n_q_heads=16, n_kv_heads=4, head_dim=128, window=32,
                ctx_lens=[6000], steps=4, seed=57, keep_mu=0.5)
    case.gen()
    r = Runner(case)
    try:
        r.prefill_all()
        _, live = r.pool.stats(0, per_head=True)
        pages = [int(sum((int(n) + 63) // 64 for n in live[l])) for l in range(case.n_layers)]
        assert all(256 < p <= 512 for p in pages), pages
        for i in range(case.steps):
            if i % 2:
                out = r.decode(i)
                r.check_outputs(out, i)
            else:
                for l in range(case.n_layers):
                    out = r.decode(i, seqs=[0], layer0=l, n_layers=1)
                    r.check_outputs(out, i, seqs=[0], layer0=l)
        r.check_live([case.ctx_lens[0] + case.steps - 1])
    finally:
        r.close()


def test_capacity_exhaustion_is_reported():
    import compact_decode_attention_amd as dms
    case = Case(n_layers=1, n_q_heads=4, n_kv_heads=1, head_dim=64, window=4,
                ctx_lens=[64], steps=3, seed=1, max_pages=1,
                logits_fn=lambda s, l, p: -np.ones((len(p), 1), np.float32))
    case.gen()
    r = Runner(case)
    r.prefill_all()            # 64 live tokens: exactly one page
    r.decode(0)                # token 64 needs a second page: none left
    with pytest.raises(dms.DMSError) as ei:
        r.pool.stats()
    assert ei.value.status == dms.DMS_E_CAPACITY
    st, _ = r.pool.stats(raise_on_error=False)
    assert st.device_error == dms.DMS_E_CAPACITY
    r.close()


def test_host_side_errors():
    import compact_decode_attention_amd as dms
    case = Case(n_layers=2, n_q_heads=4, n_kv_heads=1, head_dim=64, window=4,
                ctx_lens=[10], steps=2, seed=1)
    case.gen()
    r = Runner(case)
    with pytest.raises(dms.DMSError) as ei:
        r.decode(0)            # not prefilled
    assert ei.value.status == dms.DMS_E_STATE
    r.prefill_all()
    from dms_case import to_dev
    t = r.torch
    d = case.data[(0, 0)]
    with pytest.raises(dms.DMSError) as ei:
        r.pool.prefill(0, 0, to_dev(d.k[:10], t, t.bfloat16), to_dev(d.v[:10], t, t.bfloat16),
                       to_dev(d.logits[:10], t, t.float32))
    assert ei.value.status == dms.DMS_E_STATE
    with pytest.raises(dms.DMSError) as ei:
        dms.dms_decode_step(r.pool.handle, [0, 0], 0, 1, 1, 1, 1, 1, 1, 0)
    assert ei.value.status == dms.DMS_E_INVAL
    with pytest.raises(dms.DMSError) as ei:
        dms.dms_decode_step(r.pool.handle, [0], 1, 2, 1, 1, 1, 1, 1, 0)
    assert ei.value.status == dms.DMS_E_INVAL
    r.close()


def test_many_items_per_head_across_blocks():
    """Long live sets (tens of split-K partials per head) on several layers and
    sequences, every step checked."""
    case = Case(n_layers=4, n_q_heads=16, n_kv_heads=4, head_dim=128, window=100,
                ctx_lens=[3000, 5000, 1500], steps=12, seed=31, keep_mu=0.5)
    r, _ = run_case(case, check_live_every=6)
    r.close()


@pytest.mark.parametrize("kv_format", [0, 1])
@pytest.mark.parametrize("group", [4, 8])
def test_merge_spread_over_blocks(group, kv_format):
    """Calls of few heads with tens of pages each (a single layer of a single
    sequence): every head's merge is spread over several blocks, each writing its
    share of the head's outputs.  Checked against the oracle at every step, on
    bf16 and FP8 pools."""
    case = Case(n_layers=2, n_q_heads=2 * group, n_kv_heads=2, head_dim=128, window=48,
                ctx_lens=[6000], steps=4, seed=500 + group + kv_format, keep_mu=2.0, kv_format=kv_format)
    r, _ = run_case(case, check_live_every=2, layer_batched=False)
    r.close()


def test_hundreds_of_partials_for_one_head():
    """One kv head whose pages outnumber the partials the merge keeps in
    registers and LDS (every page its own wave): the merge's overflow paths."""
    case = Case(n_layers=1, n_q_heads=4, n_kv_heads=1, head_dim=128, window=64,
                ctx_lens=[20000], steps=3, seed=41, keep_mu=6.0)
    r, _ = run_case(case, check_live_every=3)
    r.close()
