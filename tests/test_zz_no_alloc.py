"""dms_decode_step_static (split-K scratch in the library's per-GPU static
array; the call allocates nothing) against dms_decode_step on the same inputs,
through the C ABI: two pools fed identically, calls of different sizes in a
row (the second smaller than the first, so the array keeps the first call's
contents), outputs bit-identical and within the oracle's tolerance, live sets
and stored rows exact; a call too large for the array is refused."""
import numpy as np
import pytest

from dms_case import Case, Runner, assert_close

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv_format", [0, 1])
def test_static_scratch_matches_the_arena_entry_point(kv_format):
    case = Case(n_layers=3, n_q_heads=16, n_kv_heads=4, head_dim=128, window=24, ctx_lens=[260, 131],
                steps=6, seed=91, kv_format=kv_format)
    case.gen()
    ra, rb = Runner(case), Runner(case)
    torch = ra.torch
    try:
        ra.prefill_all()
        rb.prefill_all()
        # (seqs, layer0, n_layers) per step: the second call smaller than the first
        calls = [([0, 1], 0, 3), ([1], 2, 1), ([0, 1], 0, 2), ([0], 2, 1), ([0, 1], 0, 3), ([1], 1, 1)]
        done = {(s, l): 0 for s in range(2) for l in range(3)}  # steps taken per (seq, layer)
        for seqs, l0, nl in calls:
            steps = {done[(s, l)] for s in seqs for l in range(l0, l0 + nl)}
            assert len(steps) == 1
            i = steps.pop()
            q, k, v, lg = ra.step_inputs(i, seqs, list(range(l0, l0 + nl)))
            oa = torch.empty((nl, len(seqs), case.n_q_heads, case.head_dim), dtype=torch.bfloat16, device="cuda")
            ob = torch.empty_like(oa)
            ra.pool.decode_step(seqs, l0, q, k, v, lg, oa)
            rb.pool.decode_step(seqs, l0, q, k, v, lg, ob, static_scratch=True)
            torch.cuda.synchronize()
            assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), (seqs, l0, nl)
            got = ob.view(torch.int16).cpu().numpy().view(np.uint16)
            for li in range(nl):
                for si, s in enumerate(seqs):
                    assert_close(got[li, si], case.oracle_out(s, l0 + li, case.ctx_lens[s] + i),
                                 "static scratch seq %d layer %d step %d" % (s, l0 + li, i))
            for s in seqs:
                for l in range(l0, l0 + nl):
                    done[(s, l)] += 1
        for s in range(2):
            for l in range(3):
                t = case.ctx_lens[s] + done[(s, l)] - 1
                for h in range(case.n_kv_heads):
                    pa, ka, va, _, _ = ra.pool.export_kv(s, l, h)
                    pb, kb, vb, _, _ = rb.pool.export_kv(s, l, h)
                    assert np.array_equal(pb, case.oracle_live(s, l, h, t))
                    assert np.array_equal(pa, pb) and np.array_equal(ka, kb) and np.array_equal(va, vb)
        st, _ = rb.pool.stats()
        assert st.device_error == 0
    finally:
        ra.close()
        rb.close()


def test_static_scratch_refuses_a_call_beyond_its_size():
    """504 layers x 8 kv heads at G = 8, D = 128 in one launch needs about 21 MB
    of partials: DMS_E_INVAL, nothing enqueued; the arena entry point takes it."""
    import torch
    import compact_decode_attention_amd as dms
    L, H, G, D = 504, 8, 8, 128
    pool = dms.Pool(n_layers=L, n_q_heads=G * H, n_kv_heads=H, head_dim=D, window=4, max_seqs=1,
                    max_positions=64, max_pages=1)
    try:
        q = torch.zeros((L, 1, G * H, D), dtype=torch.bfloat16, device="cuda")
        kv = torch.zeros((L, 1, H, D), dtype=torch.bfloat16, device="cuda")
        lg = torch.zeros((L, 1, H), dtype=torch.float32, device="cuda")
        with pytest.raises(dms.DMSError) as e:
            pool.decode_step([0], 0, q, kv, kv, lg, q.clone(), static_scratch=True)
        assert e.value.status == dms.DMS_E_INVAL and "scratch" in str(e.value)
        with pytest.raises(dms.DMSError) as e:  # the arena entry point: past the size check, not prefilled
            pool.decode_step([0], 0, q, kv, kv, lg, q.clone())
        assert e.value.status == dms.DMS_E_STATE
    finally:
        pool.close()
