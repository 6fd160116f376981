"""GPU parity of pools whose eviction logits are read from a K channel
(logit_source = DMS_LOGITS_K_CHANNEL), through the C ABI: outputs, live sets
and stored rows against the oracle with the logits it reads from the same
channel; and the same results, bit for bit, as a pool fed those logits through
the logits input."""
import numpy as np
import pytest

from dms_case import Case, Runner

pytestmark = pytest.mark.gpu


def run(case, check_every=5):
    case.gen()
    r = Runner(case)
    outs = []
    try:
        r.prefill_all()
        r.check_live([case.ctx_lens[s] - 1 for s in range(case.n_seqs)])
        for i in range(case.steps):
            o = r.decode(i)
            r.check_outputs(o, i)
            outs.append(o)
            if i % check_every == 0 or i == case.steps - 1:
                r.check_live([case.ctx_lens[s] + i for s in range(case.n_seqs)])
        r.check_kv([case.ctx_lens[s] + case.steps - 1 for s in range(case.n_seqs)])
    finally:
        r.close()
    return np.stack(outs)


@pytest.mark.parametrize("kv_format", [0, 1])
@pytest.mark.parametrize("head_dim,channel", [(64, 0), (64, 63), (128, 17), (128, 127)])
def test_channel_logits_decode(head_dim, channel, kv_format):
    run(Case(n_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=head_dim, window=16, ctx_lens=[150, 333],
             steps=25, seed=head_dim + channel, keep_mu=0.0, logit_channel=channel, kv_format=kv_format))


def test_channel_logits_match_the_logits_input():
    """The same K (channel 5 carrying the logits) with the logits passed in
    separately gives bit-identical outputs."""
    a = run(Case(n_layers=2, n_q_heads=16, n_kv_heads=4, head_dim=128, window=32, ctx_lens=[700, 90],
                 steps=20, seed=8, logit_channel=5))
    c2 = Case(n_layers=2, n_q_heads=16, n_kv_heads=4, head_dim=128, window=32, ctx_lens=[700, 90],
              steps=20, seed=8, logit_channel=5)
    c2.gen()
    c2.logit_channel = None  # same data (K carries the logits), logits through the input
    r = Runner(c2)
    try:
        r.prefill_all()
        b = np.stack([r.decode(i) for i in range(c2.steps)])
    finally:
        r.close()
    assert np.array_equal(a, b)


def test_channel_logits_prefill_with_output():
    """Masked prefill attention on MFMA with the marks taken from the channel."""
    import torch
    import oracle
    from dms_case import assert_close, to_dev
    case = Case(n_layers=1, n_q_heads=8, n_kv_heads=2, head_dim=128, window=24, ctx_lens=[300], steps=1,
                seed=4, keep_mu=0.0, logit_channel=9).gen()
    r = Runner(case)
    try:
        d = case.data[(0, 0)]
        T = 300
        out = torch.empty((T, 8, 128), dtype=torch.bfloat16, device="cuda")
        r.pool.prefill(0, 0, to_dev(d.k[:T], torch, torch.bfloat16), to_dev(d.v[:T], torch, torch.bfloat16),
                       None, q=to_dev(d.q[:T], torch, torch.bfloat16), out=out)
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        mk = oracle.marks(d.logits[:T])
        assert 0 < mk.sum() < mk.size
        ref = oracle.attend(d.q[:T], np.arange(T), d.k[:T], d.v[:T], mk, 24)
        assert_close(got, ref, "prefill, logits from K channel 9")
        r.check_live([T - 1])
    finally:
        r.close()
