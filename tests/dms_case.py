"""Drives the GPU library through the C ABI on seeded inputs and checks it
against the oracle: outputs within tolerance, live sets and counts exactly.

Tolerance: |gpu - ref| <= ATOL + RTOL * |ref| elementwise, with ATOL = 2e-3 and
RTOL = 1e-2 (bf16 K/V/Q inputs, fp32 accumulation, bf16 output; the reference
is the oracle in fp64 on the same bf16 inputs).  Every comparison also reports
two figures separately: the largest absolute error, and the largest relative
error over the elements with |ref| >= ATOL / RTOL (where the relative term
dominates the bound; nearer to zero a relative error says nothing).  They are
collected in ERRORS (name -> worst figures) and written out at the end of the
session when the environment names a file in DMS_PARITY_LOG.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable, List, Optional

import numpy as np

import oracle
import synth

ATOL = 2e-3
RTOL = 1e-2


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(bits).astype(np.float64)


# name -> {"max_abs", "max_rel", "elements", "checks"}: the worst figures seen
ERRORS = {}


def record_errors(name: str, max_abs: float, max_rel: float, elements: int):
    e = ERRORS.setdefault(name, {"max_abs": 0.0, "max_rel": 0.0, "elements": 0, "checks": 0})
    e["max_abs"] = max(e["max_abs"], max_abs)
    e["max_rel"] = max(e["max_rel"], max_rel)
    e["elements"] += int(elements)
    e["checks"] += 1


def error_figures(got: np.ndarray, ref: np.ndarray):
    """(largest |got - ref|, largest |got - ref| / |ref| over |ref| >= ATOL / RTOL)."""
    err = np.abs(got - ref)
    big = np.abs(ref) >= ATOL / RTOL
    rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    return float(err.max()) if err.size else 0.0, rel


def assert_close(gpu_bits: np.ndarray, ref: np.ndarray, what: str = "", record: str = "", max_abs: float = None):
    """Elementwise |gpu - ref| <= ATOL + RTOL |ref|; also, when max_abs is given,
    max |gpu - ref| <= max_abs on its own.  Returns (max-abs, max-rel) and, with
    record, adds them to ERRORS under that name."""
    got = bf16_bits_to_f64(gpu_bits)
    err = np.abs(got - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError("%s: %d of %d outside |d| <= %g + %g|ref| (worst at %s: gpu %r ref %r)"
                             % (what, int(bad.sum()), bad.size, ATOL, RTOL, i, got[i], ref[i]))
    fig = error_figures(got, ref)
    if max_abs is not None and fig[0] > max_abs:
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError("%s: max |d| %g above %g (at %s: gpu %r ref %r)" % (what, fig[0], max_abs, i, got[i],
                                                                                ref[i]))
    if record:
        record_errors(record, fig[0], fig[1], err.size)
    return fig


@dataclass
class SeqData:
    """Full per-(seq, layer) inputs for positions 0 .. total-1 (bf16 bits / f32)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    logits: np.ndarray


@dataclass
class Case:
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    ctx_lens: List[int]
    steps: int
    seed: int = 1234
    logits_fn: Optional[Callable] = None   # (seq, layer, positions[n]) -> float32 [n][Hkv]
    keep_mu: float = -1.2                  # logit = -(mu + N(0,1)) when logits_fn is None
    page_order_seed: int = 0
    max_pages: Optional[int] = None
    max_positions: Optional[int] = None
    zero_q: bool = False
    kv_format: int = 0                     # 0 bf16, 1 FP8 E4M3 (oracle: quantize_rows + attend_fp8)
    softmax_scale: float = 0.0             # 0: 1/sqrt(head_dim)
    logit_channel: Optional[int] = None    # logits carried by this K channel (the logits input unused)
    data: dict = field(default_factory=dict)
    q8: dict = field(default_factory=dict)

    @property
    def n_seqs(self):
        return len(self.ctx_lens)

    def total(self, s):
        return self.ctx_lens[s] + self.steps

    def gen(self):
        H, Hq, D = self.n_kv_heads, self.n_q_heads, self.head_dim
        for s in range(self.n_seqs):
            T = self.total(s)
            for l in range(self.n_layers):
                sid = lambda tag: synth.stream_id(tag, s, l)
                q = synth.normal_bf16(self.seed, sid(synth.TAG_Q), 0, T * Hq * D).reshape(T, Hq, D)
                if self.zero_q:
                    q[:] = 0
                k = synth.normal_bf16(self.seed, sid(synth.TAG_K), 0, T * H * D).reshape(T, H, D)
                v = synth.normal_bf16(self.seed, sid(synth.TAG_V), 0, T * H * D).reshape(T, H, D)
                if self.logits_fn is not None:
                    lg = np.asarray(self.logits_fn(s, l, np.arange(T)), np.float32).reshape(T, H)
                else:
                    z = synth.normal_f32(self.seed, sid(synth.TAG_SCORE), 0, T * H).reshape(T, H)
                    lg = (-(self.keep_mu + z.astype(np.float64))).astype(np.float32)
                if self.logit_channel is not None:
                    # the logit travels in K: channel c holds bf16(logit); the
                    # oracle reads it back from there
                    u = lg.view(np.uint32).astype(np.uint64)
                    k[:, :, self.logit_channel] = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
                    lg = oracle.k_channel_logits(k, self.logit_channel)
                self.data[(s, l)] = SeqData(q, k, v, lg)
        return self

    def pool_kwargs(self):
        maxpos = self.max_positions or max(self.total(s) for s in range(self.n_seqs))
        if self.max_pages is None:
            per_head = (maxpos + 63) // 64
            max_pages = per_head * self.n_layers * self.n_kv_heads * self.n_seqs
        else:
            max_pages = self.max_pages
        return dict(n_layers=self.n_layers, n_q_heads=self.n_q_heads, n_kv_heads=self.n_kv_heads,
                    head_dim=self.head_dim, window=self.window, max_seqs=self.n_seqs,
                    max_positions=maxpos, max_pages=max_pages, page_order_seed=self.page_order_seed,
                    kv_format=self.kv_format, logit_channel=self.logit_channel, softmax_scale=self.softmax_scale)

    # ---- oracle side
    def marks(self, s, l):
        return oracle.marks(self.data[(s, l)].logits)

    def quantized(self, s, l):
        """The oracle's E4M3 codes and row scales of every K and V row of (s, l)."""
        if (s, l) not in self.q8:
            d = self.data[(s, l)]
            k8, ks = oracle.quantize_rows(d.k)
            v8, vs = oracle.quantize_rows(d.v)
            self.q8[(s, l)] = (k8, ks, v8, vs)
        return self.q8[(s, l)]

    def oracle_out(self, s, l, t):
        d = self.data[(s, l)]
        m = self.marks(s, l)
        if self.kv_format:
            k8, ks, v8, vs = self.quantized(s, l)
            return oracle.attend_fp8(d.q[t:t + 1], [t], k8[:t + 1], ks[:t + 1], v8[:t + 1], vs[:t + 1],
                                     m[:t + 1], self.window, self.softmax_scale)[0]
        return oracle.attend(d.q[t:t + 1], [t], d.k[:t + 1], d.v[:t + 1], m[:t + 1], self.window,
                             self.softmax_scale)[0]

    def oracle_live(self, s, l, h, t):
        return oracle.live_positions(t, self.window, self.marks(s, l)[:t + 1, h])


def to_dev(arr, torch, dtype):
    a = np.ascontiguousarray(arr)
    if dtype == torch.bfloat16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def from_dev_bf16(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Runner:
    """Runs a Case on the GPU through the binding's Pool."""

    def __init__(self, case: Case):
        import torch
        import compact_decode_attention_amd as dms
        self.torch = torch
        self.dms = dms
        self.case = case
        self.pool = dms.Pool(**case.pool_kwargs())

    def prefill_all(self):
        c, torch = self.case, self.torch
        for s in range(c.n_seqs):
            T = c.ctx_lens[s]
            for l in range(c.n_layers):
                d = c.data[(s, l)]
                lg = None if c.logit_channel is not None else to_dev(d.logits[:T], torch, torch.float32)
                self.pool.prefill(s, l, to_dev(d.k[:T], torch, torch.bfloat16),
                                  to_dev(d.v[:T], torch, torch.bfloat16), lg)

    def step_inputs(self, i, seqs, layers):
        """Inputs of decode step i for the given seqs and layers, [layers][seqs]..."""
        c, torch = self.case, self.torch
        q = np.stack([np.stack([c.data[(s, l)].q[c.ctx_lens[s] + i] for s in seqs]) for l in layers])
        k = np.stack([np.stack([c.data[(s, l)].k[c.ctx_lens[s] + i] for s in seqs]) for l in layers])
        v = np.stack([np.stack([c.data[(s, l)].v[c.ctx_lens[s] + i] for s in seqs]) for l in layers])
        lg = np.stack([np.stack([c.data[(s, l)].logits[c.ctx_lens[s] + i] for s in seqs]) for l in layers])
        return (to_dev(q, torch, torch.bfloat16), to_dev(k, torch, torch.bfloat16),
                to_dev(v, torch, torch.bfloat16), to_dev(lg, torch, torch.float32))

    def decode(self, i, seqs=None, layer0=0, n_layers=None):
        c, torch = self.case, self.torch
        seqs = list(range(c.n_seqs)) if seqs is None else list(seqs)
        n_layers = c.n_layers - layer0 if n_layers is None else n_layers
        layers = list(range(layer0, layer0 + n_layers))
        q, k, v, lg = self.step_inputs(i, seqs, layers)
        if c.logit_channel is not None:
            lg = None
        out = torch.empty((n_layers, len(seqs), c.n_q_heads, c.head_dim), dtype=torch.bfloat16, device="cuda")
        self.pool.decode_step(seqs, layer0, q, k, v, lg, out)
        return from_dev_bf16(out)

    def check_live(self, t_of_seq):
        """Every (seq, layer, kv head): exported positions == oracle live set."""
        c = self.case
        st, _ = self.pool.stats()
        for s in range(c.n_seqs):
            t = t_of_seq[s]
            _, live = self.pool.stats(s, per_head=True)
            for l in range(c.n_layers):
                for h in range(c.n_kv_heads):
                    got = self.pool.export_live(s, l, h)
                    ref = c.oracle_live(s, l, h, t)
                    assert np.array_equal(got, ref), ("live set", s, l, h, t, len(got), len(ref))
                    assert live[l, h] == len(ref)
        return st

    def check_kv(self, t_of_seq):
        """Every (seq, layer, kv head): the stored rows, in position order, are
        exactly the inputs' rows (bf16 pools) or the oracle's codes and scales of
        them (FP8 pools) at the oracle's live positions."""
        c = self.case
        for s in range(c.n_seqs):
            for l in range(c.n_layers):
                d = c.data[(s, l)]
                for h in range(c.n_kv_heads):
                    pos, k, v, ks, vs = self.pool.export_kv(s, l, h)
                    ref = c.oracle_live(s, l, h, t_of_seq[s])
                    assert np.array_equal(pos, ref), ("kv positions", s, l, h)
                    if c.kv_format:
                        k8, kss, v8, vss = c.quantized(s, l)
                        assert np.array_equal(k, k8[pos, h]), ("K codes", s, l, h)
                        assert np.array_equal(v, v8[pos, h]), ("V codes", s, l, h)
                        assert np.array_equal(ks, kss[pos, h]), ("K scales", s, l, h)
                        assert np.array_equal(vs, vss[pos, h]), ("V scales", s, l, h)
                    else:
                        assert np.array_equal(k, d.k[pos, h]), ("K rows", s, l, h)
                        assert np.array_equal(v, d.v[pos, h]), ("V rows", s, l, h)

    def check_outputs(self, out, i, seqs=None, layer0=0, record=""):
        c = self.case
        seqs = list(range(c.n_seqs)) if seqs is None else list(seqs)
        worst = (0.0, 0.0)
        for li in range(out.shape[0]):
            for si, s in enumerate(seqs):
                t = c.ctx_lens[s] + i
                ref = c.oracle_out(s, layer0 + li, t)
                e = assert_close(out[li, si], ref, "seq %d layer %d t %d" % (s, layer0 + li, t), record=record)
                worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        return worst

    def close(self):
        self.pool.close()
