"""Seeded synthetic inputs for DMS decode / prefill workloads.

This package is shared by the GPU path's tests and bench and by the CPU oracle's
tests.  It holds no part of the method's arithmetic: it only draws the inputs
(queries, keys, values and eviction logits) that both sides consume, and it
describes the workload shapes.

Every tensor comes from a counter-based stream (SplitMix64, see synth_gen.c),
keyed by (seed, tensor tag, sequence, layer), indexed by the element's flat
position inside a [position][head][dim] layout.  The token at position p has
the same q/k/v/logit whether it is generated as part of a prompt or as a decode
step, so any slice can be regenerated on demand.

Eviction logits.  The workload descriptions give each token a per-kv-head score
s ~ N(mu_h, 1) with a stated keep rate of about P(s >= 0) (about 1/8 for
mu = -1.2, the "8x" compression the DMS pages name).  The library marks a token
for eviction iff its logit is > 0, so the generator hands over logit = -s
(keep iff s >= 0).  ``marks="literal"`` instead hands over logit = +s.
"""
from __future__ import annotations

import ctypes
import os
import statistics
import subprocess
import threading
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth_gen.c")
_SO = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib_handle = None

# tensor tags (top byte of a stream id)
TAG_Q, TAG_K, TAG_V, TAG_SCORE, TAG_MU, TAG_BETA, TAG_CTX = 1, 2, 3, 4, 5, 6, 7


def build(force: bool = False) -> str:
    """Compile synth_gen.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    with _lock:
        if _lib_handle is None:
            build()
            lib = ctypes.CDLL(_SO)
            u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
            lib.synth_u64.argtypes = [u64, u64, u64, i64, vp]
            lib.synth_raw_u64.argtypes = [u64, u64, i64, vp]
            lib.synth_raw_u64.restype = None
            lib.synth_uniform_f64.argtypes = [u64, u64, u64, i64, vp]
            lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
            lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
            lib.synth_normal_bf16_rows.argtypes = [u64, u64, u64, i64, i64, i64, dbl, dbl, vp, i64]
            for f in (lib.synth_u64, lib.synth_uniform_f64, lib.synth_normal_f32,
                      lib.synth_normal_bf16, lib.synth_normal_bf16_rows):
                f.restype = None
            _lib_handle = lib
    return _lib_handle


def stream_id(tag: int, seq: int = 0, layer: int = 0) -> int:
    return (tag << 56) | ((seq & 0xFFFF) << 40) | ((layer & 0xFFFF) << 24)


def u64(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, np.uint64)
    _lib().synth_u64(seed, stream, start, count, out.ctypes.data)
    return out


def uniform(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    out = np.empty(count, np.float64)
    _lib().synth_uniform_f64(seed, stream, start, count, out.ctypes.data)
    return out


def normal_f32(seed: int, stream: int, start: int, count: int, mean=0.0, std=1.0) -> np.ndarray:
    out = np.empty(count, np.float32)
    _lib().synth_normal_f32(seed, stream, start, count, float(mean), float(std), out.ctypes.data)
    return out


def normal_bf16(seed: int, stream: int, start: int, count: int, mean=0.0, std=1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(mean, std) draws rounded float -> bf16 RNE."""
    out = np.empty(count, np.uint16)
    _lib().synth_normal_bf16(seed, stream, start, count, float(mean), float(std), out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------------------
# workload shapes
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    """One synthetic DMS workload: model shape, sequence lengths and logit law."""
    name: str
    index: int               # position in the list of workloads; seed = 20261203 + index
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    n_seqs: int
    ctx_len: int             # prompt length (for ragged batches: lower bound)
    gen_len: int             # decode steps after the prompt
    keep_law: str            # "normal" | "uniform_mu" | "beta"
    keep_mu: float = -1.2    # mean of the keep score for keep_law == "normal"
    ctx_max: int = 0         # ragged batches: prompt length ~ U{ctx_len..ctx_max}
    layer_repeats: int = 1   # prefill workload: one layer's inputs prefilled this many times
    prefill_only: bool = False

    @property
    def seed(self) -> int:
        return 20261203 + self.index

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_d64_ctx1024", 0, n_layers=1, n_q_heads=32, n_kv_heads=8, head_dim=64,
                 window=256, n_seqs=1, ctx_len=1024, gen_len=16, keep_law="normal"),
        Workload("llama3.2-1b_ctx8192", 1, n_layers=16, n_q_heads=32, n_kv_heads=8, head_dim=64,
                 window=512, n_seqs=1, ctx_len=8192, gen_len=128, keep_law="normal"),
        Workload("qwen3-8b_ctx8192", 2, n_layers=36, n_q_heads=32, n_kv_heads=8, head_dim=128,
                 window=512, n_seqs=1, ctx_len=8192, gen_len=128, keep_law="uniform_mu"),
        Workload("qwen3-8b_batch32_ragged", 3, n_layers=36, n_q_heads=32, n_kv_heads=8,
                 head_dim=128, window=512, n_seqs=32, ctx_len=4096, ctx_max=32768, gen_len=64,
                 keep_law="beta"),
        Workload("qwen3-8b_prefill32k", 4, n_layers=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
                 window=512, n_seqs=1, ctx_len=32768, gen_len=0, keep_law="normal",
                 layer_repeats=36, prefill_only=True),
    ]
}


class SynthInputs:
    """Generates the inputs of one workload on demand.

    Layouts (bf16 as uint16 bit patterns, logits float32):
      q rows    [n][n_q_heads][head_dim]
      k, v rows [n][n_kv_heads][head_dim]
      logits    [n][n_kv_heads]
    for positions p0 .. p0+n-1 of (seq, layer).
    """

    def __init__(self, wl: Workload, marks: str = "keep_score", seed: Optional[int] = None):
        if marks not in ("keep_score", "literal"):
            raise ValueError("marks must be 'keep_score' or 'literal'")
        self.wl = wl
        self.marks = marks
        self.seed = wl.seed if seed is None else int(seed)
        self._mu = self._draw_mu()

    # per-(layer, kv-head) mean of the keep score
    def _draw_mu(self) -> np.ndarray:
        wl = self.wl
        L, H = wl.n_layers, wl.n_kv_heads
        if wl.keep_law == "normal":
            return np.full((L, H), wl.keep_mu, np.float64)
        if wl.keep_law == "uniform_mu":
            u = uniform(self.seed, stream_id(TAG_MU), 0, L * H)
            return (-2.0 + 2.0 * u).reshape(L, H)
        if wl.keep_law == "beta":
            # Beta(2, 14) = 2nd smallest of 15 iid uniforms; keep rate p -> mu = Phi^-1(p)
            u = uniform(self.seed, stream_id(TAG_BETA), 0, L * H * 15).reshape(L * H, 15)
            p = np.sort(u, axis=1)[:, 1]
            nd = statistics.NormalDist()
            return np.array([nd.inv_cdf(float(x)) for x in p], np.float64).reshape(L, H)
        raise ValueError(wl.keep_law)

    @property
    def mu(self) -> np.ndarray:
        return self._mu

    def keep_rate(self) -> np.ndarray:
        """Expected keep probability per (layer, kv-head): P(score >= 0)."""
        nd = statistics.NormalDist()
        return np.vectorize(lambda m: nd.cdf(m))(self._mu)

    def ctx_lens(self) -> np.ndarray:
        wl = self.wl
        if wl.ctx_max:
            u = uniform(self.seed, stream_id(TAG_CTX), 0, wl.n_seqs)
            span = wl.ctx_max - wl.ctx_len + 1
            return (wl.ctx_len + np.floor(u * span)).astype(np.int64)
        return np.full(wl.n_seqs, wl.ctx_len, np.int64)

    def _layer_of(self, layer: int) -> int:
        # the prefill workload reuses one layer's inputs for every repeat
        return 0 if self.wl.layer_repeats > 1 else layer

    def q(self, seq: int, layer: int, p0: int, n: int) -> np.ndarray:
        wl = self.wl
        row = wl.n_q_heads * wl.head_dim
        s = stream_id(TAG_Q, seq, self._layer_of(layer))
        return normal_bf16(self.seed, s, p0 * row, n * row).reshape(n, wl.n_q_heads, wl.head_dim)

    def k(self, seq: int, layer: int, p0: int, n: int) -> np.ndarray:
        wl = self.wl
        row = wl.n_kv_heads * wl.head_dim
        s = stream_id(TAG_K, seq, self._layer_of(layer))
        return normal_bf16(self.seed, s, p0 * row, n * row).reshape(n, wl.n_kv_heads, wl.head_dim)

    def v(self, seq: int, layer: int, p0: int, n: int) -> np.ndarray:
        wl = self.wl
        row = wl.n_kv_heads * wl.head_dim
        s = stream_id(TAG_V, seq, self._layer_of(layer))
        return normal_bf16(self.seed, s, p0 * row, n * row).reshape(n, wl.n_kv_heads, wl.head_dim)

    def logits(self, seq: int, layer: int, p0: int, n: int) -> np.ndarray:
        wl = self.wl
        H = wl.n_kv_heads
        lay = self._layer_of(layer)
        z = np.empty(n * H, np.float64)
        _lib()  # ensure loaded
        zf = np.empty(n * H, np.float32)
        # the score noise is drawn as float32 N(0,1); the score is mu + noise
        _lib().synth_normal_f32(self.seed, stream_id(TAG_SCORE, seq, lay), p0 * H, n * H,
                                0.0, 1.0, zf.ctypes.data)
        z[:] = zf
        score = self._mu[lay][None, :] + z.reshape(n, H)
        lam = -score if self.marks == "keep_score" else score
        return lam.astype(np.float32)
