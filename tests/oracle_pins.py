"""Checks that tie the DMS oracle to facts that do not come from the oracle.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with one of:

* a hand-derived table of live sets (tests/golden/live_sets_hand.json);
* an event-driven simulation of delayed eviction written here independently
  (a token enters at its own step; a marked token schedules its own removal for
  step s + w);
* closed forms: the live count, invariants of the live set, o_t = v_t when only
  one key is visible, the plain mean when all scores are equal, a per-position
  histogram with one-hot values, the kv-head a q head reads when values are
  constant per kv head;
* the bytes a compact store holds: the KV-memory figures the FastDMS
  announcement prints (tests/golden/fastdms_memory_table.json), the byte sizes
  of the rows the live sets retain, and the pages a slot free-list simulation
  fills;
* library routines: torch's scaled_dot_product_attention in float64 with a
  causal mask (eviction disabled: the 1M-token window the FastDMS quality
  method uses as its reference), with a band mask (every token marked: a
  sliding window), and with an arbitrary mask taken from the event-driven
  simulation (the general case).

The functions are plain so that tests can also run them against deliberately
broken copies of the oracle (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import json
import os
from collections import defaultdict

import numpy as np
import torch

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# independent reference pieces
# ---------------------------------------------------------------------------

def simulate_live_sets(marks_col, window):
    """Event-driven delayed eviction for one head: V(t) for t = 0..T-1."""
    live = set()
    removals = defaultdict(list)
    out = []
    for t, m in enumerate(marks_col):
        for s in removals.pop(t, []):
            live.discard(s)
        live.add(t)
        if m:
            removals[t + window].append(t)
        out.append(sorted(live))
    return out


def _bf16(shape, seed, stream):
    n = int(np.prod(shape))
    return synth.normal_bf16(seed, stream, 0, n).reshape(shape)


def _f64(bits):
    return synth.bf16_to_f32(bits).astype(np.float64)


def _sdpa(q_bits, k_bits, v_bits, mask):
    """torch SDPA in float64; q [T,Hq,D], k/v [T,Hkv,D] bf16 bits; mask [T,T] bool
    (True = attend) shared by all heads.  kv heads are repeated for GQA."""
    T, Hq, D = q_bits.shape
    Hkv = k_bits.shape[1]
    q = torch.from_numpy(_f64(q_bits)).permute(1, 0, 2).unsqueeze(0)
    k = torch.from_numpy(_f64(k_bits)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0).unsqueeze(0)
    v = torch.from_numpy(_f64(v_bits)).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=torch.from_numpy(mask))
    return o.squeeze(0).permute(1, 0, 2).numpy()


def _sdpa_per_kv_head(q_bits, k_bits, v_bits, masks):
    """Like _sdpa but with one [T,T] mask per kv head (masks [Hkv,T,T])."""
    T, Hq, D = q_bits.shape
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    out = np.empty((T, Hq, D))
    for h in range(Hkv):
        sl = slice(h * G, (h + 1) * G)
        out[:, sl, :] = _sdpa(q_bits[:, sl, :], k_bits[:, h:h + 1, :], v_bits[:, h:h + 1, :], masks[h])
    return out


def _all_positions(T):
    return np.arange(T, dtype=np.int64)


# ---------------------------------------------------------------------------
# pins on marks and live sets
# ---------------------------------------------------------------------------

def pin_marks(orc):
    lg = np.array([-1.0, 0.0, -0.0, 1e-30, 2.5, -1e-30, np.float32(1.4e-45)], np.float32)
    assert orc.marks(lg).tolist() == [0, 0, 0, 1, 1, 0, 1]


def pin_live_sets_hand(orc):
    with open(os.path.join(GOLDEN, "live_sets_hand.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        m = np.array(c["marks"], np.uint8)
        for t, expect in enumerate(c["live"]):
            got = orc.live_positions(t, c["window"], m).tolist()
            assert got == expect, (c["name"], t, got, expect)


def pin_live_sets_brute_force(orc, max_T=10):
    """Every mark pattern of length T <= max_T and every window 1..T+1."""
    for T in range(1, max_T + 1):
        for bits in range(1 << T):
            m = np.array([(bits >> i) & 1 for i in range(T)], np.uint8)
            for w in range(1, T + 2):
                sim = simulate_live_sets(m, w)
                for t in range(T):
                    got = orc.live_positions(t, w, m).tolist()
                    assert got == sim[t], (T, bits, w, t, got, sim[t])


def pin_live_count_closed_form(orc):
    """n(t) = #{s <= t-w : unmarked} + min(t+1, w), and the invariants of V(t)."""
    rng = np.random.default_rng(7)
    for w in (1, 2, 5, 64, 300):
        for rate in (0.0, 0.3, 0.885, 1.0):
            T = 400
            m = (rng.random(T) < rate).astype(np.uint8)
            prev = None
            for t in range(T):
                V = orc.live_positions(t, w, m)
                n = len(V)
                closed = int(np.sum(m[:max(t - w + 1, 0)] == 0)) + min(t + 1, w)
                assert n == closed, (w, rate, t, n, closed)
                assert n == orc.live_count(t, w, m)
                assert n <= int(np.sum(m[:t + 1] == 0)) + w
                assert n >= min(t + 1, w)
                if prev is not None:
                    added = set(V.tolist()) - set(prev.tolist())
                    removed = set(prev.tolist()) - set(V.tolist())
                    assert added == {t}
                    assert removed <= {t - w}
                    assert n - len(prev) in (0, 1)
                prev = V


# ---------------------------------------------------------------------------
# pins on attention outputs
# ---------------------------------------------------------------------------

def _case(T=48, Hq=8, Hkv=2, D=16, seed=11):
    q = _bf16((T, Hq, D), seed, 1)
    k = _bf16((T, Hkv, D), seed, 2)
    v = _bf16((T, Hkv, D), seed, 3)
    return q, k, v


def pin_eviction_disabled_is_causal(orc):
    """Window of 2^20 positions (the 1M-token reference window): plain causal
    attention, whatever the marks."""
    q, k, v = _case()
    T, Hkv = k.shape[0], k.shape[1]
    marks = (np.arange(T * Hkv).reshape(T, Hkv) % 3 != 0).astype(np.uint8)
    got = orc.attend(q, _all_positions(T), k, v, marks, 1 << 20)
    ref = _sdpa(q, k, v, np.tril(np.ones((T, T), bool)))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_unmarked_is_causal(orc):
    q, k, v = _case(seed=12)
    T, Hkv = k.shape[0], k.shape[1]
    marks = np.zeros((T, Hkv), np.uint8)
    got = orc.attend(q, _all_positions(T), k, v, marks, 3)
    ref = _sdpa(q, k, v, np.tril(np.ones((T, T), bool)))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_all_marked_is_sliding_window(orc):
    q, k, v = _case(seed=13)
    T, Hkv = k.shape[0], k.shape[1]
    marks = np.ones((T, Hkv), np.uint8)
    for w in (1, 4, 17):
        tt, ss = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
        band = (ss <= tt) & (ss > tt - w)
        got = orc.attend(q, _all_positions(T), k, v, marks, w)
        ref = _sdpa(q, k, v, band)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_general_mask_from_simulation(orc):
    """Random marks per kv head: SDPA with the mask the event-driven simulation gives."""
    q, k, v = _case(T=64, seed=14)
    T, Hkv = k.shape[0], k.shape[1]
    rng = np.random.default_rng(3)
    marks = (rng.random((T, Hkv)) < 0.6).astype(np.uint8)
    for w in (1, 5, 16):
        masks = np.zeros((Hkv, T, T), bool)
        for h in range(Hkv):
            for t, V in enumerate(simulate_live_sets(marks[:, h], w)):
                masks[h, t, V] = True
        got = orc.attend(q, _all_positions(T), k, v, marks, w)
        ref = _sdpa_per_kv_head(q, k, v, masks)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def pin_single_visible_key(orc):
    """All marked, w = 1: only the query's own token is visible, o_t = v_t
    exactly (one softmax weight, equal to 1).  Also pins the GQA mapping."""
    q, k, v = _case(seed=15)
    T, Hkv, D = k.shape
    Hq = q.shape[1]
    marks = np.ones((T, Hkv), np.uint8)
    got = orc.attend(q, _all_positions(T), k, v, marks, 1)
    G = Hq // Hkv
    for hq in range(Hq):
        assert np.array_equal(got[:, hq, :], _f64(v[:, hq // G, :])), hq


def pin_zero_query_is_mean(orc):
    """q = 0: every visible score is 0, so o_t is the plain mean of the visible
    values; the visible sets come from the event-driven simulation."""
    _, k, v = _case(T=40, seed=16)
    T, Hkv, D = k.shape
    Hq = 8
    q = np.zeros((T, Hq, D), np.uint16)
    rng = np.random.default_rng(5)
    marks = (rng.random((T, Hkv)) < 0.5).astype(np.uint8)
    w = 6
    got = orc.attend(q, _all_positions(T), k, v, marks, w)
    vf = _f64(v)
    G = Hq // Hkv
    for h in range(Hkv):
        sets = simulate_live_sets(marks[:, h], w)
        for t in range(T):
            ref = vf[sets[t], h, :].mean(axis=0)
            for g in range(G):
                np.testing.assert_allclose(got[t, h * G + g], ref, rtol=1e-13, atol=1e-14)


def pin_one_hot_histogram(orc):
    """q = 0 and v_s = e_(s mod D): o_t[d] = #{s in V(t): s mod D = d} / |V(t)|."""
    T, Hkv, D, Hq = 70, 2, 8, 4
    k = _bf16((T, Hkv, D), 17, 2)
    v = np.zeros((T, Hkv, D), np.uint16)
    one = np.array([1.0], np.float32).view(np.uint32)[0] >> 16
    for s in range(T):
        v[s, :, s % D] = one
    q = np.zeros((T, Hq, D), np.uint16)
    rng = np.random.default_rng(9)
    marks = (rng.random((T, Hkv)) < 0.7).astype(np.uint8)
    w = 9
    got = orc.attend(q, _all_positions(T), k, v, marks, w)
    G = Hq // Hkv
    for h in range(Hkv):
        sets = simulate_live_sets(marks[:, h], w)
        for t in range(T):
            hist = np.bincount(np.array(sets[t]) % D, minlength=D) / len(sets[t])
            for g in range(G):
                np.testing.assert_allclose(got[t, h * G + g], hist, rtol=0, atol=1e-15)


def pin_gqa_constant_values(orc):
    """Values constant per kv head (powers of two): o = that constant exactly, so
    each q head must read kv head hq // (Hq/Hkv)."""
    T, Hq, Hkv, D = 30, 12, 4, 8
    q = _bf16((T, Hq, D), 18, 1)
    k = _bf16((T, Hkv, D), 18, 2)
    consts = [0.5, 1.0, 2.0, 4.0]
    v = np.zeros((T, Hkv, D), np.uint16)
    for h, c in enumerate(consts):
        v[:, h, :] = np.array([c], np.float32).view(np.uint32)[0] >> 16
    rng = np.random.default_rng(2)
    marks = (rng.random((T, Hkv)) < 0.5).astype(np.uint8)
    got = orc.attend(q, _all_positions(T), k, v, marks, 4)
    G = Hq // Hkv
    for hq in range(Hq):
        assert np.all(got[:, hq, :] == consts[hq // G]), hq


def pin_query_subset_matches_rows(orc):
    """A query evaluated alone gives the same row as within a full pass (each
    row depends only on its own position)."""
    q, k, v = _case(T=33, seed=19)
    T, Hkv = k.shape[0], k.shape[1]
    marks = (np.arange(T * Hkv).reshape(T, Hkv) % 2).astype(np.uint8)
    full = orc.attend(q, _all_positions(T), k, v, marks, 5)
    pick = np.array([0, 7, 32], np.int64)
    sub = orc.attend(q[pick], pick, k, v, marks, 5)
    assert np.array_equal(sub, full[pick])


# ---------------------------------------------------------------------------
# pins on the bytes a compact store holds
# ---------------------------------------------------------------------------

def simulate_slots(marks_col, window):
    """Single-token decode of one head with an explicit slot free list: token t
    takes the slot of the token leaving at step t (t - w, if marked), else a
    fresh slot.  Returns the slots in use after each step (the high-water mark)."""
    free, slot_of, used, out = [], {}, 0, []
    for t, m in enumerate(marks_col):
        u = t - window
        if u >= 0 and marks_col[u]:
            free.append(slot_of.pop(u))
        if free:
            slot_of[t] = free.pop()
        else:
            slot_of[t] = used
            used += 1
        out.append(used)
    return out


def pin_kv_bytes_reproduce_memory_table(orc):
    """Eviction disabled, the Llama-3.2-1B shape: the store's bytes for 10240
    token slots round to the FastDMS memory table's vLLM BF16 figure, and the
    code bytes of the FP8 rows (without the row scales) to its vLLM FP8 figure;
    the job's own 8320 tokens do not reproduce the printed value."""
    with open(os.path.join(GOLDEN, "fastdms_memory_table.json")) as f:
        tab = json.load(f)
    sh, printed = tab["shape"], tab["printed_gib"]
    L, H, D = sh["n_layers"], sh["n_kv_heads"], sh["head_dim"]
    slots = 10240
    marks = np.zeros((slots, H), np.uint8)
    live, alloc, dense = orc.kv_bytes(slots - 1, 1 << 20, marks, D)
    assert live == dense == alloc
    assert round(L * live / 2**30, 3) == printed["vllm_bf16"]
    _, scales = orc.quantize_rows(np.zeros((1, D), np.uint16))
    live8, _, _ = orc.kv_bytes(slots - 1, 1 << 20, marks, D, fp8=True)
    codes_only = live8 - slots * H * 2 * scales.itemsize
    assert round(L * codes_only / 2**30, 3) == printed["vllm_fp8"]
    job = sh["ctx_len"] + sh["gen_len"]
    live_job, _, _ = orc.kv_bytes(job - 1, 1 << 20, marks[:job], D)
    assert round(L * live_job / 2**30, 3) != printed["vllm_bf16"]


def pin_kv_bytes_are_the_rows_held(orc):
    """Live bytes = the bytes of the K and V rows the live sets retain (rows of
    the inputs for bf16 stores, the quantiser's codes and scales for FP8),
    with the live sets from the event-driven simulation."""
    rng = np.random.default_rng(21)
    for D, H, T, w in ((64, 3, 90, 7), (128, 2, 140, 33)):
        k = _bf16((T, H, D), 23, 2)
        v = _bf16((T, H, D), 23, 3)
        k8, ks = orc.quantize_rows(k)
        v8, vs = orc.quantize_rows(v)
        marks = (rng.random((T, H)) < 0.6).astype(np.uint8)
        sets = [simulate_live_sets(marks[:, h], w) for h in range(H)]
        for t in (0, w - 1, w, T // 2, T - 1):
            held = sum(k[s, h].nbytes + v[s, h].nbytes for h in range(H) for s in sets[h][t])
            held8 = sum(k8[s, h].nbytes + ks[s, h].nbytes + v8[s, h].nbytes + vs[s, h].nbytes
                        for h in range(H) for s in sets[h][t])
            assert orc.kv_bytes(t, w, marks, D)[0] == held, (D, t)
            assert orc.kv_bytes(t, w, marks, D, fp8=True)[0] == held8, (D, t)
            dense = sum(k[s, h].nbytes + v[s, h].nbytes for h in range(H) for s in range(t + 1))
            assert orc.kv_bytes(t, w, marks, D)[2] == dense, (D, t)
            assert orc.kv_bytes(t, w, marks, D, fp8=True)[2] == dense, (D, t)


def pin_kv_bytes_allocated_pages(orc):
    """Allocated bytes = whole pages of 64 slots over the slots a head has used,
    with the slots from the free-list simulation (a freed slot is taken by the
    next token, so no head ever leaves a hole)."""
    rng = np.random.default_rng(22)
    D, H, T = 64, 4, 700
    row = _bf16((1, 1, D), 24, 2)[0, 0]
    for w in (1, 16, 130):
        for rate in (0.0, 0.5, 0.95, 1.0):
            marks = (rng.random((T, H)) < rate).astype(np.uint8)
            used = [simulate_slots(marks[:, h], w) for h in range(H)]
            for t in (0, 63, 64, 65, 300, T - 1):
                pages = sum(-(-used[h][t] // 64) for h in range(H))
                live = sum(used[h][t] for h in range(H))
                got = orc.kv_bytes(t, w, marks, D)
                assert got[1] == pages * 64 * 2 * row.nbytes, (w, rate, t)
                assert got[0] == live * 2 * row.nbytes, (w, rate, t)
            assert orc.kv_bytes(T - 1, w, marks, D, page_slots=32)[1] == \
                sum(-(-used[h][T - 1] // 32) for h in range(H)) * 32 * 2 * row.nbytes


def pin_kv_bytes_extremes(orc):
    """Nothing ever expires (the 1M-token window, or no marks): live = dense.
    Every token marked: a window of min(t+1, w) rows per head."""
    T, H, D = 300, 5, 128
    rng = np.random.default_rng(25)
    some = (rng.random((T, H)) < 0.5).astype(np.uint8)
    for t in (0, 10, 299):
        assert orc.kv_bytes(t, 1 << 20, some, D)[0] == orc.kv_bytes(t, 1 << 20, some, D)[2]
        assert orc.kv_bytes(t, 3, np.zeros((T, H), np.uint8), D)[0] == orc.kv_bytes(t, 3, some, D)[2]
        for w in (1, 7, 64):
            live, alloc, _ = orc.kv_bytes(t, w, np.ones((T, H), np.uint8), D)
            assert live == H * min(t + 1, w) * 2 * 2 * D
            assert alloc == H * 64 * 2 * 2 * D


ALL_PINS = [
    pin_marks,
    pin_live_sets_hand,
    pin_live_sets_brute_force,
    pin_live_count_closed_form,
    pin_eviction_disabled_is_causal,
    pin_unmarked_is_causal,
    pin_all_marked_is_sliding_window,
    pin_general_mask_from_simulation,
    pin_single_visible_key,
    pin_zero_query_is_mean,
    pin_one_hot_histogram,
    pin_gqa_constant_values,
    pin_query_subset_matches_rows,
    pin_kv_bytes_reproduce_memory_table,
    pin_kv_bytes_are_the_rows_held,
    pin_kv_bytes_allocated_pages,
    pin_kv_bytes_extremes,
]
