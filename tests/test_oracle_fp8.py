"""Pins of the oracle's FP8 (OCP E4M3) K/V definition, on the CPU.

E4M3 (OCP 8-bit floating point, E4M3 variant): sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 holds zero and the subnormals
(quantum 2^-9), S.1111.111 is NaN, there is no infinity and the largest finite
value is 448.  The pins check the oracle's value table against anchor values of
that definition and against its structure (monotone codes, 8 equal steps per
binade, sign symmetry), its encoder against every code (round trip), every
rounding tie (to the even code) and saturation, its row quantiser against the
invariants of "amax / 448" scaling, and its FP8 attention against torch SDPA in
float64 on the dequantised K/V.  Planted mistakes (truncating or ties-away
rounding, a wrong maximum, a dropped scale) must each fail a pin.
"""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from oracle_pins import simulate_live_sets

FINITE_POS = list(range(0x00, 0x7F))  # 0x00 .. 0x7e


def table(o=None):
    o = o or oracle.default()
    return np.array([o.e4m3_value(c) for c in range(256)])


def test_anchor_values():
    o = oracle.default()
    anchors = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x40: 2.0,
               0x77: 240.0, 0x7E: 448.0, 0xC0: -2.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in anchors.items():
        assert o.e4m3_value(c) == v, hex(c)
    assert math.copysign(1.0, o.e4m3_value(0x80)) == -1.0 and o.e4m3_value(0x80) == 0.0
    assert math.isnan(o.e4m3_value(0x7F)) and math.isnan(o.e4m3_value(0xFF))


def test_table_structure():
    t = table()
    pos = t[FINITE_POS]
    assert np.all(np.diff(pos) > 0)                               # strictly increasing codes
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])             # sign symmetry
    assert np.all(np.diff(pos[:9]) == 2.0 ** -9)                   # subnormal quantum up to 2^-6
    for e in range(1, 16):                                         # 8 equal steps per binade
        lo = 8 * e
        vals = t[lo:lo + 8] if e < 15 else t[lo:lo + 7]
        steps = np.diff(np.concatenate([vals, [2.0 ** (e - 6)]])) if e < 15 else np.diff(vals)
        assert np.allclose(steps, 2.0 ** (e - 7) / 8), e


def test_encode_round_trip_every_code():
    o = oracle.default()
    t = table(o)
    for c in list(range(0x00, 0x7F)) + list(range(0x80, 0xFF)):
        assert o.e4m3_encode(float(t[c])) == c, hex(c)


def test_encode_ties_to_even_and_nearest():
    o = oracle.default()
    t = table(o)
    for c in range(0x00, 0x7E):
        a, b = t[c], t[c + 1]
        mid = np.float32((a + b) / 2)
        assert float(mid) == (a + b) / 2                           # exact in fp32
        even = c if c % 2 == 0 else c + 1
        assert o.e4m3_encode(float(mid)) == even, hex(c)
        assert o.e4m3_encode(-float(mid)) == 0x80 | even, hex(c)
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(np.inf))
        assert o.e4m3_encode(float(below)) == c, hex(c)
        assert o.e4m3_encode(float(above)) == c + 1, hex(c)


def test_encode_saturates_and_keeps_nan():
    o = oracle.default()
    for x in [448.5, 464.0, 480.0, 1e6, 3.4e38, float("inf")]:
        assert o.e4m3_encode(x) == 0x7E
        assert o.e4m3_encode(-x) == 0xFE
    assert o.e4m3_encode(float("nan")) == 0x7F
    assert o.e4m3_encode(2.0 ** -10) == 0x00 and o.e4m3_encode(-(2.0 ** -10)) == 0x80
    assert o.e4m3_encode(1.5 * 2.0 ** -10) == 0x01


def _rne_bf16(x):
    u = x.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_quantize_rows_invariants():
    o = oracle.default()
    t = table(o)
    rng = np.random.default_rng(1)
    x = _rne_bf16((rng.standard_normal((300, 128)) * rng.choice([1e-3, 1.0, 50.0], (300, 1))).astype(np.float32))
    codes, scales = o.quantize_rows(x)
    xf = synth.bf16_to_f32(x).astype(np.float32)
    amax = np.max(np.abs(xf), axis=1)
    assert np.array_equal(scales, amax / np.float32(448.0))        # fp32 amax / 448
    i = np.argmax(np.abs(xf), axis=1)
    top = codes[np.arange(300), i]
    assert np.all((top & 0x7F) == 0x7E)                            # the largest element maps to +-448
    deq = t[codes] * scales[:, None].astype(np.float64)
    err = np.abs(deq - xf)
    assert np.all(err <= 2.0 ** -4 * np.abs(xf) + 2.0 ** -10 * scales[:, None] + 1e-30)
    assert np.all(np.sign(deq[deq != 0]) == np.sign(xf[deq != 0]))


def test_quantize_exact_rows_and_zero_rows():
    o = oracle.default()
    t = table(o)
    rng = np.random.default_rng(2)
    picks = rng.choice(np.array(FINITE_POS + [0x80 | c for c in FINITE_POS[1:]]), (16, 64))
    picks[:, 0] = 0x7E                                             # amax = 448 * 2^k
    k = rng.integers(-20, 20, 16)
    vals = t[picks] * (2.0 ** k)[:, None]
    x = _rne_bf16(vals.astype(np.float32))
    assert np.array_equal(synth.bf16_to_f32(x).astype(np.float64), vals)  # exact in bf16
    codes, scales = o.quantize_rows(x)
    assert np.array_equal(scales.astype(np.float64), 2.0 ** k)
    assert np.array_equal(t[codes] * scales[:, None].astype(np.float64), vals)
    z = np.zeros((3, 64), np.uint16)
    codes, scales = o.quantize_rows(z)
    assert np.all(scales == 1.0) and np.all(codes == 0)


def _sdpa_fp8(q, k8, ks, v8, vs, mask_fn, T, window):
    import torch
    t = table()
    hq, d = q.shape[1], q.shape[2]
    hkv = k8.shape[1]
    kd = torch.from_numpy(t[k8] * ks[..., None].astype(np.float64))
    vd = torch.from_numpy(t[v8] * vs[..., None].astype(np.float64))
    qd = torch.from_numpy(synth.bf16_to_f32(q).astype(np.float64))
    g = hq // hkv
    kq = kd.repeat_interleave(g, dim=1).permute(1, 0, 2)
    vq = vd.repeat_interleave(g, dim=1).permute(1, 0, 2)
    outs = []
    for hi in range(hq):
        h = hi // g
        m = torch.from_numpy(mask_fn(h))
        outs.append(torch.nn.functional.scaled_dot_product_attention(
            qd[:, hi][None], kq[hi][None], vq[hi][None], attn_mask=m[None]).numpy()[0])
    return np.stack(outs, axis=1)


@pytest.mark.parametrize("case", ["disabled", "all_marked", "random"])
def test_attend_fp8_matches_sdpa_on_dequantised_kv(case):
    o = oracle.default()
    T, Hq, Hkv, D, w = 70, 4, 2, 64, 9
    seed = 77
    q = synth.normal_bf16(seed, synth.stream_id(synth.TAG_Q), 0, T * Hq * D).reshape(T, Hq, D)
    k = synth.normal_bf16(seed, synth.stream_id(synth.TAG_K), 0, T * Hkv * D).reshape(T, Hkv, D)
    v = synth.normal_bf16(seed, synth.stream_id(synth.TAG_V), 0, T * Hkv * D).reshape(T, Hkv, D)
    k8, ks = o.quantize_rows(k)
    v8, vs = o.quantize_rows(v)
    if case == "disabled":
        marks = np.ones((T, Hkv), np.uint8)
        window = 1 << 20
    elif case == "all_marked":
        marks = np.ones((T, Hkv), np.uint8)
        window = w
    else:
        marks = (synth.uniform(seed, synth.stream_id(synth.TAG_SCORE), 0, T * Hkv).reshape(T, Hkv) < 0.5
                 ).astype(np.uint8)
        window = w
    got = o.attend_fp8(q, np.arange(T), k8, ks, v8, vs, marks, window)

    def mask_fn(h):
        live = simulate_live_sets(marks[:, h], window)
        m = np.zeros((T, T), bool)
        for t_, s_ in enumerate(live):
            m[t_, list(s_)] = True
        return m
    ref = _sdpa_fp8(q, k8, ks, v8, vs, mask_fn, T, window)
    assert np.allclose(got, ref, rtol=1e-10, atol=1e-12)


MUTANTS = {
    "truncating_rounding": ("if (d < best_d || (d == best_d && (c & 1) == 0))",
                            "if (dms_oracle_e4m3_value((uint8_t)c) <= a)"),
    "ties_away_from_zero": ("(d == best_d && (c & 1) == 0)", "(d == best_d)"),
    "wrong_maximum": ("amax / 448.0f", "amax / 240.0f"),
    "scale_dropped_in_keys": ("(table[krow[d]] * kscale)", "(table[krow[d]])"),
    "subnormal_exponent": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_fp8_mistakes_are_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "dms_oracle.c")).read()
    old, new = MUTANTS[name]
    assert old in src
    mut_src = tmp_path / "mut.c"
    mut_src.write_text(src.replace(old, new))
    so = str(tmp_path / "libmut.so")
    oracle.build(force=True, src=str(mut_src), so=so)
    mo = oracle.Oracle(oracle.load(so))
    checks = [test_anchor_values, test_table_structure, test_encode_round_trip_every_code,
              test_encode_ties_to_even_and_nearest, test_encode_saturates_and_keeps_nan,
              test_quantize_rows_invariants, test_quantize_exact_rows_and_zero_rows]
    failed = False
    saved = oracle.default
    try:
        oracle.default = lambda: mo
        for fn in checks:
            try:
                fn()
            except AssertionError:
                failed = True
                break
        if not failed:
            for case in ["disabled", "random"]:
                try:
                    test_attend_fp8_matches_sdpa_on_dequantised_kv(case)
                except AssertionError:
                    failed = True
                    break
    finally:
        oracle.default = saved
    assert failed, "mutant %s passed every FP8 pin" % name
