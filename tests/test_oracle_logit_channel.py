"""Pins of the oracle's eviction logits read from a K channel, on the CPU.

The logit of (token, kv head h) is channel c of the token's K row for h.  Pins:
the values equal the bf16 values at [..., h, c] decoded independently (bit shift
into a float32); a channel of all +1 marks every token (a sliding window of w),
all -1 marks none (full causal attention); planted indexing mistakes (a
neighbouring channel, heads and tokens swapped in the row index) each fail."""
import os

import numpy as np
import pytest

import oracle
import synth


def bf16_value(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_values_are_the_channel_of_each_row():
    rng = np.random.default_rng(3)
    for shape, c in [((40, 3, 64), 0), ((17, 8, 128), 127), ((5, 2, 4, 64), 33)]:
        k = rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)
        k[..., :] &= 0x7F7F  # finite values only
        got = oracle.default().k_channel_logits(k, c)
        assert got.shape == shape[:-1]
        assert np.array_equal(got, bf16_value(k[..., c]))


def test_channel_sign_sets_the_marks():
    T, H, D, w, c = 50, 2, 64, 7, 5
    k = synth.normal_bf16(9, synth.stream_id(synth.TAG_K), 0, T * H * D).reshape(T, H, D)
    o = oracle.default()
    k[:, 0, c] = 0x3F80  # +1: every token marked -> a window of the last w tokens
    k[:, 1, c] = 0xBF80  # -1: nothing marked -> every token stays
    m = o.marks(o.k_channel_logits(k, c))
    assert m[:, 0].all() and not m[:, 1].any()
    for t in range(T):
        assert o.live_count(t, w, m[:, 0]) == min(t + 1, w)
        assert o.live_count(t, w, m[:, 1]) == t + 1


MUTANTS = {
    "neighbouring_channel": ("out[r * n_kv_heads + h] = (float)bf16_bits_to_double(k[(r * n_kv_heads + h) * d + c]);",
                             "out[r * n_kv_heads + h] = (float)bf16_bits_to_double(k[(r * n_kv_heads + h) * d + (c + 1) % d]);"),
    "heads_and_rows_swapped": ("out[r * n_kv_heads + h] = (float)bf16_bits_to_double(k[(r * n_kv_heads + h) * d + c]);",
                               "out[r * n_kv_heads + h] = (float)bf16_bits_to_double(k[(h * n_rows + r) * d + c]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_indexing_mistakes_are_caught(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "dms_oracle.c")).read()
    old, new = MUTANTS[name]
    assert old in src
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    so = str(tmp_path / "libmut.so")
    oracle.build(force=True, src=str(mut), so=so)
    mo = oracle.Oracle(oracle.load(so))
    saved = oracle.default
    try:
        oracle.default = lambda: mo
        with pytest.raises(AssertionError):
            test_values_are_the_channel_of_each_row()
    finally:
        oracle.default = saved
