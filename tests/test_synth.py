"""CPU tests of the seeded input generator (shared by both sides)."""
import numpy as np

import synth


def test_counter_slices_agree():
    full = synth.normal_bf16(5, 9, 0, 4096)
    part = synth.normal_bf16(5, 9, 1000, 500)
    assert np.array_equal(full[1000:1500], part)


def test_deterministic_and_seed_sensitive():
    a = synth.normal_bf16(5, 9, 0, 1000)
    assert np.array_equal(a, synth.normal_bf16(5, 9, 0, 1000))
    assert not np.array_equal(a, synth.normal_bf16(6, 9, 0, 1000))
    assert not np.array_equal(a, synth.normal_bf16(5, 10, 0, 1000))


def test_splitmix64_reference_values():
    # SplitMix64 started from state 0 gives 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
    # 0x06C45D188009454F as its first outputs (the generator's reference C code).
    out = np.empty(3, np.uint64)
    synth._lib().synth_raw_u64(0, 0, 3, out.ctypes.data)
    assert [int(x) for x in out] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_normal_moments_and_bf16_rounding():
    x = synth.normal_f32(1, 2, 0, 200000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    b = synth.normal_bf16(1, 2, 0, 200000)
    # bf16 values are the float values rounded to nearest even
    u = x.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(b, rne)


def test_workload_keep_rates():
    w = synth.WORKLOADS
    inp = synth.SynthInputs(w["tiny_d64_ctx1024"])
    lam = inp.logits(0, 0, 0, 1024)
    assert abs((lam <= 0).mean() - 0.115) < 0.02
    lit = synth.SynthInputs(w["tiny_d64_ctx1024"], marks="literal").logits(0, 0, 0, 1024)
    assert np.array_equal(lit, -lam)
    q3 = synth.SynthInputs(w["qwen3-8b_ctx8192"])
    assert q3.mu.shape == (36, 8) and q3.mu.min() >= -2 and q3.mu.max() <= 0
    q4 = synth.SynthInputs(w["qwen3-8b_batch32_ragged"])
    ctx = q4.ctx_lens()
    assert ctx.min() >= 4096 and ctx.max() <= 32768 and len(ctx) == 32
    assert 0.08 < q4.keep_rate().mean() < 0.17


def test_prompt_and_decode_rows_are_one_stream():
    inp = synth.SynthInputs(synth.WORKLOADS["tiny_d64_ctx1024"])
    a = inp.k(0, 0, 0, 20)
    b = inp.k(0, 0, 10, 10)
    assert np.array_equal(a[10:], b)
    assert np.array_equal(inp.logits(0, 0, 0, 20)[10:], inp.logits(0, 0, 10, 10))
