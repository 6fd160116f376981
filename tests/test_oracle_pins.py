"""CPU tests: the oracle against facts that do not come from it (oracle_pins.py),
and the same checks run against copies of the oracle with one plausible mistake
planted, each of which some check must reject."""
import os

import pytest

import oracle
import oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(oracle.__file__), "dms_oracle.c")


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


# (name, text in dms_oracle.c, replacement): each is a mistake someone could make
MUTANTS = [
    ("window_off_by_one", "return t < s + window;", "return t <= s + window;"),
    ("window_too_short", "return t < s + window;", "return t < s + window - 1;"),
    ("zero_logit_marked", "logits[i] > 0.0f ? 1 : 0", "logits[i] >= 0.0f ? 1 : 0"),
    ("mark_sign_flipped", "logits[i] > 0.0f ? 1 : 0", "logits[i] < 0.0f ? 1 : 0"),
    ("self_not_visible", "if (s > t) return 0;", "if (s >= t) return 0;"),
    ("live_scan_stops_early", "for (int64_t s = 0; s <= t; ++s) {\n        if (visible", "for (int64_t s = 0; s < t; ++s) {\n        if (visible"),
    ("gqa_interleaved", "const int32_t h = hq / group;", "const int32_t h = hq % n_kv_heads;"),
    ("scale_dropped", "z[s] = scale * dot;", "z[s] = dot;"),
    ("keys_as_values", "const uint16_t* vrow = v +", "const uint16_t* vrow = k +"),
    ("no_normalisation", "o[d] /= denom;", "o[d] /= 1.0;"),
    ("kv_bytes_k_rows_only", "out[0] += n * 2 * row;", "out[0] += n * row;"),
    ("pages_rounded_down", "(n + page_slots - 1) / page_slots * page_slots", "n / page_slots * page_slots"),
    ("fp8_rows_without_scale", "(int64_t)head_dim * 1 + 4", "(int64_t)head_dim * 1"),
    ("dense_without_current_token", "out[2] = (t + 1) *", "out[2] = t *"),
    ("marks_of_wrong_head", "marks[s * n_kv_heads + h], window)) continue;\n                    const uint16_t* krow",
     "marks[s * n_kv_heads + (h + 1) % n_kv_heads], window)) continue;\n                    const uint16_t* krow"),
]


def _quick_pins():
    out = []
    for p in pins.ALL_PINS:
        if p is pins.pin_live_sets_brute_force:
            out.append(lambda o: pins.pin_live_sets_brute_force(o, max_T=6))
        else:
            out.append(p)
    return out


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, "mutation target not found: " + name
    mutated = src.replace(old, new)
    c_path = tmp_path / ("oracle_%s.c" % name)
    so_path = tmp_path / ("liboracle_%s.so" % name)
    c_path.write_text(mutated)
    oracle.build(force=True, src=str(c_path), so=str(so_path))
    bad = oracle.Oracle(oracle.load(str(so_path)))
    caught = []
    for p in _quick_pins():
        try:
            p(bad)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(p)
    assert caught, "no check rejects the planted mistake " + name
