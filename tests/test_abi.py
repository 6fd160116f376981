"""The C ABI without a GPU: libdms.so loads, exports every function that
include/dms.h declares (and no other dms_* function), the Python binding has one
wrapper per entry point, and the host-side checks of the configuration and of
the arguments return their documented status codes before any HIP call.

Nothing here launches a kernel or allocates device memory."""
import ctypes
import os
import re
import subprocess

import pytest

import compact_decode_attention_amd as dms

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def qwen_cfg(**kw):
    base = dict(n_layers=36, n_q_heads=32, n_kv_heads=8, head_dim=128, window=512, max_seqs=1,
                max_positions=8320, max_pages=36 * 8 * 131)
    base.update(kw)
    return dms.make_config(**base)


def test_header_declares_the_boundary():
    names = dms.header_symbols()
    for n in ["dms_pool_bytes", "dms_pool_create", "dms_pool_destroy", "dms_prefill", "dms_decode_step",
              "dms_query_stats", "dms_export_live", "dms_export_kv", "dms_seq_release", "dms_timing_enable",
              "dms_timing_read", "dms_last_error"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = dms.lib()
    for n in dms.header_symbols():
        assert hasattr(L, n), "libdms.so does not export %s" % n


def test_library_exports_no_undeclared_dms_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", dms.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {m.group(1) for m in re.finditer(r"\sT\s+(dms_\w+)$", out, re.M)}
    assert exported == set(dms.header_symbols())


def test_binding_has_one_wrapper_per_entry_point():
    for n in dms.header_symbols():
        assert callable(getattr(dms, n, None)), "binding lacks %s" % n


def test_pool_bytes_of_the_qwen_pool():
    cfg = qwen_cfg()
    n = dms.dms_pool_bytes(cfg)
    pages = 36 * 8 * 131
    kv = 2 * pages * 64 * 128 * 2
    assert n % 256 == 0
    assert kv < n < kv * 1.2


@pytest.mark.parametrize("field,value,msg", [
    ("head_dim", 96, "head_dim"),
    ("n_q_heads", 12, "multiple"),
    ("n_q_heads", 8 * 16, "1, 2, 4 or 8"),
    ("window", 0, "window"),
    ("max_seqs", 0, "max_seqs"),
    ("max_positions", 0, "max_positions"),
    ("max_pages", 0, "max_pages"),
    ("n_layers", 0, "n_layers"),
    ("n_kv_heads", 0, "n_kv_heads"),
])
def test_pool_bytes_rejects_bad_configs(field, value, msg):
    with pytest.raises(dms.DMSError) as e:
        dms.dms_pool_bytes(qwen_cfg(**{field: value}))
    assert e.value.status == dms.DMS_E_INVAL
    assert msg in str(e.value)


def test_pool_bytes_rejects_page_slots_and_reserved():
    cfg = qwen_cfg()
    cfg.page_slots = 32
    with pytest.raises(dms.DMSError):
        dms.dms_pool_bytes(cfg)
    cfg = qwen_cfg()
    cfg.reserved[0] = 1
    with pytest.raises(dms.DMSError):
        dms.dms_pool_bytes(cfg)
    cfg = qwen_cfg()
    cfg.softmax_scale = float("nan")
    with pytest.raises(dms.DMSError):
        dms.dms_pool_bytes(cfg)


@pytest.mark.parametrize("source,channel,ok", [
    (0, 0, True), (0, 3, False), (1, 0, True), (1, 127, True), (1, 128, False), (1, -1, False), (2, 0, False)])
def test_logit_source_and_channel_are_checked(source, channel, ok):
    cfg = qwen_cfg()
    cfg.logit_source, cfg.logit_channel = source, channel
    if ok:
        assert dms.dms_pool_bytes(cfg) > 0
    else:
        with pytest.raises(dms.DMSError) as e:
            dms.dms_pool_bytes(cfg)
        assert "logit" in str(e.value)


def test_kv_format_is_checked():
    for bad in (-1, 2, 7):
        with pytest.raises(dms.DMSError) as e:
            dms.dms_pool_bytes(qwen_cfg(kv_format=bad))
        assert "kv_format" in str(e.value)


def test_fp8_pool_holds_codes_and_scales():
    """An FP8 pool's pages take head_dim + 4 bytes per row (codes and an fp32
    scale) instead of 2 * head_dim, plus the prompt scratch for its codes.  The
    page arrays hold the shared pool and ceil(max_positions / 64) scratch pages
    per kv head.  A bf16 pool also holds the prompt's V as fp16 values, 2 bytes
    per (position, kv head, dim), for its prefill attention."""
    pages = 36 * 8 * 131 + 8 * 130
    b16 = dms.dms_pool_bytes(qwen_cfg())
    f8 = dms.dms_pool_bytes(qwen_cfg(kv_format=dms.DMS_KV_FP8_E4M3))
    saved = 2 * pages * 64 * (2 * 128 - (128 + 4))
    scratch = 2 * 8320 * 8 * (128 + 4)
    vt16 = 8320 * 8 * 128 * 2
    assert b16 - f8 == saved - scratch + vt16


def test_window_beyond_positions_needs_no_ring():
    """Eviction disabled (window >= every position) keeps no window ring."""
    a = dms.dms_pool_bytes(qwen_cfg(window=1 << 20))
    b = dms.dms_pool_bytes(qwen_cfg(window=512))
    assert b - a >= 36 * 8 * 512 * 4 - 256


def test_create_checks_arguments_before_touching_the_device():
    L = dms.lib()
    cfg = qwen_cfg()
    n = dms.dms_pool_bytes(cfg)
    h = ctypes.c_void_p()
    assert L.dms_pool_create(ctypes.byref(cfg), None, n, None, ctypes.byref(h)) == dms.DMS_E_INVAL
    assert "NULL" in dms.dms_last_error()
    assert L.dms_pool_create(ctypes.byref(cfg), ctypes.c_void_p(0x1008), n, None,
                             ctypes.byref(h)) == dms.DMS_E_INVAL
    assert "aligned" in dms.dms_last_error()
    assert L.dms_pool_create(ctypes.byref(cfg), ctypes.c_void_p(0x1000), n - 256, None,
                             ctypes.byref(h)) == dms.DMS_E_NOMEM
    assert L.dms_pool_create(ctypes.byref(cfg), ctypes.c_void_p(0x1000), n, None, None) == dms.DMS_E_INVAL


def test_calls_on_a_null_pool_fail_cleanly():
    L = dms.lib()
    st = dms.dms_stats()
    n = ctypes.c_int32()
    assert L.dms_pool_destroy(None) == dms.DMS_E_INVAL
    assert L.dms_prefill(None, 0, 0, 1, None, None, None, None, None, None) == dms.DMS_E_INVAL
    ids = (ctypes.c_int32 * 1)(0)
    assert L.dms_decode_step(None, 1, ids, 0, 1, None, None, None, None, None, None) == dms.DMS_E_INVAL
    assert L.dms_query_stats(None, 0, ctypes.byref(st), None) == dms.DMS_E_INVAL
    assert L.dms_export_live(None, 0, 0, 0, None, 0, ctypes.byref(n)) == dms.DMS_E_INVAL
    assert L.dms_export_kv(None, 0, 0, 0, 0, None, None, None, None, None, ctypes.byref(n)) == dms.DMS_E_INVAL
    assert L.dms_seq_release(None, 0, None) == dms.DMS_E_INVAL
    assert L.dms_timing_enable(None, 1) == dms.DMS_E_INVAL
    assert L.dms_timing_read(None, None) == dms.DMS_E_INVAL


def test_product_path_does_not_reach_the_oracle():
    """The package and its sources never name the oracle or the input generator."""
    pkg = os.path.join(ROOT, "compact_decode_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b|dms_oracle|\bsynth\b", text), f
