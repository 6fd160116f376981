"""Python binding of libdms.so, the DMS compact-KV decode library for MI355X.

The functions named ``dms_*`` mirror the C entry points of include/dms.h one to
one and only marshal arguments (device pointers as integers, hipStream_t as an
integer).  ``Pool`` is a convenience wrapper that takes torch tensors: torch
provides the device memory (the arena, inputs and outputs) and the stream; every
step of the computation runs in the library's HIP kernels.  There is no CPU
fallback: if libdms.so is missing, importing the binding's entry points raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdms.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "dms.h")

DMS_OK, DMS_E_INVAL, DMS_E_NOMEM, DMS_E_CAPACITY, DMS_E_STATE, DMS_E_HIP = 0, -1, -2, -3, -4, -5
DMS_PAGE_SLOTS = 64
DMS_KV_BF16, DMS_KV_FP8_E4M3 = 0, 1
DMS_LOGITS_INPUT, DMS_LOGITS_K_CHANNEL = 0, 1
_STATUS_NAMES = {0: "DMS_OK", -1: "DMS_E_INVAL", -2: "DMS_E_NOMEM", -3: "DMS_E_CAPACITY",
                 -4: "DMS_E_STATE", -5: "DMS_E_HIP"}


class DMSError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, str(status)), message))
        self.status = status


class dms_pool_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("max_seqs", ctypes.c_int32),
        ("max_positions", ctypes.c_int32),
        ("page_slots", ctypes.c_int32),
        ("max_pages", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("page_order_seed", ctypes.c_uint32),
        ("kv_format", ctypes.c_int32),
        ("logit_source", ctypes.c_int32),
        ("logit_channel", ctypes.c_int32),
        ("reserved", ctypes.c_int32 * 1),
    ]


class dms_timing(ctypes.Structure):
    _fields_ = [
        ("decode_attend_ms", ctypes.c_double),
        ("decode_merge_ms", ctypes.c_double),
        ("prefill_compact_ms", ctypes.c_double),
        ("prefill_attend_ms", ctypes.c_double),
        ("decode_launches", ctypes.c_int64),
        ("prefill_calls", ctypes.c_int64),
        ("extend_attend_ms", ctypes.c_double),
        ("extend_calls", ctypes.c_int64),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class dms_stats(ctypes.Structure):
    _fields_ = [
        ("live_slots", ctypes.c_int64),
        ("kv_bytes_live", ctypes.c_int64),
        ("kv_bytes_allocated", ctypes.c_int64),
        ("kv_bytes_dense_equiv", ctypes.c_int64),
        ("pages_used", ctypes.c_int64),
        ("pages_free", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_int64),
        ("position", ctypes.c_int32),
        ("device_error", ctypes.c_int32),
    ]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


_lock = threading.Lock()
_lib_handle = None


def header_symbols() -> list:
    """Names of the functions include/dms.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dms_\w+)\s*\(", text, re.M)))


def lib() -> ctypes.CDLL:
    """Load libdms.so (raises if it was not built)."""
    global _lib_handle
    with _lock:
        if _lib_handle is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libdms.so is not built; run __graft_entry__.build() "
                                   "(or python compact_decode_attention_amd/build.py)")
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
            P = ctypes.POINTER
            L.dms_pool_bytes.argtypes = [P(dms_pool_config)]
            L.dms_pool_bytes.restype = sz
            L.dms_pool_create.argtypes = [P(dms_pool_config), vp, sz, vp, P(vp)]
            L.dms_pool_destroy.argtypes = [vp]
            L.dms_prefill.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
            L.dms_decode_step.argtypes = [vp, i32, P(i32), i32, i32, vp, vp, vp, vp, vp, vp]
            L.dms_decode_step_static.argtypes = [vp, i32, P(i32), i32, i32, vp, vp, vp, vp, vp, vp]
            L.dms_extend.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]
            L.dms_query_stats.argtypes = [vp, i32, P(dms_stats), P(i32)]
            L.dms_export_live.argtypes = [vp, i32, i32, i32, P(i32), i32, P(i32)]
            L.dms_export_kv.argtypes = [vp, i32, i32, i32, i32, P(i32), vp, vp, P(ctypes.c_float),
                                        P(ctypes.c_float), P(i32)]
            L.dms_seq_release.argtypes = [vp, i32, vp]
            L.dms_timing_enable.argtypes = [vp, i32]
            L.dms_timing_read.argtypes = [vp, P(dms_timing)]
            for f in (L.dms_pool_create, L.dms_pool_destroy, L.dms_prefill, L.dms_decode_step,
                      L.dms_decode_step_static, L.dms_extend,
                      L.dms_query_stats, L.dms_export_live, L.dms_export_kv, L.dms_seq_release,
                      L.dms_timing_enable, L.dms_timing_read):
                f.restype = ctypes.c_int32
            L.dms_last_error.argtypes = []
            L.dms_last_error.restype = ctypes.c_char_p
            _lib_handle = L
    return _lib_handle


def dms_last_error() -> str:
    return lib().dms_last_error().decode()


def _check(status: int):
    if status != DMS_OK:
        raise DMSError(status, dms_last_error())


def make_config(n_layers, n_q_heads, n_kv_heads, head_dim, window, max_seqs, max_positions,
                max_pages, softmax_scale=0.0, page_order_seed=0, kv_format=0, logit_channel=None) -> dms_pool_config:
    """logit_channel=None: eviction logits come from the calls' logits argument;
    an int c: from channel c of each kv head's K row (logits may then be None)."""
    c = dms_pool_config()
    c.n_layers, c.n_q_heads, c.n_kv_heads, c.head_dim = n_layers, n_q_heads, n_kv_heads, head_dim
    c.window, c.max_seqs, c.max_positions = window, max_seqs, max_positions
    c.page_slots = 0
    c.max_pages = max_pages
    c.softmax_scale = softmax_scale
    c.page_order_seed = page_order_seed
    c.kv_format = kv_format
    if logit_channel is not None:
        c.logit_source, c.logit_channel = DMS_LOGITS_K_CHANNEL, logit_channel
    return c


# ---- one wrapper per C entry point -------------------------------------------

def dms_pool_bytes(cfg: dms_pool_config) -> int:
    n = lib().dms_pool_bytes(ctypes.byref(cfg))
    if n == 0:
        raise DMSError(DMS_E_INVAL, dms_last_error())
    return int(n)


def dms_pool_create(cfg: dms_pool_config, arena_ptr: int, arena_bytes: int, stream: int) -> int:
    h = ctypes.c_void_p()
    _check(lib().dms_pool_create(ctypes.byref(cfg), ctypes.c_void_p(arena_ptr), arena_bytes,
                                 ctypes.c_void_p(stream), ctypes.byref(h)))
    return h.value


def dms_pool_destroy(pool: int):
    _check(lib().dms_pool_destroy(ctypes.c_void_p(pool)))


def dms_prefill(pool: int, seq: int, layer: int, n_tokens: int, q: int, k: int, v: int,
                logits: int, out: int, stream: int):
    vp = ctypes.c_void_p
    _check(lib().dms_prefill(vp(pool), seq, layer, n_tokens, vp(q or None), vp(k), vp(v), vp(logits),
                             vp(out or None), vp(stream)))


def dms_extend(pool: int, seq: int, layer: int, n_tokens: int, q: int, k: int, v: int, logits: int, out: int,
               stream: int):
    vp = ctypes.c_void_p
    _check(lib().dms_extend(vp(pool), seq, layer, n_tokens, vp(q or None), vp(k), vp(v), vp(logits or None),
                            vp(out or None), vp(stream)))


def dms_decode_step(pool: int, seq_ids: Sequence[int], layer0: int, n_layers: int, q: int, k: int,
                    v: int, logits: int, out: int, stream: int):
    ids = (ctypes.c_int32 * len(seq_ids))(*[int(s) for s in seq_ids])
    vp = ctypes.c_void_p
    _check(lib().dms_decode_step(vp(pool), len(seq_ids), ids, layer0, n_layers, vp(q), vp(k), vp(v),
                                 vp(logits), vp(out), vp(stream)))


def dms_decode_step_static(pool: int, seq_ids: Sequence[int], layer0: int, n_layers: int, q: int, k: int,
                           v: int, logits: int, out: int, stream: int):
    ids = (ctypes.c_int32 * len(seq_ids))(*[int(s) for s in seq_ids])
    vp = ctypes.c_void_p
    _check(lib().dms_decode_step_static(vp(pool), len(seq_ids), ids, layer0, n_layers, vp(q), vp(k), vp(v),
                                        vp(logits), vp(out), vp(stream)))


def dms_query_stats(pool: int, seq: int, n_layers: int = 0, n_kv_heads: int = 0, raise_on_error=True):
    """Returns (dms_stats, live counts [n_layers][n_kv_heads] or None, status).
    With raise_on_error false, a sticky device status (DMS_E_CAPACITY or
    DMS_E_STATE) is returned instead of raised; the stats are filled in."""
    st = dms_stats()
    live = None
    ptr = None
    if n_layers and n_kv_heads:
        live = np.zeros((n_layers, n_kv_heads), np.int32)
        ptr = live.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    rc = lib().dms_query_stats(ctypes.c_void_p(pool), seq, ctypes.byref(st), ptr)
    if rc != DMS_OK and (raise_on_error or rc not in (DMS_E_CAPACITY, DMS_E_STATE)):
        _check(rc)
    return st, live, rc


def dms_export_live(pool: int, seq: int, layer: int, kv_head: int, cap: int) -> np.ndarray:
    buf = np.zeros(max(cap, 1), np.int32)
    n = ctypes.c_int32()
    _check(lib().dms_export_live(ctypes.c_void_p(pool), seq, layer, kv_head,
                                 buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), cap, ctypes.byref(n)))
    return buf[:n.value].copy()


def dms_export_kv(pool: int, seq: int, layer: int, kv_head: int, cap: int, head_dim: int, fp8: bool):
    """(positions int32 [n], k, v [n][head_dim] (uint16 bf16 bits, or uint8 E4M3 codes),
    k_scale, v_scale float32 [n]) of what one (seq, layer, kv head) stores."""
    dt = np.uint8 if fp8 else np.uint16
    cap1 = max(cap, 1)
    pos = np.zeros(cap1, np.int32)
    k = np.zeros((cap1, head_dim), dt)
    v = np.zeros((cap1, head_dim), dt)
    ks = np.zeros(cap1, np.float32)
    vs = np.zeros(cap1, np.float32)
    n = ctypes.c_int32()
    fp = ctypes.POINTER(ctypes.c_float)
    _check(lib().dms_export_kv(ctypes.c_void_p(pool), seq, layer, kv_head, cap,
                               pos.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.c_void_p(k.ctypes.data),
                               ctypes.c_void_p(v.ctypes.data), ks.ctypes.data_as(fp), vs.ctypes.data_as(fp),
                               ctypes.byref(n)))
    m = n.value
    return pos[:m].copy(), k[:m].copy(), v[:m].copy(), ks[:m].copy(), vs[:m].copy()


def dms_seq_release(pool: int, seq: int, stream: int):
    _check(lib().dms_seq_release(ctypes.c_void_p(pool), seq, ctypes.c_void_p(stream)))


def dms_timing_enable(pool: int, enable: bool):
    _check(lib().dms_timing_enable(ctypes.c_void_p(pool), 1 if enable else 0))


def dms_timing_read(pool: int) -> dms_timing:
    """Kernel times (ms) and call counts recorded since the last read."""
    t = dms_timing()
    _check(lib().dms_timing_read(ctypes.c_void_p(pool), ctypes.byref(t)))
    return t


# ---- torch convenience wrapper ------------------------------------------------

class Pool:
    """A pool whose arena is a torch uint8 tensor on a HIP device.

    Tensors passed in must be contiguous, on the pool's device, bf16 for
    q/k/v/out and float32 for logits, with the shapes include/dms.h states.
    """

    def __init__(self, n_layers, n_q_heads, n_kv_heads, head_dim, window, max_seqs, max_positions,
                 max_pages, softmax_scale=0.0, page_order_seed=0, kv_format=0, logit_channel=None,
                 device="cuda"):
        import torch
        self.torch = torch
        self.cfg = make_config(n_layers, n_q_heads, n_kv_heads, head_dim, window, max_seqs,
                               max_positions, max_pages, softmax_scale, page_order_seed, kv_format,
                               logit_channel)
        self.logits_from_k = logit_channel is not None
        self.fp8 = kv_format == DMS_KV_FP8_E4M3
        self.device = torch.device(device)
        self.nbytes = dms_pool_bytes(self.cfg)
        self.arena = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=self.device)
        base = self.arena.data_ptr()
        self._arena_ptr = (base + 255) // 256 * 256
        self.handle = dms_pool_create(self.cfg, self._arena_ptr, self.nbytes, self._stream())
        self.n_layers, self.n_q_heads, self.n_kv_heads, self.head_dim = n_layers, n_q_heads, n_kv_heads, head_dim
        self.window, self.max_seqs, self.max_positions = window, max_seqs, max_positions

    def _stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def _check_tensor(self, t, shape, dtype, name):
        torch = self.torch
        if t is None:
            raise ValueError(name + " is None")
        if t.device != self.device and not (t.device.type == self.device.type and
                                            (t.device.index or 0) == (self.device.index or 0)):
            raise ValueError("%s must be on %s" % (name, self.device))
        if t.dtype != dtype:
            raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
        if not t.is_contiguous():
            raise ValueError(name + " must be contiguous")
        return t.data_ptr()

    def prefill(self, seq, layer, k, v, logits, q=None, out=None):
        torch = self.torch
        T = k.shape[0]
        H, Hq, D = self.n_kv_heads, self.n_q_heads, self.head_dim
        kp = self._check_tensor(k, (T, H, D), torch.bfloat16, "k")
        vpp = self._check_tensor(v, (T, H, D), torch.bfloat16, "v")
        lp = 0 if (logits is None and self.logits_from_k) else self._check_tensor(logits, (T, H), torch.float32,
                                                                                   "logits")
        qp = self._check_tensor(q, (T, Hq, D), torch.bfloat16, "q") if q is not None else 0
        op = self._check_tensor(out, (T, Hq, D), torch.bfloat16, "out") if out is not None else 0
        dms_prefill(self.handle, seq, layer, T, qp, kp, vpp, lp, op, self._stream())

    def extend(self, seq, layer, k, v, logits, q=None, out=None):
        """Append k.shape[0] new tokens to (seq, layer); out (if given) gets their
        attention outputs."""
        torch = self.torch
        T = k.shape[0]
        H, Hq, D = self.n_kv_heads, self.n_q_heads, self.head_dim
        kp = self._check_tensor(k, (T, H, D), torch.bfloat16, "k")
        vpp = self._check_tensor(v, (T, H, D), torch.bfloat16, "v")
        lp = 0 if (logits is None and self.logits_from_k) else self._check_tensor(logits, (T, H), torch.float32,
                                                                                   "logits")
        qp = self._check_tensor(q, (T, Hq, D), torch.bfloat16, "q") if q is not None else 0
        op = self._check_tensor(out, (T, Hq, D), torch.bfloat16, "out") if out is not None else 0
        dms_extend(self.handle, seq, layer, T, qp, kp, vpp, lp, op, self._stream())

    def decode_step(self, seq_ids, layer0, q, k, v, logits, out, static_scratch=False):
        """static_scratch: through dms_decode_step_static (split-K scratch in the
        library's per-GPU device array; the call allocates nothing)."""
        torch = self.torch
        n = len(seq_ids)
        L = q.shape[0]
        H, Hq, D = self.n_kv_heads, self.n_q_heads, self.head_dim
        qp = self._check_tensor(q, (L, n, Hq, D), torch.bfloat16, "q")
        kp = self._check_tensor(k, (L, n, H, D), torch.bfloat16, "k")
        vpp = self._check_tensor(v, (L, n, H, D), torch.bfloat16, "v")
        lp = 0 if (logits is None and self.logits_from_k) else self._check_tensor(logits, (L, n, H), torch.float32,
                                                                                   "logits")
        op = self._check_tensor(out, (L, n, Hq, D), torch.bfloat16, "out")
        fn = dms_decode_step_static if static_scratch else dms_decode_step
        fn(self.handle, list(seq_ids), layer0, L, qp, kp, vpp, lp, op, self._stream())

    def stats(self, seq=-1, per_head=False, raise_on_error=True):
        if per_head and seq >= 0:
            st, live, rc = dms_query_stats(self.handle, seq, self.n_layers, self.n_kv_heads, raise_on_error)
        else:
            st, live, rc = dms_query_stats(self.handle, seq, raise_on_error=raise_on_error)
        return st, live

    def export_live(self, seq, layer, kv_head):
        return dms_export_live(self.handle, seq, layer, kv_head, self.max_positions)

    def export_kv(self, seq, layer, kv_head):
        return dms_export_kv(self.handle, seq, layer, kv_head, self.max_positions, self.head_dim, self.fp8)

    def release(self, seq):
        dms_seq_release(self.handle, seq, self._stream())

    def close(self):
        if getattr(self, "handle", None):
            dms_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
