"""DMS oracle -- TEST INFRASTRUCTURE ONLY.

Plain CPU statement of DMS decode / prefill attention (see dms_oracle.c for the
rule and its sources).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package; the GPU library never
does, and this package imports nothing from it.

Everything here is argument marshalling around dms_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dms_oracle.c")
_SO = os.path.join(_HERE, "libdms_oracle.so")
_lock = threading.Lock()
_handle = None


def build(force: bool = False, src: str = _SRC, so: str = _SO) -> str:
    """Compile the oracle (gcc -O2 -fopenmp) into a shared library."""
    if force or not os.path.exists(so) or os.path.getmtime(so) < os.path.getmtime(src):
        tmp = so + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, so)
    return so


def load(so: str) -> ctypes.CDLL:
    """Load an oracle library and declare its entry points."""
    lib = ctypes.CDLL(so)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.dms_oracle_marks.argtypes = [vp, i64, vp]
    lib.dms_oracle_marks.restype = None
    lib.dms_oracle_k_channel_logits.argtypes = [vp, i64, i32, i32, i32, vp]
    lib.dms_oracle_k_channel_logits.restype = None
    lib.dms_oracle_live_positions.argtypes = [i64, i64, vp, i64, vp]
    lib.dms_oracle_live_positions.restype = i64
    lib.dms_oracle_attend.argtypes = [i32, i32, i32, i64, dbl, i64, vp, vp, i64, vp, vp, vp, vp]
    lib.dms_oracle_attend.restype = ctypes.c_int
    lib.dms_oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.dms_oracle_e4m3_value.restype = dbl
    lib.dms_oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.dms_oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.dms_oracle_quantize_rows.argtypes = [vp, i64, i32, vp, vp]
    lib.dms_oracle_quantize_rows.restype = None
    lib.dms_oracle_attend_fp8.argtypes = [i32, i32, i32, i64, dbl, i64, vp, vp, i64, vp, vp, vp, vp, vp, vp]
    lib.dms_oracle_attend_fp8.restype = ctypes.c_int
    lib.dms_oracle_row_bytes.argtypes = [i32, i32]
    lib.dms_oracle_row_bytes.restype = i64
    lib.dms_oracle_kv_bytes.argtypes = [i64, i64, vp, i32, i32, i32, i64, vp]
    lib.dms_oracle_kv_bytes.restype = None
    return lib


def _lib():
    global _handle
    with _lock:
        if _handle is None:
            build()
            _handle = load(_SO)
    return _handle


class Oracle:
    """The oracle's entry points bound to one compiled library (the default one,
    or a differently compiled copy that a test wants to exercise)."""

    def __init__(self, lib: ctypes.CDLL):
        self.lib = lib

    def marks(self, logits: np.ndarray) -> np.ndarray:
        lg = np.ascontiguousarray(logits, np.float32)
        out = np.empty(lg.shape, np.uint8)
        self.lib.dms_oracle_marks(lg.ctypes.data, lg.size, out.ctypes.data)
        return out

    def k_channel_logits(self, k: np.ndarray, channel: int) -> np.ndarray:
        """k [..., Hkv, D] bf16 bits -> eviction logits float32 [..., Hkv] read
        from channel `channel` of every K row."""
        k = np.ascontiguousarray(k, np.uint16)
        hkv, d = k.shape[-2], k.shape[-1]
        if not 0 <= channel < d:
            raise ValueError("channel out of range")
        rows = k.size // (hkv * d)
        out = np.empty(k.shape[:-1], np.float32)
        self.lib.dms_oracle_k_channel_logits(k.ctypes.data, rows, hkv, d, int(channel), out.ctypes.data)
        return out

    def live_positions(self, t: int, window: int, marks_col: np.ndarray) -> np.ndarray:
        """Live set of one head at query position t; marks_col[s] is the mark of s."""
        m = np.ascontiguousarray(marks_col, np.uint8)
        if t >= m.shape[0]:
            raise ValueError("t beyond the marks given")
        out = np.empty(t + 1, np.int32)
        n = self.lib.dms_oracle_live_positions(t, window, m.ctypes.data, 1, out.ctypes.data)
        return out[:n].copy()

    def live_count(self, t: int, window: int, marks_col: np.ndarray) -> int:
        m = np.ascontiguousarray(marks_col, np.uint8)
        return int(self.lib.dms_oracle_live_positions(t, window, m.ctypes.data, 1, None))

    def attend(self, q: np.ndarray, query_pos, k: np.ndarray, v: np.ndarray,
               marks: np.ndarray, window: int, scale: float = 0.0) -> np.ndarray:
        """q [nq][Hq][D], k/v [T][Hkv][D] bf16 bits (uint16); marks [T][Hkv].
        Returns out [nq][Hq][D] float64."""
        q = np.ascontiguousarray(q, np.uint16)
        k = np.ascontiguousarray(k, np.uint16)
        v = np.ascontiguousarray(v, np.uint16)
        marks = np.ascontiguousarray(marks, np.uint8)
        qp = np.ascontiguousarray(np.asarray(query_pos, np.int64).reshape(-1))
        nq, hq, d = q.shape
        nk, hkv, d2 = k.shape
        if d2 != d or v.shape != k.shape or marks.shape != (nk, hkv) or qp.shape[0] != nq:
            raise ValueError("shape mismatch")
        if hq % hkv:
            raise ValueError("n_q_heads must be a multiple of n_kv_heads")
        out = np.empty((nq, hq, d), np.float64)
        rc = self.lib.dms_oracle_attend(hq, hkv, d, int(window), float(scale), nq, qp.ctypes.data,
                                        q.ctypes.data, nk, k.ctypes.data, v.ctypes.data,
                                        marks.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError("query position outside the keys given")
        return out


    # ---- FP8 (E4M3) K/V
    def e4m3_value(self, code: int) -> float:
        return float(self.lib.dms_oracle_e4m3_value(int(code) & 0xFF))

    def e4m3_encode(self, x: float) -> int:
        return int(self.lib.dms_oracle_e4m3_encode(float(x)))

    def quantize_rows(self, x: np.ndarray):
        """x [..., D] bf16 bits -> (codes uint8 [..., D], scales float32 [...])."""
        x = np.ascontiguousarray(x, np.uint16)
        d = x.shape[-1]
        rows = x.size // d
        codes = np.empty(x.shape, np.uint8)
        scales = np.empty(x.shape[:-1], np.float32)
        self.lib.dms_oracle_quantize_rows(x.ctypes.data, rows, d, codes.ctypes.data, scales.ctypes.data)
        return codes, scales

    def attend_fp8(self, q: np.ndarray, query_pos, k8: np.ndarray, ks: np.ndarray, v8: np.ndarray,
                   vs: np.ndarray, marks: np.ndarray, window: int, scale: float = 0.0) -> np.ndarray:
        """q [nq][Hq][D] bf16 bits; k8/v8 [T][Hkv][D] E4M3 codes; ks/vs [T][Hkv]
        scales; marks [T][Hkv].  Returns out [nq][Hq][D] float64."""
        q = np.ascontiguousarray(q, np.uint16)
        k8 = np.ascontiguousarray(k8, np.uint8)
        v8 = np.ascontiguousarray(v8, np.uint8)
        ks = np.ascontiguousarray(ks, np.float32)
        vs = np.ascontiguousarray(vs, np.float32)
        marks = np.ascontiguousarray(marks, np.uint8)
        qp = np.ascontiguousarray(np.asarray(query_pos, np.int64).reshape(-1))
        nq, hq, d = q.shape
        nk, hkv, d2 = k8.shape
        if d2 != d or v8.shape != k8.shape or ks.shape != (nk, hkv) or vs.shape != (nk, hkv) \
                or marks.shape != (nk, hkv) or qp.shape[0] != nq:
            raise ValueError("shape mismatch")
        out = np.empty((nq, hq, d), np.float64)
        rc = self.lib.dms_oracle_attend_fp8(hq, hkv, d, int(window), float(scale), nq, qp.ctypes.data,
                                            q.ctypes.data, nk, k8.ctypes.data, ks.ctypes.data, v8.ctypes.data,
                                            vs.ctypes.data, marks.ctypes.data, out.ctypes.data)
        if rc != 0:
            raise ValueError("query position outside the keys given")
        return out

    # ---- bytes a compact store holds
    def row_bytes(self, head_dim: int, fp8: bool = False) -> int:
        return int(self.lib.dms_oracle_row_bytes(int(head_dim), 1 if fp8 else 0))

    def kv_bytes(self, t: int, window: int, marks: np.ndarray, head_dim: int, fp8: bool = False,
                 page_slots: int = 64):
        """(live, allocated, dense-equivalent) bytes of one (seq, layer) after
        the token at position t; marks [>t][Hkv]."""
        m = np.ascontiguousarray(marks, np.uint8)
        if m.ndim != 2 or t >= m.shape[0]:
            raise ValueError("marks must be [positions > t][n_kv_heads]")
        out = np.zeros(3, np.int64)
        self.lib.dms_oracle_kv_bytes(int(t), int(window), m.ctypes.data, m.shape[1], int(head_dim),
                                     1 if fp8 else 0, int(page_slots), out.ctypes.data)
        return int(out[0]), int(out[1]), int(out[2])


def default() -> Oracle:
    return Oracle(_lib())


def marks(logits):
    return default().marks(logits)


def k_channel_logits(k, channel):
    return default().k_channel_logits(k, channel)


def live_positions(t, window, marks_col):
    return default().live_positions(t, window, marks_col)


def live_count(t, window, marks_col):
    return default().live_count(t, window, marks_col)


def attend(q, query_pos, k, v, marks_, window, scale=0.0):
    return default().attend(q, query_pos, k, v, marks_, window, scale)


def e4m3_value(code):
    return default().e4m3_value(code)


def e4m3_encode(x):
    return default().e4m3_encode(x)


def quantize_rows(x):
    return default().quantize_rows(x)


def attend_fp8(q, query_pos, k8, ks, v8, vs, marks_, window, scale=0.0):
    return default().attend_fp8(q, query_pos, k8, ks, v8, vs, marks_, window, scale)


def row_bytes(head_dim, fp8=False):
    return default().row_bytes(head_dim, fp8)


def kv_bytes(t, window, marks_, head_dim, fp8=False, page_slots=64):
    return default().kv_bytes(t, window, marks_, head_dim, fp8, page_slots)
