"""Python side of the fp64 attention oracle (ctypes over attn_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only tests/, __graft_entry__.smoke()
and the cpu_baseline leg of bench.py may import this module.  It never imports
the GPU package, and the GPU package never imports it.

The arithmetic lives in attn_oracle.c (plain softmax attention in binary64,
from the exact fp16 input bits); this module only builds that file with gcc,
marshals numpy arrays and loops over batch entries.  It takes fp16 numpy
arrays (or anything numpy can view as float16) in the [B, S, H, D] layout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "libattn_oracle.so")

# -ffp-contract=off: no fused multiply-add, so every sum is the written one.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread", "-std=c11"]

_lock = threading.Lock()
_libs: dict[str, ctypes.CDLL] = {}


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle C source into a shared library (always recompiles)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f64p = ctypes.POINTER(ctypes.c_double)
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_attn_rows.argtypes = [u16p, u16p, u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_float, i32p, i32p, ctypes.c_int64, f64p, f64p,
                                     ctypes.c_int]
    lib.oracle_attn_rows_ex.restype = ctypes.c_int
    lib.oracle_attn_rows_ex.argtypes = [u16p, u16p, u16p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_float, i32p, i32p, ctypes.c_int64, f64p,
                                        f64p, ctypes.c_int]
    lib.oracle_half_to_double.restype = ctypes.c_double
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    return lib


def load(path: str = LIB) -> ctypes.CDLL:
    """Load the built oracle library; builds it only if it is not there yet."""
    with _lock:
        if path not in _libs:
            if not os.path.exists(path):
                if path != LIB:
                    raise FileNotFoundError(path)
                build()
            _libs[path] = _bind(ctypes.CDLL(path))
        return _libs[path]


MAX_THREADS = 16  # a one-GPU job's share of host cores


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(MAX_THREADS, n))


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    if a.dtype == np.uint16:
        return a
    raise TypeError("oracle inputs must be float16 (or their uint16 bit patterns), got %s" % a.dtype)


def _p(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Oracle:
    """fp64 attention oracle bound to one built library (the default one, or a test build)."""

    def __init__(self, path: str = LIB):
        self.lib = load(path)

    def half_to_double(self, bits: int) -> float:
        return self.lib.oracle_half_to_double(int(bits))

    def rows(self, q, k, v, heads, rows, causal: bool, scale: float, nthreads: int | None = None):
        """O rows and LSE for one batch entry.

        q: [Sq, Hq, D] fp16; k, v: [Sk, Hkv, D] fp16 (Sk may differ from Sq; causal then aligns the last
        query row with the last key, and needs Sq <= Sk); heads, rows: int sequences of equal length n.
        Returns (o [n, D] float64, lse [n] float64).
        """
        qb, kb, vb = _u16(q), _u16(k), _u16(v)
        if qb.ndim != 3 or kb.ndim != 3 or vb.ndim != 3:
            raise ValueError("expected [S, H, D] arrays for one batch entry")
        S, Hq, D = qb.shape
        Sk, Hkv, Dk = kb.shape
        if kb.shape != vb.shape or Dk != D:
            raise ValueError("shape mismatch q %s k %s v %s" % (qb.shape, kb.shape, vb.shape))
        hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int32).reshape(-1))
        rs = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1))
        if hs.shape != rs.shape:
            raise ValueError("heads and rows differ in length")
        n = hs.shape[0]
        o = np.empty((n, D), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
        rc = self.lib.oracle_attn_rows_ex(_p(qb, ctypes.c_uint16), _p(kb, ctypes.c_uint16),
                                          _p(vb, ctypes.c_uint16), S, Sk, Hq, Hkv, D, int(bool(causal)),
                                          float(scale), _p(hs, ctypes.c_int32), _p(rs, ctypes.c_int32), n,
                                          _p(o, ctypes.c_double), _p(lse, ctypes.c_double),
                                          int(nthreads or default_threads()))
        if rc != 0:
            raise RuntimeError("oracle_attn_rows failed with code %d" % rc)
        return o, lse

    def full(self, q, k, v, causal: bool, scale: float, nthreads: int | None = None):
        """Whole-tensor oracle: q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] fp16 -> (O [B,Sq,Hq,D], LSE [B,Hq,Sq]) float64."""
        qn, kn, vn = _u16(q), _u16(k), _u16(v)
        B, S, Hq, D = qn.shape
        O = np.empty((B, S, Hq, D), dtype=np.float64)
        L = np.empty((B, Hq, S), dtype=np.float64)
        hh, ii = np.meshgrid(np.arange(Hq, dtype=np.int32), np.arange(S, dtype=np.int32), indexing="ij")
        for b in range(B):
            o, lse = self.rows(qn[b], kn[b], vn[b], hh.reshape(-1), ii.reshape(-1), causal, scale, nthreads)
            O[b] = o.reshape(Hq, S, D).transpose(1, 0, 2)
            L[b] = lse.reshape(Hq, S)
        return O, L


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def attn_full(q, k, v, causal: bool, scale: float, nthreads: int | None = None):
    return default().full(q, k, v, causal, scale, nthreads)


def attn_rows(q, k, v, heads, rows, causal: bool, scale: float, nthreads: int | None = None):
    return default().rows(q, k, v, heads, rows, causal, scale, nthreads)
