"""CPU fp64 reference for exact attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU library never imports it, and nothing here imports the
GPU library: the two share no code.

Python side: argument marshalling to liboracle.so (built from oracle.c by
oracle/build.py). All arithmetic happens in oracle.c in fp64.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

MASK_BLOCK = 128


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ctype=ctypes.c_double):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _mask(blockmask, N, blk):
    if blockmask is None:
        return None
    m = np.ascontiguousarray(blockmask, dtype=np.uint8)
    nb = (N + blk - 1) // blk
    if m.shape != (nb, nb):
        raise ValueError(f"block mask must be [{nb},{nb}], got {m.shape}")
    return m


def _shape(q, k, v):
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("Q, K, V must share one [B,H,N,d] shape")
    return q.shape


class Oracle:
    """ctypes view of one build of oracle.c (the default one, or a test build)."""

    def __init__(self, path=LIB_PATH):
        if not os.path.exists(path):
            if path != LIB_PATH:
                raise FileNotFoundError(path)
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        up = ctypes.POINTER(ctypes.c_ubyte)
        L = ctypes.c_long
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                         L, L, L, L, ctypes.c_double, ctypes.c_int, up, L]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_attention_rows.argtypes = [dp, dp, dp, L, L, L, L, ctypes.c_double,
                                              ctypes.c_int, up, L, lp, lp, L, dp, dp]
        u32p = ctypes.POINTER(ctypes.c_uint)
        lib.oracle_philox4x32_10.restype = None
        lib.oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
        lib.oracle_dropout_keep.restype = ctypes.c_int
        lib.oracle_dropout_keep.argtypes = [L, L, L, ctypes.c_double, ctypes.c_ulonglong]
        lib.oracle_attention_dropout.restype = ctypes.c_int
        lib.oracle_attention_dropout.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                                 L, L, L, L, ctypes.c_double, ctypes.c_int, up,
                                                 L, ctypes.c_double, ctypes.c_ulonglong, L]
        lib.oracle_attention_kv.restype = ctypes.c_int
        lib.oracle_attention_kv.argtypes = [dp, dp, dp, dp, dp, L, L, L, L, L,
                                            ctypes.c_double, ctypes.c_int]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        self.lib = lib
        self.path = path

    def attention(self, q, k, v, scale, causal=False, blockmask=None, blk=MASK_BLOCK,
                  do=None):
        """Exact attention in fp64. Returns (O, LSE) or, when dO is given,
        (O, LSE, dQ, dK, dV). Inputs are real arrays of shape [B,H,N,d]."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, N, d = _shape(q, k, v)
        m = _mask(blockmask, N, blk)
        O = np.empty_like(q)
        LSE = np.empty((B, H, N), dtype=np.float64)
        if do is not None:
            do = _f64(do)
            if do.shape != q.shape:
                raise ValueError("dO must have Q's shape")
            dQ, dK, dV = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        else:
            dQ = dK = dV = None
        rc = self.lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(O),
                                       _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV),
                                       B, H, N, d, float(scale), int(bool(causal)),
                                       _ptr(m, ctypes.c_ubyte), blk)
        if rc != 0:
            raise RuntimeError(f"oracle_attention failed with code {rc}")
        if do is None:
            return O, LSE
        return O, LSE, dQ, dK, dV

    def attention_rows(self, q, k, v, scale, row_bh, row_i, causal=False,
                       blockmask=None, blk=MASK_BLOCK):
        """Forward for selected query rows. row_bh[r] is the head index b*H+h
        and row_i[r] the query index. Returns (O_rows [R,d], LSE_rows [R])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, N, d = _shape(q, k, v)
        m = _mask(blockmask, N, blk)
        rb = np.ascontiguousarray(row_bh, dtype=np.int64)
        ri = np.ascontiguousarray(row_i, dtype=np.int64)
        if rb.shape != ri.shape or rb.ndim != 1:
            raise ValueError("row_bh and row_i must be 1-D and equal length")
        R = rb.shape[0]
        O = np.empty((R, d), dtype=np.float64)
        LSE = np.empty((R,), dtype=np.float64)
        rc = self.lib.oracle_attention_rows(_ptr(q), _ptr(k), _ptr(v), B, H, N, d,
                                            float(scale), int(bool(causal)),
                                            _ptr(m, ctypes.c_ubyte), blk,
                                            _ptr(rb, ctypes.c_long), _ptr(ri, ctypes.c_long),
                                            R, _ptr(O), _ptr(LSE))
        if rc != 0:
            raise RuntimeError(f"oracle_attention_rows failed with code {rc}")
        return O, LSE

    def philox4x32_10(self, ctr, key):
        """Philox4x32-10 of a 4-word counter and 2-word key -> 4 words."""
        c = (ctypes.c_uint * 4)(*[int(x) & 0xFFFFFFFF for x in ctr])
        kk = (ctypes.c_uint * 2)(*[int(x) & 0xFFFFFFFF for x in key])
        o = (ctypes.c_uint * 4)()
        self.lib.oracle_philox4x32_10(c, kk, o)
        return [int(x) for x in o]

    def dropout_keep(self, bh, i, j, p_drop, seed):
        """1 if element (i, j) of head bh is kept under dropout p_drop, seed."""
        return int(self.lib.oracle_dropout_keep(bh, i, j, float(p_drop), int(seed)))

    def attention_dropout(self, q, k, v, scale, p_drop, seed, causal=False, blockmask=None,
                          blk=MASK_BLOCK, do=None, bh_offset=0):
        """attention() with dropout on P: returns (O, LSE) or (O, LSE, dQ, dK, dV).
        Head bh of the arrays draws its mask as head bh + bh_offset."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, N, d = _shape(q, k, v)
        m = _mask(blockmask, N, blk)
        O = np.empty_like(q)
        LSE = np.empty((B, H, N), dtype=np.float64)
        if do is not None:
            do = _f64(do)
            dQ, dK, dV = np.empty_like(q), np.empty_like(q), np.empty_like(q)
        else:
            dQ = dK = dV = None
        rc = self.lib.oracle_attention_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(O),
                                               _ptr(LSE), _ptr(dQ), _ptr(dK), _ptr(dV),
                                               B, H, N, d, float(scale), int(bool(causal)),
                                               _ptr(m, ctypes.c_ubyte), blk, float(p_drop),
                                               int(seed), int(bh_offset))
        if rc != 0:
            raise RuntimeError(f"oracle_attention_dropout failed with code {rc}")
        if do is None:
            return O, LSE
        return O, LSE, dQ, dK, dV

    def attention_kv(self, q, k, v, scale, causal=False):
        """Forward of Nq queries against Nk keys per head (decode shape):
        q [B,H,Nq,d], k and v [B,H,Nk,d]. causal: query i is at position
        Nk - Nq + i and sees keys up to it. Returns (O [B,H,Nq,d], LSE [B,H,Nq])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        if q.ndim != 4 or k.shape != v.shape or k.ndim != 4 or q.shape[:2] != k.shape[:2] \
                or q.shape[3] != k.shape[3]:
            raise ValueError("q [B,H,Nq,d] and k, v [B,H,Nk,d] expected")
        B, H, Nq, d = q.shape
        Nk = k.shape[2]
        O = np.empty_like(q)
        LSE = np.empty((B, H, Nq), dtype=np.float64)
        rc = self.lib.oracle_attention_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(O), _ptr(LSE),
                                          B, H, Nq, Nk, d, float(scale), int(bool(causal)))
        if rc != 0:
            raise RuntimeError(f"oracle_attention_kv failed with code {rc}")
        return O, LSE

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def attention(*args, **kwargs):
    return default().attention(*args, **kwargs)


def attention_rows(*args, **kwargs):
    return default().attention_rows(*args, **kwargs)


def attention_kv(*args, **kwargs):
    return default().attention_kv(*args, **kwargs)


def attention_dropout(*args, **kwargs):
    return default().attention_dropout(*args, **kwargs)


def dropout_keep(*args, **kwargs):
    return default().dropout_keep(*args, **kwargs)


def philox4x32_10(*args, **kwargs):
    return default().philox4x32_10(*args, **kwargs)


def num_threads() -> int:
    return default().num_threads()
