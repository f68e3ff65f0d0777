"""ctypes front end of the C oracle.  TEST INFRASTRUCTURE ONLY.

Wraps ``oracle_cpu.c`` (plain fp64 loops, OpenMP over rows); see that file
for the definition it follows.  Inputs are bf16 bit arrays (uint16).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """Load ``liboracle.so``, building it once if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        p, i, i64, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_attn_rows.argtypes = [p, p, p, i, i, i, i, i, i, d, i, p, i64, p, p, i]
        L.oracle_attn_rows.restype = i
        L.oracle_attn_varlen_rows.argtypes = [p, p, p, p, p, i, i, i, i, d, i, p, i64, p, p, i]
        L.oracle_attn_varlen_rows.restype = i
        L.oracle_num_threads.argtypes = [i]
        L.oracle_num_threads.restype = i
        _lib = L
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def attn_rows(q, k, v, scale, causal, rows, nthreads=0):
    """Rows ``(b, h, i)`` of attention over q ``[B,Sq,Hq,d]``, k/v ``[B,Skv,Hkv,d]``.

    Returns o ``[n,d]`` and lse ``[n]`` in float64.
    """
    q, k, v = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v))
    B, Sq, Hq, d = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    o = np.zeros((n, d))
    lse = np.zeros(n)
    rc = lib().oracle_attn_rows(_ptr(q), _ptr(k), _ptr(v), B, Hq, Hkv, Sq, Skv, d,
                                float(scale), int(bool(causal)), _ptr(rows), n, _ptr(o),
                                _ptr(lse), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    return o, lse


def all_rows(B, Hq, Sq):
    """Every ``(b, h, i)`` triple, in (b, h, i) order."""
    b, h, i = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Sq), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int64)


def attn_full(q, k, v, scale, causal, nthreads=0):
    """Whole output: o ``[B,Sq,Hq,d]``, lse ``[B,Hq,Sq]``."""
    B, Sq, Hq, d = q.shape
    o, lse = attn_rows(q, k, v, scale, causal, all_rows(B, Hq, Sq), nthreads)
    return o.reshape(B, Hq, Sq, d).transpose(0, 2, 1, 3), lse.reshape(B, Hq, Sq)


def varlen_rows(q, k, v, cu_q, cu_k, scale, causal, rows, nthreads=0):
    """Rows ``(s, h, i_local)`` of packed ragged attention, q ``[Tq,Hq,d]``."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v))
    cu_q = np.ascontiguousarray(cu_q, dtype=np.int32)
    cu_k = np.ascontiguousarray(cu_k, dtype=np.int32)
    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    n = rows.shape[0]
    o = np.zeros((n, d))
    lse = np.zeros(n)
    rc = lib().oracle_attn_varlen_rows(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_q), _ptr(cu_k),
                                       len(cu_q) - 1, Hq, Hkv, d, float(scale),
                                       int(bool(causal)), _ptr(rows), n, _ptr(o), _ptr(lse),
                                       int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_varlen_rows rejected its arguments")
    return o, lse


def decode_full(q, k, v, scale, nthreads=0):
    """Decode: q ``[B,Hq,d]`` against cache ``[B,Skv,Hkv,d]`` -> o ``[B,Hq,d]``, lse ``[B,Hq]``."""
    B, Hq, d = q.shape
    o, lse = attn_full(q[:, None], k, v, scale, False, nthreads)
    return o[:, 0], lse[:, :, 0]


def num_threads(nthreads=0):
    return lib().oracle_num_threads(int(nthreads))
