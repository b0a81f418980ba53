"""ctypes front end of the C oracle (oracle/kla_ref.c).

TEST INFRASTRUCTURE, like the rest of ``oracle/``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .build import LIB, build

_lib = None
_f = ctypes.POINTER(ctypes.c_float)
_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        lib = ctypes.CDLL(LIB)
        lib.kla_ref_forward.argtypes = [_f, _f, _f, _f, _f, ctypes.c_double, _f, _i64, ctypes.c_int,
                                        _d, _d] + [ctypes.c_int] * 7
        lib.kla_ref_forward.restype = ctypes.c_int
        lib.kla_ref_decode_step.argtypes = [_f, _f, _f, _f, _f, ctypes.c_double, _d, _i64,
                                            ctypes.c_int, _d] + [ctypes.c_int] * 6
        lib.kla_ref_decode_step.restype = ctypes.c_int
        lib.kla_ref_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _fp(a):
    return a.ctypes.data_as(_f) if a is not None else None


def _c32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def max_threads() -> int:
    return _load().kla_ref_max_threads()


_MODES = {"kaczmarz": 0, "direct": 1}


def forward(q, k, v, log_alpha, eta, eps, init_state=None, heads=None, nthreads=0, beta_mode="kaczmarz"):
    """Token-by-token float64 forward for a list of (b, h) heads (None = all heads).

    Returns (out [n, T, dv], final_state [n, dk, dv]) as float64, n = number of heads.
    """
    lib = _load()
    q, k, v, la, et, s0 = (_c32(x) for x in (q, k, v, log_alpha, eta, init_state))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if heads is None:
        idx = None
        n = B * H
    else:
        idx = np.ascontiguousarray([b * H + h for (b, h) in heads], dtype=np.int64)
        n = len(idx)
    out = np.zeros((n, T, dv), np.float64)
    fin = np.zeros((n, dk, dv), np.float64)
    rc = lib.kla_ref_forward(_fp(q), _fp(k), _fp(v), _fp(la), _fp(et), float(np.float32(eps)),
                             _fp(s0), idx.ctypes.data_as(_i64) if idx is not None else None, n,
                             out.ctypes.data_as(_d), fin.ctypes.data_as(_d), B, T, H, dk, dv,
                             int(nthreads), _MODES[beta_mode])
    if rc != 0:
        raise ValueError("kla_ref_forward: bad arguments")
    return out, fin


def decode_step(state, q, k, v, log_alpha, eta, eps, heads=None, nthreads=0, beta_mode="kaczmarz"):
    """One decode step for the listed (n, h) heads. ``state`` is float64 [n_heads, dk, dv]
    for exactly those heads and is updated in place. Returns out [n_heads, dv]."""
    lib = _load()
    q, k, v, la, et = (_c32(x) for x in (q, k, v, log_alpha, eta))
    N, H, dk = q.shape
    dv = v.shape[-1]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    if heads is None:
        idx = None
        n = N * H
    else:
        idx = np.ascontiguousarray([a * H + h for (a, h) in heads], dtype=np.int64)
        n = len(idx)
    assert state.shape == (n, dk, dv)
    out = np.zeros((n, dv), np.float64)
    rc = lib.kla_ref_decode_step(_fp(q), _fp(k), _fp(v), _fp(la), _fp(et), float(np.float32(eps)),
                                 state.ctypes.data_as(_d),
                                 idx.ctypes.data_as(_i64) if idx is not None else None, n,
                                 out.ctypes.data_as(_d), N, H, dk, dv, int(nthreads), _MODES[beta_mode])
    if rc != 0:
        raise ValueError("kla_ref_decode_step: bad arguments")
    return out
