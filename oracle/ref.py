"""ctypes wrapper over the fp64 C oracle (the sequential recurrence).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

from . import build

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)


def load(path: Optional[str] = None):
    """Load the oracle library (building it with gcc if it is missing)."""
    global _lib
    if path is not None:
        lib = ctypes.CDLL(path)
    else:
        if _lib is not None:
            return _lib
        lib = ctypes.CDLL(build.ensure_built())
    i = ctypes.c_int
    lib.ssd_oracle_prefill.argtypes = [_dp] * 9 + [i] * 7
    lib.ssd_oracle_prefill.restype = i
    lib.ssd_oracle_step.argtypes = [_dp] * 8 + [i] * 6
    lib.ssd_oracle_step.restype = i
    lib.ssd_oracle_max_threads.argtypes = []
    lib.ssd_oracle_max_threads.restype = i
    if path is None:
        _lib = lib
    return lib


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def max_threads() -> int:
    return load().ssd_oracle_max_threads()


def prefill(x, dt, A, B, C, D=None, h0=None, *, nthreads: int = 0, lib=None):
    """fp64 sequential prefill.  Returns (y [B,L,H,P], final_state [B,H,P,N])."""
    lib = lib or load()
    x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, h0))
    batch, seqlen, nheads, headdim = x.shape
    ngroups, dstate = B.shape[2], B.shape[3]
    assert dt.shape == (batch, seqlen, nheads) and A.shape == (nheads,)
    assert B.shape == C.shape == (batch, seqlen, ngroups, dstate)
    assert D is None or D.shape == (nheads,)
    assert h0 is None or h0.shape == (batch, nheads, headdim, dstate)
    y = np.empty_like(x)
    hT = np.empty((batch, nheads, headdim, dstate), np.float64)
    st = lib.ssd_oracle_prefill(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0),
                                _ptr(y), _ptr(hT), batch, seqlen, nheads, headdim, dstate, ngroups,
                                int(nthreads))
    if st != 0:
        raise RuntimeError(f"ssd_oracle_prefill failed with status {st}")
    return y, hT


def step(state, x, dt, A, B, C, D=None, *, nthreads: int = 0, lib=None):
    """One fp64 decode token; ``state`` (fp64, [B,H,P,N]) is updated in place.

    x [B,H,P], dt [B,H], B/C [B,G,N].  Returns y [B,H,P].
    """
    lib = lib or load()
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise TypeError("state must be a C-contiguous float64 array (updated in place)")
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    batch, nheads, headdim, dstate = state.shape
    ngroups = B.shape[1]
    assert x.shape == (batch, nheads, headdim) and dt.shape == (batch, nheads)
    assert B.shape == C.shape == (batch, ngroups, dstate)
    y = np.empty_like(x)
    st = lib.ssd_oracle_step(_ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y),
                             batch, nheads, headdim, dstate, ngroups, int(nthreads))
    if st != 0:
        raise RuntimeError(f"ssd_oracle_step failed with status {st}")
    return y


def decode(state0, xs, dts, A, Bs, Cs, D=None, *, nthreads: int = 0):
    """Run ``len(xs)`` decode tokens from ``state0``.  Returns (ys [S,B,H,P], state)."""
    state = np.array(state0, dtype=np.float64, order="C", copy=True)
    ys = np.empty(np.shape(xs), np.float64)
    for s in range(len(xs)):
        ys[s] = step(state, xs[s], dts[s], A, Bs[s], Cs[s], D, nthreads=nthreads)
    return ys, state
