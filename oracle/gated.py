"""fp64 oracle of the model-adjacent prefill/decode options.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

The in-projection of a Mamba block emits, next to x, B and C, a raw step-size
channel and a gate channel z ("Mamba-Family State-Space Model Kernels on a
Programmable CGLA", Sec. III-A).  The options apply the plainest reading of
what those channels do around the SSD core (the pages do not write it out):

  step size:  dt_eff = softplus(dt + dt_bias) = log(1 + exp(dt + dt_bias))
              (or dt + dt_bias without the softplus)
  gate:       y_out  = y * z * sigmoid(z)          (the whole output, skip term included)

Both are plain element-wise steps around the unchanged recurrence, so the
oracle is: preprocess dt in fp64, run the sequential fp64 oracle
(``oracle.ref``), gate its output in fp64.
"""
from __future__ import annotations

import numpy as np

from . import ref


def softplus(v):
    """log(1 + exp(v)) in fp64, without overflow for large v."""
    return np.logaddexp(0.0, np.asarray(v, np.float64))


def silu(z):
    """z * sigmoid(z) in fp64."""
    z = np.asarray(z, np.float64)
    return z * (0.5 * (1.0 + np.tanh(0.5 * z)))


def effective_dt(dt, dt_bias=None, dt_softplus=False):
    """The step size the recurrence uses.  dt [..., H]; dt_bias [H] or None."""
    v = np.asarray(dt, np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, np.float64)
    return softplus(v) if dt_softplus else v


def prefill(x, dt, A, B, C, D=None, h0=None, *, dt_bias=None, dt_softplus=False, z=None, nthreads: int = 0):
    """fp64 prefill with the options.  Returns (y [B,L,H,P], final_state [B,H,P,N])."""
    y, hT = ref.prefill(x, effective_dt(dt, dt_bias, dt_softplus), A, B, C, D, h0, nthreads=nthreads)
    if z is not None:
        y = y * silu(z)
    return y, hT


def step(state, x, dt, A, B, C, D=None, *, dt_bias=None, dt_softplus=False, z=None):
    """One fp64 decode token with the options; ``state`` (fp64) is updated in place."""
    y = ref.step(state, x, effective_dt(dt, dt_bias, dt_softplus), A, B, C, D)
    if z is not None:
        y = y * silu(z)
    return y
