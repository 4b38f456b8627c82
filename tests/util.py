"""Shared test helpers: error metrics and tolerances."""
import numpy as np

# Tolerances on the normwise relative error below, per input storage type.
# fp8 (e4m3 x, B and C; bf16 dt): the inputs are exact values, and every matrix-core operand
# computed from them is fp16 as for bf16 inputs, so the bf16 bar applies.
TOL = {"bf16": 2e-3, "f32": 1e-4, "fp8": 2e-3}


def rel_err(t, o) -> float:
    """max_i |t_i - o_i| / max_i |o_i|  (normwise infinity-norm relative error).

    Elementwise |t-o|/|o| is undefined where the oracle value is near zero, so
    the error is measured against the largest oracle magnitude of the tensor.
    """
    t = np.asarray(t, np.float64)
    o = np.asarray(o, np.float64)
    if o.size == 0:
        return 0.0
    scale = np.max(np.abs(o))
    diff = np.max(np.abs(t - o))
    if scale == 0.0:
        return float(diff)
    return float(diff / scale)
