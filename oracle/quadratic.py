"""fp64 brute-force quadratic ("masked attention") form of the SSD layer core.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Unrolling the per-head recurrence (state decayed by exp(dt_t * A_h) at every
token, input dt_t * x_t * B_t^T added, output read as state times C_t) gives,
for one (b, h) with s_t = sum_{k<=t} dt_k * A_h over the whole sequence:

    y_t = sum_{s<=t} exp(s_t - s_s) * dt_s * (C_t . B_s) * x_s      (intra)
        + exp(s_t) * H0 C_t                                        (initial state)
        + D_h * x_t                                                (skip)
    H_L = sum_s exp(s_{L-1} - s_s) * dt_s * x_s B_s^T + exp(s_{L-1}) * H0

This is the "dual" (attention-like) view that the SSD method's intra-chunk
step uses on each chunk: GEMM over the state dimension (C B^T), a Hadamard
mask with the decay matrix, then a GEMM over the time axis
("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec. III-A
and Sec. IV-B).  Here it is applied to the whole sequence at once, with no
chunking, as a second, independent formulation of the definition.
Only meant for short sequences (it is O(L^2) per head).
"""
from __future__ import annotations

import numpy as np


def quadratic_form(x, dt, A, B, C, D=None, h0=None):
    """Returns (y [Bt,L,H,P], final_state [Bt,H,P,N]) in fp64."""
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    Bm = np.asarray(B, np.float64)
    Cm = np.asarray(C, np.float64)
    nb, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((nb, L, H, P))
    hT = np.zeros((nb, H, P, N))
    if L == 0:
        if h0 is not None:
            hT[...] = h0
        return y, hT
    causal = np.tril(np.ones((L, L), dtype=bool))
    for b in range(nb):
        for h in range(H):
            g = h // hpg
            s = np.cumsum(dt[b, :, h] * A[h])                    # s_t
            seg = s[:, None] - s[None, :]                        # s_t - s_s
            decay = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
            scores = Cm[b, :, g, :] @ Bm[b, :, g, :].T           # (C_t . B_s)
            M = scores * decay * dt[b, None, :, h]               # [t, s]
            yy = M @ x[b, :, h, :]
            w_end = np.exp(s[-1] - s) * dt[b, :, h]              # weight of token s in H_L
            hh = (x[b, :, h, :] * w_end[:, None]).T @ Bm[b, :, g, :]
            if h0 is not None:
                H0 = np.asarray(h0[b, h], np.float64)
                yy = yy + np.exp(s)[:, None] * (Cm[b, :, g, :] @ H0.T)
                hh = hh + np.exp(s[-1]) * H0
            if D is not None:
                yy = yy + float(D[h]) * x[b, :, h, :]
            y[b, :, h, :] = yy
            hT[b, h] = hh
    return y, hT
