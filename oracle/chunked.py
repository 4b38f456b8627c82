"""fp64 chunked evaluation of the SSD layer core, step by step.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

The sequence is cut into chunks of Q tokens ("Mamba-Family State-Space Model
Kernels on a Programmable CGLA", Sec. III-A).  With a_t = dt_t * A_h and
A_cum[i] the inclusive sum of a over the chunk's tokens 0..i:

  Step-0  per-chunk cumulative decay A_cum, the chunk's total decay
          exp(A_cum[last]), the decay matrix Lmat[i,j] = exp(A_cum[i]-A_cum[j])
          for j <= i (zero above the diagonal; Lmat[i,i] = 1).
  Step-1  intra-chunk output: GEMM1 over the state dim (C_c B_c^T), Hadamard
          mask with Lmat and dt_j, GEMM2 over the chunk's time axis with X_c
          (Sec. III-A and Sec. IV-B of the same page).
  Step-2  chunk state: S_c = sum_j exp(A_cum[last]-A_cum[j]) dt_j x_j B_j^T,
          the state a chunk would leave behind from a zero start.
  Step-3  inter-chunk recurrence, sequential over chunks: the state entering
          chunk c+1 is exp(A_cum_c[last]) * (state entering c) + S_c, the
          diagonal per-head decay being a scalar per head (Sec. III-A and
          Sec. IV-C of the same page).
  Step-4  off-diagonal output: exp(A_cum[i]) * C_i . H_enter[c], plus the
          skip term D_h * x_i.

A ragged last chunk simply has fewer tokens.  The intermediates are returned
in the layouts the GPU library's stage entry points use, with the last chunk
padded as if by tokens with dt = 0 and x = 0 (A_cum stays constant, dt = 0);
the GEMM1 products come back as full [Q, Q] matrices per (batch, group,
chunk), lower triangle only (zero above the diagonal and past the sequence).
"""
from __future__ import annotations

import numpy as np


def chunked(x, dt, A, B, C, D=None, h0=None, *, Q: int):
    x = np.asarray(x, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    Bm = np.asarray(B, np.float64)
    Cm = np.asarray(C, np.float64)
    nb, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    nc = -(-L // Q)
    y = np.zeros((nb, L, H, P))
    acum = np.zeros((nb, H, nc, Q))
    dtp = np.zeros((nb, H, nc, Q))
    states = np.zeros((nb, H, nc, P, N))
    h_enter = np.zeros((nb, H, nc, P, N))
    final = np.zeros((nb, H, P, N))
    gemm1 = np.zeros((nb, G, nc, Q, Q))
    for b in range(nb):
        for h in range(H):
            g = h // hpg
            run = np.zeros((P, N)) if h0 is None else np.asarray(h0[b, h], np.float64).copy()
            for c in range(nc):
                t0, t1 = c * Q, min(L, (c + 1) * Q)
                q = t1 - t0
                dtc = dt[b, t0:t1, h]
                Xc = x[b, t0:t1, h, :]
                Bc = Bm[b, t0:t1, g, :]
                Cc = Cm[b, t0:t1, g, :]
                # Step-0
                ac = np.cumsum(dtc * A[h])
                acum[b, h, c, :q] = ac
                acum[b, h, c, q:] = ac[-1]
                dtp[b, h, c, :q] = dtc
                seg = ac[:, None] - ac[None, :]
                lower = np.tril(np.ones((q, q), dtype=bool))
                Lmat = np.where(lower, np.exp(np.where(lower, seg, 0.0)), 0.0)
                # Step-1: GEMM1 -> Hadamard -> GEMM2
                G1 = Cc @ Bc.T
                gemm1[b, g, c, :q, :q] = np.tril(G1)
                R = G1 * Lmat * dtc[None, :]
                y_diag = R @ Xc
                # Step-2
                w = np.exp(ac[-1] - ac) * dtc
                S = (Xc * w[:, None]).T @ Bc
                states[b, h, c] = S
                # Step-3 (entering state for this chunk, then advance)
                h_enter[b, h, c] = run
                y_off = np.exp(ac)[:, None] * (Cc @ run.T)
                run = np.exp(ac[-1]) * run + S
                # Step-4
                yc = y_diag + y_off
                if D is not None:
                    yc = yc + float(D[h]) * Xc
                y[b, t0:t1, h, :] = yc
            final[b, h] = run
    return dict(y=y, final=final, acum=acum, dt=dtp, states=states, h_enter=h_enter, gemm1=gemm1)
