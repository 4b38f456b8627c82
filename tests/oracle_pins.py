"""Pins for the fp64 C oracle (the sequential SSD recurrence).

The pages print no worked example with numbers, so the oracle is pinned to
things other than itself: a second fp64 formulation (the quadratic form), an
fp64 chunked evaluation in the method's step order, closed forms worked by
hand, a textbook special case (causal linear attention), and invariants.

Each ``pin_*`` takes the loaded oracle library so that the mutation test can
run the same pins against deliberately broken copies of the oracle.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from mamba_ssd_scan_amd import synth
from oracle import chunked, quadratic, ref
from tests.util import rel_err

TIGHT = 1e-12
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _pf(lib, inp, h0="use", D="use", nthreads=0):
    return ref.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                       inp["D"] if D == "use" else D,
                       inp["h0"] if isinstance(h0, str) else h0, nthreads=nthreads, lib=lib)


def pin_two_tokens_by_hand(lib):
    """L=2, P=2, N=3 worked by hand from the definition (tests/golden/two_tokens_by_hand.json)."""
    g = json.load(open(os.path.join(GOLDEN, "two_tokens_by_hand.json")))
    assert g["A_is_minus_ln2"]
    x = np.array(g["x"]).reshape(1, 2, 1, 2)
    dt = np.array(g["dt"]).reshape(1, 2, 1)
    A = np.array([-math.log(2.0)])
    Bm = np.array(g["B"]).reshape(1, 2, 1, 3)
    Cm = np.array(g["C"]).reshape(1, 2, 1, 3)
    H0 = np.array(g["h0"]).reshape(1, 1, 2, 3)
    y, hT = ref.prefill(x, dt, A, Bm, Cm, np.array([g["D"]]), H0, lib=lib)
    assert np.max(np.abs(y - np.array(g["y"]).reshape(1, 2, 1, 2))) < 1e-14, y
    assert np.max(np.abs(hT - np.array(g["final_state"]).reshape(1, 1, 2, 3))) < 1e-14, hT


def pin_scalar_geometric(lib):
    """H=P=N=G=1, x=B=C=1, constant dt and A: a geometric series.

    h_t = r^(t+1) h0 + dt (1 - r^(t+1)) / (1 - r),   r = exp(dt A);   y_t = h_t + D.
    """
    L, dtv, Av, h0v, Dv = 50, 0.3, -0.7, 0.5, 0.25
    ones = np.ones((1, L, 1, 1))
    y, hT = ref.prefill(ones, np.full((1, L, 1), dtv), np.array([Av]), ones, ones,
                        np.array([Dv]), np.array([[[[h0v]]]]), lib=lib)
    r = math.exp(dtv * Av)
    t = np.arange(L)
    h = r ** (t + 1) * h0v + dtv * (1 - r ** (t + 1)) / (1 - r)
    assert rel_err(y[0, :, 0, 0], h + Dv) < TIGHT
    assert rel_err(hT[0, 0, 0, 0], h[-1]) < TIGHT


def pin_causal_linear_attention(lib):
    """A = 0, D = 0, dt = 1: no decay, so y = tril(C B^T) X + C H0^T (per b, h)."""
    inp = synth.random_prefill(_rng(11), 2, 29, 3, 5, 7, 1, "f32")
    inp["A"] = np.zeros(3, np.float32)
    inp["dt"] = np.ones_like(inp["dt"])
    y, hT = _pf(lib, inp, D=None)
    for b in range(2):
        for h in range(3):
            Cb, Bb, Xb = (inp["C"][b, :, 0].astype(np.float64), inp["B"][b, :, 0].astype(np.float64),
                          inp["x"][b, :, h].astype(np.float64))
            H0 = inp["h0"][b, h].astype(np.float64)
            want = np.tril(Cb @ Bb.T) @ Xb + Cb @ H0.T
            assert rel_err(y[b, :, h], want) < TIGHT
            assert rel_err(hT[b, h], Xb.T @ Bb + H0) < TIGHT


def pin_decay_only(lib):
    """x = 0: the state only decays, H_t = exp(A * sum_{s<=t} dt_s) H0."""
    inp = synth.random_prefill(_rng(12), 1, 40, 2, 3, 4, 1, "f32")
    inp["x"] = np.zeros_like(inp["x"])
    y, hT = _pf(lib, inp)
    for h in range(2):
        cum = np.cumsum(inp["dt"][0, :, h].astype(np.float64)) * float(inp["A"][h])
        H0 = inp["h0"][0, h].astype(np.float64)
        want_y = np.exp(cum)[:, None] * (inp["C"][0, :, 0].astype(np.float64) @ H0.T)
        assert rel_err(y[0, :, h], want_y) < TIGHT
        assert rel_err(hT[0, h], math.exp(cum[-1]) * H0) < TIGHT


def pin_dt_zero(lib):
    """dt = 0: the state is bitwise unchanged and y_t = H0 C_t + D x_t."""
    inp = synth.random_prefill(_rng(13), 2, 17, 3, 4, 6, 1, "f32")
    inp["dt"] = np.zeros_like(inp["dt"])
    y, hT = _pf(lib, inp)
    assert np.array_equal(hT, inp["h0"].astype(np.float64))
    for b in range(2):
        for h in range(3):
            want = (inp["C"][b, :, 0].astype(np.float64) @ inp["h0"][b, h].astype(np.float64).T
                    + float(inp["D"][h]) * inp["x"][b, :, h].astype(np.float64))
            assert rel_err(y[b, :, h], want) < TIGHT


def pin_quadratic_form(lib):
    """Sequential recurrence == brute-force quadratic form (two fp64 algorithms)."""
    cases = [((2, 37, 4, 8, 16, 2), "softplus", True), ((1, 64, 3, 5, 7, 1), "weak", True),
             ((1, 1, 2, 3, 4, 2), "softplus", False), ((1, 50, 2, 4, 4, 1), "strong", True)]
    for k, (shape, mode, h0) in enumerate(cases):
        inp = synth.random_prefill(_rng(100 + k), *shape, "f32", init_state=h0, dt_mode=mode)
        y1, h1 = _pf(lib, inp)
        y2, h2 = quadratic.quadratic_form(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
        assert rel_err(y1, y2) < TIGHT, (shape, mode)
        assert rel_err(h1, h2) < TIGHT, (shape, mode)
        # the SSD part alone (D = 0) so that the skip term cannot hide an error
        y1, _ = _pf(lib, inp, D=None)
        y2, _ = quadratic.quadratic_form(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], None, inp["h0"])
        assert rel_err(y1, y2) < TIGHT, (shape, mode)


def pin_group_mapping(lib):
    """Head h reads group h // (H/G): compare G=2 with per-group G=1 runs."""
    inp = synth.random_prefill(_rng(14), 1, 21, 4, 3, 5, 2, "f32")
    y, hT = _pf(lib, inp)
    for h in range(4):
        g = h // 2
        sub = synth.select_heads(dict(inp), [h], 2, 4)
        assert np.array_equal(sub["B"], inp["B"][:, :, g:g + 1])
        ys, hs = _pf(lib, sub)
        assert np.array_equal(ys[:, :, 0], y[:, :, h])
        assert np.array_equal(hs[:, 0], hT[:, h])


def pin_split_sequence(lib):
    """prefill(0:L1) -> final -> prefill(L1:L) == prefill(0:L): the state is the cache."""
    inp = synth.random_prefill(_rng(15), 2, 45, 2, 4, 6, 1, "f32", dt_mode="weak")
    y, hT = _pf(lib, inp)
    L1 = 19
    a = {k: (v[:, :L1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    b = {k: (v[:, L1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    ya, ha = _pf(lib, a)
    yb, hb = _pf(lib, b, h0=ha)
    assert rel_err(np.concatenate([ya, yb], axis=1), y) < TIGHT
    assert rel_err(hb, hT) < TIGHT


def pin_linearity(lib):
    """y and the final state are linear in (x, H0) jointly."""
    i1 = synth.random_prefill(_rng(16), 1, 23, 3, 4, 5, 1, "f32")
    i2 = synth.random_prefill(_rng(17), 1, 23, 3, 4, 5, 1, "f32")
    i2.update({k: i1[k] for k in ("dt", "A", "B", "C", "D")})
    mix = dict(i1)
    mix["x"] = i1["x"].astype(np.float64) - 2.5 * i2["x"].astype(np.float64)
    mix["h0"] = i1["h0"].astype(np.float64) - 2.5 * i2["h0"].astype(np.float64)
    y1, h1 = _pf(lib, i1)
    y2, h2 = _pf(lib, i2)
    ym, hm = _pf(lib, mix)
    assert rel_err(ym, y1 - 2.5 * y2) < 1e-12
    assert rel_err(hm, h1 - 2.5 * h2) < 1e-12


def pin_bc_rescale(lib):
    """With H0 = 0: B -> sB, C -> C/s leaves y unchanged and scales the state by s."""
    inp = synth.random_prefill(_rng(18), 1, 31, 2, 4, 6, 1, "f32", init_state=False)
    y, hT = _pf(lib, inp)
    s = 4.0  # a power of two: the rescaling is exact
    sc = dict(inp)
    sc["B"] = inp["B"] * s
    sc["C"] = inp["C"] / s
    ys, hs = _pf(lib, sc)
    assert rel_err(ys, y) < TIGHT
    assert rel_err(hs, s * hT) < TIGHT


def pin_permutations(lib):
    """Permuting heads or batch entries permutes the outputs (G = 1)."""
    inp = synth.random_prefill(_rng(19), 3, 13, 4, 3, 4, 1, "f32")
    y, hT = _pf(lib, inp)
    ph = np.array([2, 0, 3, 1])
    p = dict(inp, x=inp["x"][:, :, ph], dt=inp["dt"][:, :, ph], A=inp["A"][ph], D=inp["D"][ph],
             h0=inp["h0"][:, ph])
    yp, hp = _pf(lib, p)
    assert np.array_equal(yp, y[:, :, ph]) and np.array_equal(hp, hT[:, ph])
    pb = np.array([1, 2, 0])
    p = dict(inp, x=inp["x"][pb], dt=inp["dt"][pb], B=inp["B"][pb], C=inp["C"][pb], h0=inp["h0"][pb])
    yp, hp = _pf(lib, p)
    assert np.array_equal(yp, y[pb]) and np.array_equal(hp, hT[pb])


def pin_step_extends_prefill(lib):
    """prefill(L) followed by k decode steps == prefill(L + k)."""
    inp = synth.random_prefill(_rng(20), 2, 30, 3, 4, 5, 1, "f32")
    y, hT = _pf(lib, inp)
    L0 = 26
    head = {k: (v[:, :L0] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    _, st = _pf(lib, head)
    st = np.ascontiguousarray(st)
    for t in range(L0, 30):
        ys = ref.step(st, inp["x"][:, t], inp["dt"][:, t], inp["A"], inp["B"][:, t], inp["C"][:, t],
                      inp["D"], lib=lib)
        assert rel_err(ys, y[:, t]) < TIGHT
    assert rel_err(st, hT) < TIGHT


def pin_chunked_every_Q(lib):
    """The fp64 chunked evaluation equals the recurrence for every chunk length Q."""
    inp = synth.random_prefill(_rng(21), 1, 23, 2, 4, 6, 1, "f32", dt_mode="weak")
    y, hT = _pf(lib, inp)
    for Q in list(range(1, 24)) + [32, 64]:
        r = chunked.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], Q=Q)
        assert rel_err(r["y"], y) < TIGHT, Q
        assert rel_err(r["final"], hT) < TIGHT, Q


def pin_chunked_intermediates(lib):
    """Chunk states and entering states equal runs of the recurrence itself.

    S_c is the state left by chunk c's tokens from a zero start; H_enter[c]
    is the state after tokens 0 .. cQ-1 from H0; exp(A_cum[i]) is the decay a
    state suffers over chunk tokens 0..i (an x = 0 run from an all-ones state).
    """
    Q = 8
    inp = synth.random_prefill(_rng(22), 1, 29, 2, 3, 4, 1, "f32", dt_mode="weak")
    r = chunked.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], Q=Q)
    sl = lambda d, t0, t1: {k: (v[:, t0:t1] if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    for c in range(4):
        t0, t1 = c * Q, min(29, (c + 1) * Q)
        _, S = _pf(lib, sl(inp, t0, t1), h0=None)
        assert rel_err(r["states"][:, :, c], S) < TIGHT
        if c > 0:
            _, He = _pf(lib, sl(inp, 0, t0))
            assert rel_err(r["h_enter"][:, :, c], He) < TIGHT
        for i in range(t1 - t0):
            z = sl(inp, t0, t0 + i + 1)
            z["x"] = np.zeros_like(z["x"])
            ones = np.ones_like(inp["h0"])
            _, Hd = _pf(lib, z, h0=ones)
            assert rel_err(np.exp(r["acum"][0, :, c, i]), Hd[0, :, 0, 0]) < TIGHT


ALL_PINS = [
    pin_two_tokens_by_hand, pin_scalar_geometric, pin_causal_linear_attention, pin_decay_only,
    pin_dt_zero, pin_quadratic_form, pin_group_mapping, pin_split_sequence, pin_linearity,
    pin_bc_rescale, pin_permutations, pin_step_extends_prefill, pin_chunked_every_Q,
    pin_chunked_intermediates,
]
