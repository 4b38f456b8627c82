"""Pins for the fp64 oracle of the model-adjacent options (oracle/gated.py).

softplus and the gate are pinned by values fixed by their definitions and by
special cases that reduce the option path to the plain recurrence:
  - softplus(0) = ln 2; softplus(v) -> v for large v, -> exp(v) for very negative v;
    softplus(v) - softplus(-v) = v (an identity of log(1 + e^v));
  - silu(0) = 0, silu(1) = 1 / (1 + e^-1), silu(-v) = silu(v) - v;
  - dt_raw = log(expm1(d)) - bias gives softplus(dt_raw + bias) = d, so the option
    path must reproduce the plain oracle run with step size d;
  - z = 0 zeroes the output; z large gives y * z (sigmoid -> 1).
"""
from __future__ import annotations

import math

import numpy as np

from mamba_ssd_scan_amd import synth
from oracle import gated, ref
from tests.util import rel_err


def _inp(seed=7, L=40, H=4, P=8, N=16, G=2):
    rng = np.random.Generator(np.random.PCG64(seed))
    return synth.random_prefill(rng, 2, L, H, P, N, G, "f32")


def test_softplus_values():
    assert abs(gated.softplus(0.0) - math.log(2.0)) < 1e-15
    assert gated.softplus(800.0) == 800.0                      # no overflow, exact in fp64
    assert abs(gated.softplus(-50.0) / math.exp(-50.0) - 1.0) < 1e-15
    v = np.linspace(-30, 30, 121)
    assert np.max(np.abs(gated.softplus(v) - gated.softplus(-v) - v)) < 1e-13


def test_silu_values():
    assert gated.silu(0.0) == 0.0
    assert abs(gated.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    v = np.linspace(-20, 20, 81)
    assert np.max(np.abs(gated.silu(-v) - (gated.silu(v) - v))) < 1e-13


def test_softplus_path_reduces_to_plain_recurrence():
    inp = _inp()
    H = inp["A"].shape[0]
    bias = np.linspace(-1.0, 1.0, H)
    d = np.asarray(inp["dt"], np.float64)                       # positive step sizes
    dt_raw = np.log(np.expm1(d)) - bias                         # softplus(dt_raw + bias) = d
    y1, h1 = gated.prefill(inp["x"], dt_raw, inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                           dt_bias=bias, dt_softplus=True)
    y0, h0 = ref.prefill(inp["x"], d, inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    assert rel_err(y1, y0) < 1e-12 and rel_err(h1, h0) < 1e-12
    # bias alone, no softplus: dt + bias
    y2, _ = gated.prefill(inp["x"], d - bias, inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], dt_bias=bias)
    assert rel_err(y2, y0) < 1e-12


def test_gate_special_cases():
    inp = _inp(seed=8)
    y0, h0 = ref.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    yz, hz = gated.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                           z=np.zeros_like(inp["x"]))
    assert np.all(yz == 0.0) and np.array_equal(hz, h0)         # the gate never touches the state
    big = np.full_like(inp["x"], 40.0)                          # sigmoid(40) = 1 - 4e-18
    yb, _ = gated.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], z=big)
    assert rel_err(yb, 40.0 * y0) < 1e-15


def test_step_options_match_prefill_options():
    """One option step per token reproduces the option prefill (the cache property)."""
    inp = _inp(seed=9, L=12)
    H = inp["A"].shape[0]
    rng = np.random.Generator(np.random.PCG64(10))
    bias = rng.normal(size=H)
    dt_raw = rng.normal(-1.0, 1.0, size=inp["dt"].shape)
    z = rng.normal(size=inp["x"].shape)
    yp, hp = gated.prefill(inp["x"], dt_raw, inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                           dt_bias=bias, dt_softplus=True, z=z)
    st = np.array(inp["h0"], np.float64)
    for t in range(inp["x"].shape[1]):
        ys = gated.step(st, inp["x"][:, t], dt_raw[:, t], inp["A"], inp["B"][:, t], inp["C"][:, t], inp["D"],
                        dt_bias=bias, dt_softplus=True, z=z[:, t])
        assert rel_err(ys, yp[:, t]) < 1e-12
    assert rel_err(st, hp) < 1e-12
