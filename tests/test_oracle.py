"""CPU tests of the fp64 oracle: pins, determinism, edge cases, and a
mutation test showing that the pins catch plausible mistakes."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

from mamba_ssd_scan_amd import synth
from oracle import build, chunked, quadratic, ref
from tests import oracle_pins
from tests.util import rel_err


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ref.load())


def test_bitwise_deterministic_across_thread_counts():
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(5)), 3, 40, 5, 8, 16, 1, "f32")
    outs = [ref.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], nthreads=n)
            for n in (1, 3, 8)]
    for y, h in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(h, outs[0][1])


def test_empty_sequence_keeps_state():
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(6)), 2, 0, 2, 4, 4, 1, "f32")
    y, hT = ref.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    assert y.shape == (2, 0, 2, 4)
    assert np.array_equal(hT, inp["h0"].astype(np.float64))


def test_final_state_may_alias_initial_state():
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(7)), 2, 19, 3, 4, 5, 1, "f32")
    f64 = lambda a: np.ascontiguousarray(a, np.float64)
    y_ref, h_ref = ref.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    x, dt, A, Bm, Cm, D = map(f64, (inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"]))
    st = f64(inp["h0"]).copy()
    y = np.empty_like(x)
    p = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    rc = ref.load().ssd_oracle_prefill(p(x), p(dt), p(A), p(Bm), p(Cm), p(D), p(st), p(y), p(st),
                                      2, 19, 3, 4, 5, 1, 0)
    assert rc == 0
    assert np.array_equal(y, y_ref) and np.array_equal(st, h_ref)


def test_rejects_bad_shapes():
    lib = ref.load()
    z = ctypes.POINTER(ctypes.c_double)()
    assert lib.ssd_oracle_prefill(z, z, z, z, z, z, z, z, z, 1, 4, 3, 4, 4, 2, 1) < 0  # H % G != 0
    assert lib.ssd_oracle_prefill(z, z, z, z, z, z, z, z, z, 0, 4, 2, 4, 4, 1, 1) < 0  # batch 0


def test_decode_wrapper_matches_prefill():
    rng = np.random.Generator(np.random.PCG64(8))
    inp = synth.random_prefill(rng, 2, 12, 3, 4, 6, 1, "f32")
    y, hT = ref.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])
    ys, st = ref.decode(inp["h0"], inp["x"].transpose(1, 0, 2, 3), inp["dt"].transpose(1, 0, 2), inp["A"],
                        inp["B"].transpose(1, 0, 2, 3), inp["C"].transpose(1, 0, 2, 3), inp["D"])
    assert rel_err(ys.transpose(1, 0, 2, 3), y) < 1e-13
    assert rel_err(st, hT) < 1e-13


def test_chunked_ragged_padding_layout():
    """The padded tail of the last chunk holds A_cum constant and dt = 0."""
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(9)), 1, 21, 2, 4, 4, 1, "f32")
    r = chunked.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], Q=8)
    assert r["acum"].shape == (1, 2, 3, 8)
    assert np.all(r["acum"][:, :, 2, 5:] == r["acum"][:, :, 2, 4:5])
    assert np.all(r["dt"][:, :, 2, 5:] == 0.0)


def test_chunked_intermediates_against_recurrence_and_quadratic_form():
    """The chunked oracle's intermediates, each pinned to another formulation (the end-to-end
    pins only see y and the final state):

    - the entering state of chunk c is the sequential recurrence's state after the first cQ
      tokens (the C oracle run on that prefix);
    - the chunk state S_c is the recurrence's state after chunk c alone, from a zero state;
    - the GEMM1 product of a chunk is the quadratic form's score matrix on that chunk's block:
      with A = 0 and dt = 1 the decay mask is 1 under the diagonal, and with one-hot x (P = L
      channels) the form's output row t is row t of that matrix.
    """
    rng = np.random.Generator(np.random.PCG64(31))
    B_, L, H, P, N, G, Q = 2, 37, 4, 5, 6, 2, 8
    inp = synth.random_prefill(rng, B_, L, H, P, N, G, "f32", init_state="randn")
    r = chunked.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], Q=Q)
    nc = -(-L // Q)
    for c in range(nc):
        t0, t1 = c * Q, min(L, (c + 1) * Q)
        if c > 0:
            _, h_pre = ref.prefill(inp["x"][:, :t0], inp["dt"][:, :t0], inp["A"], inp["B"][:, :t0],
                                   inp["C"][:, :t0], None, inp["h0"])
        else:
            h_pre = inp["h0"]
        assert rel_err(r["h_enter"][:, :, c], h_pre) < 1e-12, c
        _, s_c = ref.prefill(inp["x"][:, t0:t1], inp["dt"][:, t0:t1], inp["A"], inp["B"][:, t0:t1],
                             inp["C"][:, t0:t1], None, None)
        assert rel_err(r["states"][:, :, c], s_c) < 1e-12, c
    # GEMM1 against the quadratic form's scores
    Lg = 2 * Q + 3
    Bm = rng.standard_normal((1, Lg, 1, N))
    Cm = rng.standard_normal((1, Lg, 1, N))
    onehot = np.eye(Lg)[None, :, None, :]               # x[0, s, 0, :] = e_s
    ones, zero = np.ones((1, Lg, 1)), np.zeros(1)
    yq, _ = quadratic.quadratic_form(onehot, ones, zero, Bm, Cm)
    g1 = chunked.chunked(onehot, ones, zero, Bm, Cm, Q=Q)["gemm1"]
    for c in range(-(-Lg // Q)):
        t0, t1 = c * Q, min(Lg, (c + 1) * Q)
        block = yq[0, t0:t1, 0, t0:t1]                    # scores of the chunk's own tokens
        assert np.allclose(g1[0, 0, c, :t1 - t0, :t1 - t0], block, rtol=0, atol=1e-12), c
        assert np.all(g1[0, 0, c, :, :][np.triu_indices(Q, 1)] == 0.0)


# ---------------------------------------------------------------------------
# Mutation test: plant a mistake in a copy of the oracle source, build it, and
# check that at least one pin fails.  Each mutant is a plausible slip.
MUTANTS = {
    "drop_skip_term": ("yt[p] = acc + Dh * xt[p];", "yt[p] = acc;"),
    "read_state_before_update": (
        "row[n] = r * row[n] + u * Bt[n];\n            acc += row[n] * Ct[n];",
        "acc += row[n] * Ct[n];\n            row[n] = r * row[n] + u * Bt[n];"),
    "decay_current_input": ("row[n] = r * row[n] + u * Bt[n];", "row[n] = r * (row[n] + u * Bt[n]);"),
    "flip_decay_sign": ("exp(dtv * Ah)", "exp(-dtv * Ah)"),
    "decay_without_dt": ("exp(dtv * Ah)", "exp(Ah)"),
    "input_without_dt": ("const double u = dtv * xt[p];", "const double u = xt[p];"),
    "swap_B_and_C": ("u * Bt[n];\n            acc += row[n] * Ct[n];", "u * Ct[n];\n            acc += row[n] * Bt[n];"),
    "interleaved_groups": ("const int g = h / heads_per_group;\n        double *M", "const int g = h % G;\n        double *M"),
    "ignore_initial_state": ("if (h0)\n", "if (0)\n"),
    "previous_token_B": ("Bm + (tok * G + g) * N", "Bm + ((t > 0 ? tok - 1 : tok) * G + g) * N"),
    "drop_last_token": ("for (int t = 0; t < L; ++t)", "for (int t = 0; t < L - 1; ++t)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    old, new = MUTANTS[name]
    src = open(build.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/present"
    tmp = tempfile.mkdtemp(prefix="ssd_oracle_mut_")
    try:
        msrc = os.path.join(tmp, "mut.c")
        with open(msrc, "w") as f:
            f.write(src.replace(old, new))
        lib_path = os.path.join(tmp, "libmut.so")
        build.compile_oracle(msrc, lib_path, extra=["-Wno-unused-variable", "-Wno-unused-parameter",
                                                    "-Wno-error"])
        lib = ref.load(lib_path)
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"no pin caught mutant {name}"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_oracle_regression_fixture():
    """Bitwise match with the fixture written by tests/golden/make_golden.py."""
    import json
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
    import make_golden
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")))
    assert g["case"] == make_golden.CASE
    _, (y, hT) = make_golden.compute()
    assert [float.hex(float(v)) for v in y.ravel()] == g["y"]
    assert [float.hex(float(v)) for v in hT.ravel()] == g["final_state"]
