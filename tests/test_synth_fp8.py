"""CPU pins of the fp8 (OCP e4m3) input helpers that both sides use: the rounding that makes
fp8 inputs, the codes the kernels read and the value of every code.  Pinned to the format's
definition (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent 0, the
all-ones codes NaN, no infinities), to hand-worked values, and to torch's own float8_e4m3fn
conversion as an independent implementation."""
from __future__ import annotations

import numpy as np
import pytest

from mamba_ssd_scan_amd import synth


def test_named_codes_have_the_formats_values():
    # 0x38: exponent 7 (bias 7), mantissa 0 -> 1.0;  0x7e: exponent 15, mantissa 6 -> 1.75 * 2^8
    # 0x08: the least normal 2^-6;  0x01: the least subnormal 2^-9;  0x07: the largest subnormal 7 * 2^-9
    pins = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0,
            0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x77: 240.0, 0x78: 256.0}
    for code, v in pins.items():
        assert synth.e4m3_value(code) == v, hex(code)
    assert np.isnan(synth.e4m3_value(0x7F)) and np.isnan(synth.e4m3_value(0xFF))
    assert synth.E4M3_MAX == 448.0
    assert np.signbit(synth.e4m3_value(0x80)) and synth.e4m3_value(0x80) == 0.0


def test_every_code_matches_torch_float8_e4m3fn():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ours = np.array([synth.e4m3_value(c) for c in range(256)], np.float32)
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], ours[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(ours[fin]))


def test_codes_round_trip_every_finite_value():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = np.array([synth.e4m3_value(c) for c in finite], np.float32)
    assert np.array_equal(synth.e4m3_codes(vals), np.array(finite, np.uint8))
    assert np.array_equal(synth.e4m3_round(vals), vals)  # representable values are fixed points


def test_rounding_ties_go_to_the_even_mantissa():
    # spacing 1/8 in [1, 2): 1.0625 is halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1)
    assert synth.e4m3_round(np.float32(1.0625)) == 1.0
    assert synth.e4m3_round(np.float32(1.1875)) == 1.25     # between mantissas 1 and 2: to 2
    assert synth.e4m3_round(np.float32(-1.1875)) == -1.25
    # spacing 2^-9 among the subnormals: 1.5 * 2^-9 goes to 2 * 2^-9, 0.5 * 2^-9 to zero
    assert synth.e4m3_round(np.float32(1.5 * 2.0 ** -9)) == 2.0 ** -8
    assert synth.e4m3_round(np.float32(0.5 * 2.0 ** -9)) == 0.0
    # spacing 32 in [256, 512): 432 is halfway between 416 (mantissa 5) and 448 (mantissa 6)
    assert synth.e4m3_round(np.float32(432.0)) == 448.0
    assert synth.e4m3_round(np.float32(463.0)) == 448.0


def test_rounding_matches_torch_on_random_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    a = np.concatenate([rng.standard_normal(20000), rng.uniform(-460, 460, 20000),
                        rng.standard_normal(20000) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(synth.e4m3_round(a), ref)


def test_values_past_the_largest_finite_are_refused():
    with pytest.raises(ValueError):
        synth.e4m3_round(np.float32(464.0))
    with pytest.raises(ValueError):
        synth.e4m3_round(np.float32(-1000.0))
