"""GPU tests of ssd_prefill_timed, the prefill with every kernel launch bound to HIP events.

The timed call runs the kernels of the untimed one, so its y and final state must equal
ssd_prefill's bit for bit.  It reports the launches the prefill makes (the kernels bench.py
expects for the shape, in order), each with a positive duration and a non-negative gap to
the next; launches past the events given run untimed and are still counted.
"""
from __future__ import annotations

import numpy as np
import pytest

import bench
from mamba_ssd_scan_amd import ssd, synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


# (B, L, H, P, N, G, Q)
CASES = [
    (1, 4 * 256 - 30, 8, 64, 128, 1, 256),   # 32 items: two launches, Step-3 inside the scan
    (1, 24 * 256 + 7, 24, 64, 128, 1, 256),  # 600 items: three launches, the pipelined scan
    (2, 700, 6, 64, 64, 2, 64),              # 64-token chunks: the one-head first launch, persistent scan
    (1, 500, 4, 48, 80, 1, 64),              # unbuilt sizes: padding copies around the prefill
]


def _expected(B, L, H, P, N, G, Q):
    """The kernels of the prefill's own launches, or None where padding adds copies."""
    if P not in (32, 64, 128) or N not in (32, 64, 128, 256):
        return None
    return bench.step_kernels(synth.PrefillShape(B, L, H, P, N, G, Q, "bf16"))


@pytest.mark.parametrize("B,L,H,P,N,G,Q", CASES)
def test_timed_prefill_is_the_prefill(B, L, H, P, N, G, Q):
    torch = gh.torch()
    print(f"[timed] B={B} L={L} H={H} P={P} N={N} G={G} Q={Q}", flush=True)
    rng = np.random.Generator(np.random.PCG64(9100 + L))
    g = gh.upload(synth.random_prefill(rng, B, L, H, P, N, G, "bf16", dt_mode="weak"))
    ws = ssd.alloc_workspace(B, L, H, P, N, G, Q)
    y0, f0 = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q, workspace=ws)
    ev = ssd.LaunchEvents(16)
    y1, f1, n = ssd.prefill_timed(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], events=ev, chunk=Q,
                                  workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    assert n == len(ev.names) and 1 <= n <= 16
    want = _expected(B, L, H, P, N, G, Q)
    if want is not None:
        assert ev.names == want
    else:
        assert "pad_copy_kernel" in ev.names and n > 3
    dur = ev.durations_ms()
    assert all(0.0 < d < 1000.0 for d in dur), dur
    assert all(-1e-3 <= gap < 1000.0 for gap in ev.gaps_ms()), ev.gaps_ms()
    print(f"[timed] launches {list(zip(ev.names, [round(d * 1e3, 1) for d in dur]))}", flush=True)

    # fewer event pairs than launches: the first is timed, the others run and are counted
    one = ssd.LaunchEvents(1)
    y2, f2, n2 = ssd.prefill_timed(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], events=one, chunk=Q,
                                   workspace=ws)
    torch.cuda.synchronize()
    assert n2 == n and one.names == ev.names[:1]
    assert torch.equal(y0, y2) and torch.equal(f0, f2)


def test_timed_prefill_with_options_and_bf16_y():
    """The z gate, softplus dt with a bias and a bf16 y: the same bits as prefill_ex."""
    torch = gh.torch()
    B, L, H, P, N, G, Q = 1, 3000, 8, 64, 128, 2, 256
    rng = np.random.Generator(np.random.PCG64(9200))
    g = gh.upload(synth.random_prefill(rng, B, L, H, P, N, G, "bf16", dt_mode="softplus"))
    z = torch.randn((B, L, H, P), device="cuda").to(torch.bfloat16)
    bias = torch.linspace(-1.0, 0.5, H, device="cuda")
    kw = dict(dt_bias=bias, dt_softplus=True, z=z, y_dtype=torch.bfloat16, chunk=Q)
    y0, f0 = ssd.prefill_ex(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], **kw)
    ev = ssd.LaunchEvents(4)
    y1, f1, n = ssd.prefill_timed(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], events=ev, **kw)
    torch.cuda.synchronize()
    assert y1.dtype == torch.bfloat16
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    assert n == len(ev.names) >= 2
