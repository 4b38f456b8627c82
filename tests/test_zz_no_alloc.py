"""GPU test of ssd_prefill_noalloc (the prefill with the library's own scratch) against
ssd_prefill: bit for bit on two calls in a row, the second on a smaller problem, and the
refusal of a problem whose scratch exceeds the library's array."""
from __future__ import annotations

import numpy as np
import pytest

from mamba_ssd_scan_amd import ssd, synth
from tests import gpu_helpers as gh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


def _both(inp, Q):
    torch = gh.torch()
    g = gh.upload(inp)
    B, L, H, P = g["x"].shape
    N = g["B"].shape[3]
    y = torch.full((B, L, H, P), float("nan"), dtype=torch.float32, device="cuda")
    fin = torch.full((B, H, P, N), float("nan"), dtype=torch.float32, device="cuda")
    ssd.prefill_noalloc(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q, y=y, final_state=fin)
    yr, fr = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q)
    torch.cuda.synchronize()
    return y, fin, yr, fr


def test_noalloc_equals_prefill_on_two_calls():
    """The 130M-shaped layer (scratch about 16 MB), then a smaller ragged problem with two
    groups and N = 64 on the same array: each equals ssd_prefill bit for bit."""
    s1 = synth.WORKLOADS[1]
    print("[noalloc] call 1: 130M layer, 4096 tokens", flush=True)
    y, fin, yr, fr = _both(synth.prefill_inputs(s1, synth.SEED_BASE + 1), s1.chunk)
    assert bool((y == yr).all()) and bool((fin == fr).all())
    print("[noalloc] call 2: B=2 L=1000 H=8 N=64 G=2", flush=True)
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(4100)), 2, 1000, 8, 64, 64, 2, "bf16",
                               init_state=True, dt_mode="weak")
    y, fin, yr, fr = _both(inp, 128)
    assert bool((y == yr).all()) and bool((fin == fr).all())


def test_noalloc_refuses_a_problem_beyond_its_array():
    torch = gh.torch()
    B, L, H, P, N, G, Q = 1, 16384, 80, 64, 128, 1, 256  # the 2.7B layer: far more scratch than 64 MiB
    assert ssd.workspace_size(B, L, H, P, N, G, Q) > ssd.NOALLOC_MAX_BYTES
    x = torch.zeros((B, L, H, P), dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros((B, L, H), dtype=torch.bfloat16, device="cuda")
    Bm = torch.zeros((B, L, G, N), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros(H, dtype=torch.float32, device="cuda")
    y = torch.zeros((B, L, H, P), dtype=torch.float32, device="cuda")
    with pytest.raises(ssd.SsdError) as e:
        ssd.prefill_noalloc(x, dt, A, Bm, Bm, None, None, chunk=Q, y=y)
    assert e.value.status == ssd.SSD_ERR_WORKSPACE
