"""GPU parity tests of head and state dimensions beyond the built sizes.

The prefill and the decode step take any P and N that are multiples of 16 up to 256.  N = 256
runs natively in the staged kernels; other sizes run padded to the next built size (zero
channels and zero state columns, which add exact zeros to every sum), and P over 128 as two
heads of half the channels.  Every case is checked against the fp64 oracle: y with the
configured D, y with D = 0 and the final state, within the bar of the input type.
"""
from __future__ import annotations

import numpy as np
import pytest

from mamba_ssd_scan_amd import ssd, synth
from oracle import gated, ref
from tests import gpu_helpers as gh
from tests.util import TOL, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


# (P, N, Q, dtype, B, L, H, G)
PREFILL = [
    (16, 16, 64, "bf16", 2, 300, 4, 2),       # both padded to 32
    (16, 128, 256, "bf16", 1, 700, 6, 1),     # P padded to 32 (Q = 256 at P = 32: the staged kernels)
    (48, 80, 128, "bf16", 2, 515, 4, 2),      # both padded (64, 128)
    (64, 256, 256, "bf16", 1, 1100, 8, 1),    # N = 256 natively (staged kernels)
    (128, 256, 64, "bf16", 1, 640, 4, 2),     # P = 128, N = 256 natively
    (96, 48, 64, "f32", 2, 333, 4, 1),        # fp32 padded (128, 64)
    (32, 256, 128, "f32", 1, 400, 4, 4),      # fp32, N = 256 natively
    (144, 64, 64, "bf16", 1, 400, 4, 2),      # P over 128: two heads of 128 (padded from 144 to 256)
    (256, 32, 256, "bf16", 2, 300, 3, 1),     # P = 256: two heads of 128, no padding
    (256, 256, 128, "f32", 1, 200, 2, 1),     # the largest: split heads, N = 256
]


@pytest.mark.parametrize("P,N,Q,dtype,B,L,H,G", PREFILL)
def test_prefill_any_multiple_of_16(P, N, Q, dtype, B, L, H, G):
    ci = PREFILL.index((P, N, Q, dtype, B, L, H, G))
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(5000 + ci)), B, L, H, P, N, G, dtype,
                               init_state=True, dt_mode="weak" if ci % 2 else "softplus")
    print(f"[shapes] prefill P={P} N={N} Q={Q} {dtype} B={B} L={L} H={H} G={G}", flush=True)
    gh.check_prefill(inp, Q, label=f"P={P} N={N}")


def test_prefill_options_and_strides_through_the_padded_route():
    """P = 144 (split heads, padded): dt = softplus(dt + bias), the z gate and a bf16 y against the
    oracle of the options, and x, B, C read from wider rows equal the dense call bit for bit."""
    torch = gh.torch()
    B, L, H, P, N, G, Q = 2, 450, 4, 144, 48, 2, 128
    rng = np.random.Generator(np.random.PCG64(5100))
    inp = synth.random_prefill(rng, B, L, H, P, N, G, "bf16", init_state=True)
    opt = synth.option_inputs(rng, inp)
    g = gh.upload(inp)
    dtr = synth.to_torch(opt["dt_raw"], "bf16")
    z = synth.to_torch(opt["z"], "bf16")
    bias = torch.from_numpy(np.ascontiguousarray(opt["dt_bias"], np.float32)).cuda()
    y, fin = ssd.prefill_ex(g["x"], dtr, g["A"], g["B"], g["C"], g["D"], g["h0"], dt_bias=bias, dt_softplus=True,
                            z=z, y_dtype=torch.bfloat16, chunk=Q)
    torch.cuda.synchronize()
    yo, ho = gated.prefill(inp["x"], opt["dt_raw"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                           dt_bias=opt["dt_bias"], dt_softplus=True, z=opt["z"])
    ey, es = rel_err(y.float().cpu().numpy(), yo), rel_err(fin.cpu().numpy(), ho)
    print(f"[shapes] options P={P} N={N}: y={ey:.2e} state={es:.2e}", flush=True)
    assert ey < TOL["bf16"] + 2.0 ** -8 and es < TOL["bf16"]
    # strided: x, B, C inside one [x | B | C] row per token, dt inside a wider row
    hp, gn = H * P, G * N
    xbc = torch.zeros((B, L, hp + 2 * gn + 8), dtype=torch.bfloat16, device="cuda")
    xbc[..., :hp] = g["x"].reshape(B, L, hp)
    xbc[..., hp:hp + gn] = g["B"].reshape(B, L, gn)
    xbc[..., hp + gn:hp + 2 * gn] = g["C"].reshape(B, L, gn)
    dtw = torch.zeros((B, L, H + 3), dtype=torch.bfloat16, device="cuda")
    dtw[..., :H] = g["dt"]
    ys, fs = ssd.prefill(xbc[..., :hp].view(B, L, H, P), dtw[..., :H], g["A"], xbc[..., hp:hp + gn].view(B, L, G, N),
                         xbc[..., hp + gn:hp + 2 * gn].view(B, L, G, N), g["D"], g["h0"], chunk=Q)
    yd, fd = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q)
    torch.cuda.synchronize()
    assert torch.equal(ys, yd) and torch.equal(fs, fd)


# (P, N, dtype, B, H, G, steps)
STEP = [(16, 16, "bf16", 3, 4, 2, 5), (48, 80, "bf16", 2, 6, 3, 4), (64, 256, "bf16", 2, 4, 1, 3),
        (144, 48, "f32", 2, 2, 1, 3), (256, 256, "f32", 1, 2, 2, 2), (128, 128, "bf16", 4, 8, 1, 3)]


@pytest.mark.parametrize("P,N,dtype,B,H,G,steps", STEP)
def test_step_any_multiple_of_16(P, N, dtype, B, H, G, steps):
    torch = gh.torch()
    ci = STEP.index((P, N, dtype, B, H, G, steps))
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(5200 + ci)), B, steps, H, P, N, G, dtype,
                               init_state=True)
    g = gh.upload(inp)
    state = g["h0"].clone()
    so = np.array(inp["h0"], np.float64)
    print(f"[shapes] step P={P} N={N} {dtype} B={B} H={H} G={G}", flush=True)
    for t in range(steps):
        y = ssd.step(state, g["x"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"], g["B"][:, t].contiguous(),
                     g["C"][:, t].contiguous(), g["D"])
        torch.cuda.synchronize()
        yo = ref.step(so, inp["x"][:, t], inp["dt"][:, t], inp["A"], inp["B"][:, t], inp["C"][:, t], inp["D"])
        ey, es = rel_err(y.cpu().numpy(), yo), rel_err(state.cpu().numpy(), so)
        assert ey < TOL[dtype] and es < TOL[dtype], (t, ey, es)
    print(f"    last token: y={ey:.2e} state={es:.2e}", flush=True)
