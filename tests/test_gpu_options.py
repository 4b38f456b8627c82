"""GPU parity of the option entry points (ssd_prefill_ex, ssd_step_ex) against the
fp64 oracle of the options (oracle/gated.py).

Bars: y and the final state within the input dtype's tolerance (2e-3 bf16, 1e-4 fp32)
with fp32 y.  bf16 y adds its own rounding: bf16 keeps 8 significant bits, so
rounding to nearest costs at most half an ulp, 2^-8 of the element and so of max|y|.
Its bar is the fp32-y bar plus 2^-8, and its bits must equal the
round-to-nearest-even of the fp32-y result of the same call.
"""
from __future__ import annotations

import numpy as np
import pytest

from mamba_ssd_scan_amd import ssd, synth
from oracle import gated
from tests import gpu_helpers as gh
from tests.util import TOL, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


def _case(dtype, B=2, L=700, H=4, P=64, N=128, G=1, seed=21):
    rng = np.random.Generator(np.random.PCG64(seed))
    inp = synth.random_prefill(rng, B, L, H, P, N, G, dtype)
    opt = synth.option_inputs(rng, inp)
    return inp, opt


def _upload(inp, opt):
    torch = gh.torch()
    g = gh.upload(inp)
    d = inp["dtype"]
    g["dt_raw"] = synth.to_torch(opt["dt_raw"], d)
    g["z"] = synth.to_torch(opt["z"], d)
    g["dt_bias"] = torch.from_numpy(opt["dt_bias"]).cuda()
    return g


def _expect_pipelined(B, L, H, P, N, G, Q):
    """The shape has more items than two per CU: the pipelined chunk scan takes it."""
    import bench
    kernels = bench.step_kernels(synth.PrefillShape(B, L, H, P, N, G, Q, "bf16"))
    assert "chunk_scan_pipe_kernel" in kernels, kernels


@pytest.mark.parametrize("dtype,Q,L,P,N,G,H", [("bf16", 256, 700, 64, 128, 1, 4), ("bf16", 64, 333, 32, 64, 2, 4),
                                               ("f32", 64, 300, 64, 64, 1, 4), ("bf16", 128, 129, 128, 32, 4, 4),
                                               ("bf16", 256, 2100, 64, 128, 4, 40)])
def test_prefill_ex_softplus_gate(dtype, Q, L, P, N, G, H):
    torch = gh.torch()
    inp, opt = _case(dtype, L=L, P=P, N=N, G=G, H=H)
    if H == 40:
        _expect_pipelined(2, L, H, P, N, G, Q)
    g = _upload(inp, opt)
    y, hT = ssd.prefill_ex(g["x"], g["dt_raw"], g["A"], g["B"], g["C"], g["D"], g["h0"], dt_bias=g["dt_bias"],
                           dt_softplus=True, z=g["z"], chunk=Q)
    y0, _ = ssd.prefill_ex(g["x"], g["dt_raw"], g["A"], g["B"], g["C"], None, g["h0"], dt_bias=g["dt_bias"],
                           dt_softplus=True, z=g["z"], chunk=Q)
    torch.cuda.synchronize()
    kw = dict(dt_bias=opt["dt_bias"], dt_softplus=True, z=opt["z"])
    yo, ho = gated.prefill(inp["x"], opt["dt_raw"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], **kw)
    yo0, _ = gated.prefill(inp["x"], opt["dt_raw"], inp["A"], inp["B"], inp["C"], None, inp["h0"], **kw)
    e = dict(y=rel_err(y.cpu().numpy(), yo), y_D0=rel_err(y0.cpu().numpy(), yo0), state=rel_err(hT.cpu().numpy(), ho))
    print(f"[prefill_ex] {dtype} Q={Q} L={L} P={P} N={N} G={G} " + " ".join(f"{k}={v:.2e}" for k, v in e.items()),
          flush=True)
    assert all(np.isfinite(v) and v < TOL[dtype] for v in e.values()), e


@pytest.mark.parametrize("dtype,Q,L,H,G", [("bf16", 256, 611, 4, 1), ("bf16", 64, 611, 4, 1), ("f32", 128, 611, 4, 1),
                                         ("bf16", 256, 2100, 40, 4)])
def test_prefill_ex_bf16_output(dtype, Q, L, H, G):
    torch = gh.torch()
    inp, opt = _case(dtype, L=L, H=H, G=G, seed=22)
    if H == 40:
        _expect_pipelined(2, L, H, 64, 128, G, Q)
    g = _upload(inp, opt)
    for z in (None, g["z"]):
        y32, _ = ssd.prefill_ex(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], z=z, chunk=Q)
        y16, _ = ssd.prefill_ex(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], z=z, chunk=Q,
                                y_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        a32 = y32.cpu().numpy()
        bits = y16.cpu().view(torch.int16).numpy().view(np.uint16)
        # the stored bits are the round-to-nearest-even of the same call's fp32 result
        assert np.array_equal(bits, synth.bf16_bits(synth.bf16_round(a32))), "bf16 y is not the RNE of the fp32 y"
        yo, _ = gated.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"],
                              z=None if z is None else opt["z"])
        e = rel_err(y16.float().cpu().numpy(), yo)
        print(f"[prefill_ex bf16 y] {dtype} Q={Q} L={L} H={H} G={G} gate={z is not None} err={e:.2e}", flush=True)
        assert e < TOL[dtype] + 2.0 ** -8


@pytest.mark.parametrize("dtype,y16", [("bf16", False), ("bf16", True), ("f32", False)])
def test_step_ex_matches_oracle(dtype, y16):
    torch = gh.torch()
    B, H, P, N, G, S = 3, 8, 64, 128, 2, 10
    rng = np.random.Generator(np.random.PCG64(23))
    inp = synth.random_prefill(rng, B, S, H, P, N, G, dtype)
    opt = synth.option_inputs(rng, inp)
    g = _upload(inp, opt)
    st = g["h0"].clone()
    st_o = np.array(inp["h0"], np.float64)
    worst = 0.0
    for t in range(S):
        y = ssd.step_ex(st, g["x"][:, t].contiguous(), g["dt_raw"][:, t].contiguous(), g["A"],
                        g["B"][:, t].contiguous(), g["C"][:, t].contiguous(), g["D"], dt_bias=g["dt_bias"],
                        dt_softplus=True, z=g["z"][:, t].contiguous(), y_dtype=torch.bfloat16 if y16 else None)
        yo = gated.step(st_o, inp["x"][:, t], opt["dt_raw"][:, t], inp["A"], inp["B"][:, t], inp["C"][:, t], inp["D"],
                        dt_bias=opt["dt_bias"], dt_softplus=True, z=opt["z"][:, t])
        torch.cuda.synchronize()
        worst = max(worst, rel_err(y.float().cpu().numpy(), yo))
    es = rel_err(st.cpu().numpy(), st_o)
    print(f"[step_ex] {dtype} bf16_y={y16} y={worst:.2e} state={es:.2e}", flush=True)
    assert worst < TOL[dtype] + (2.0 ** -8 if y16 else 0.0) and es < TOL[dtype]
