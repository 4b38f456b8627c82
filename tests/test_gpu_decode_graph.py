"""GPU tests of the decode loop as a HIP graph.

- The library's own graph (ssd_decode_graph_*) against the eager ssd_step_ex
  loop on the same buffers: the same kernel on the same inputs, so the outputs
  and the state must be bitwise equal; and against the fp64 oracle's token loop.
- ssd_step captured by a caller's graph (torch.cuda.CUDAGraph): the entry point
  allocates nothing, synchronises nothing and records no memset, so it can sit
  inside a caller's captured decode step.

Every graph is replayed several times, with new inputs written into the
captured buffers and unrelated eager work and synchronisations between
replays; every replay is checked.
"""
from __future__ import annotations

import numpy as np
import pytest

from mamba_ssd_scan_amd import ssd, synth
from oracle import gated
from tests import gpu_helpers as gh
from tests.util import TOL, rel_err

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


def _inputs(shape, seed, opts):
    """Step-major decode inputs as device tensors, plus the host copies (fp32 values)."""
    torch = gh.torch()
    inp = synth.decode_inputs(shape, seed)
    d = shape.dtype
    dev = {k: synth.to_torch(inp[k], d) for k in ("x", "B", "C")}
    dev["A"] = torch.from_numpy(inp["A"]).cuda()
    dev["D"] = torch.from_numpy(inp["D"]).cuda()
    dev["state"] = torch.from_numpy(inp["state"]).cuda()
    if opts:
        rng = np.random.Generator(np.random.PCG64(seed + 1))
        raw = rng.normal(-3.0, 1.0, size=inp["dt"].shape).astype(np.float32)
        inp["dt"] = synth.bf16_round(raw) if d == "bf16" else raw
        inp["dt_bias"] = rng.normal(0.0, 0.5, size=(shape.nheads,)).astype(np.float32)
        z = rng.standard_normal(inp["x"].shape, dtype=np.float32)
        inp["z"] = synth.bf16_round(z) if d == "bf16" else z
        dev["dt_bias"] = torch.from_numpy(inp["dt_bias"]).cuda()
        dev["z"] = synth.to_torch(inp["z"], d)
    else:
        dev["dt_bias"] = dev["z"] = None
    dev["dt"] = synth.to_torch(inp["dt"], d)
    return inp, dev


def _rewrite(dev, inp, shape, seed, opts):
    """Overwrite the captured input buffers in place with a fresh draw."""
    new, nd = _inputs(shape, seed, opts)
    for k in ("x", "dt", "B", "C", "z", "state", "A", "D", "dt_bias"):
        if dev[k] is not None:
            dev[k].copy_(nd[k])
    return new


def _eager(dev, state, opts, y_dtype):
    ys = []
    for t in range(dev["x"].shape[0]):
        ys.append(ssd.step_ex(state, dev["x"][t], dev["dt"][t], dev["A"], dev["B"][t], dev["C"][t], dev["D"],
                              dt_bias=dev["dt_bias"], dt_softplus=opts,
                              z=None if dev["z"] is None else dev["z"][t], y_dtype=y_dtype))
    return gh.torch().stack(ys)


def _oracle(inp, opts):
    st = np.array(inp["state"], np.float64)
    ys = []
    for t in range(inp["x"].shape[0]):
        kw = dict(dt_bias=inp["dt_bias"], dt_softplus=True, z=inp["z"][t]) if opts else {}
        ys.append(gated.step(st, inp["x"][t], inp["dt"][t], inp["A"], inp["B"][t], inp["C"][t], inp["D"], **kw))
    return np.stack(ys), st


def _unrelated_work():
    torch = gh.torch()
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()  # eager kernels and a synchronisation between replays


@pytest.mark.parametrize("dtype,opts,y16,shape", [
    ("bf16", False, False, (4, 8, 64, 128, 2, 24)),
    ("f32", False, False, (2, 4, 32, 64, 1, 17)),
    ("bf16", True, True, (3, 6, 128, 32, 3, 9)),
])
def test_decode_graph_matches_eager_and_oracle(dtype, opts, y16, shape):
    torch = gh.torch()
    B, H, P, N, G, T = shape
    s = synth.DecodeShape(B, H, P, N, G, T, dtype)
    y_dtype = torch.bfloat16 if y16 else torch.float32
    inp, dev = _inputs(s, 300, opts)
    state_g = dev["state"].clone()
    g = ssd.DecodeGraph(state_g, dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dt_bias=dev["dt_bias"],
                        dt_softplus=opts, z=dev["z"], y_dtype=y_dtype)
    assert g.nsteps == T
    try:
        for r in range(REPLAYS):
            print(f"[decode graph] {dtype} opts={opts} bf16_y={y16} shape={shape} replay {r}", flush=True)
            if r:
                inp = _rewrite(dev, inp, s, 300 + r, opts)
            state_g.copy_(dev["state"])
            y_g = g.launch()
            torch.cuda.synchronize()
            yg, sg = y_g.clone(), state_g.clone()
            state_e = dev["state"].clone()
            y_e = _eager(dev, state_e, opts, y_dtype)
            torch.cuda.synchronize()
            assert torch.equal(yg.view(torch.int16) if y16 else yg, y_e.view(torch.int16) if y16 else y_e), \
                "graph replay differs from the eager loop"
            assert torch.equal(sg, state_e), "graph state differs from the eager loop"
            yo, so = _oracle(inp, opts)
            ey = rel_err(yg.float().cpu().numpy(), yo)
            es = rel_err(sg.cpu().numpy(), so)
            print(f"    y err {ey:.2e} state err {es:.2e}", flush=True)
            assert ey < TOL[dtype] + (2.0 ** -8 if y16 else 0.0) and es < TOL[dtype]
            _unrelated_work()
        # Two launches back to back continue the state: 2T tokens with the inputs repeated.
        state_g.copy_(dev["state"])
        g.launch()
        g.launch()
        torch.cuda.synchronize()
        state_e = dev["state"].clone()
        _eager(dev, state_e, opts, y_dtype)
        _eager(dev, state_e, opts, y_dtype)
        torch.cuda.synchronize()
        assert torch.equal(state_g, state_e)
    finally:
        g.close()


def test_step_inside_a_callers_graph():
    torch = gh.torch()
    B, H, P, N, G, T = 2, 8, 64, 128, 1, 16
    s = synth.DecodeShape(B, H, P, N, G, T, "bf16")
    inp, dev = _inputs(s, 310, False)
    state = dev["state"].clone()
    y = torch.empty((T, B, H, P), dtype=torch.float32, device="cuda")
    # warm the library and the stream before capture
    ssd.step(state.clone(), dev["x"][0], dev["dt"][0], dev["A"], dev["B"][0], dev["C"][0], dev["D"], y=y[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for t in range(T):
                ssd.step(state, dev["x"][t], dev["dt"][t], dev["A"], dev["B"][t], dev["C"][t], dev["D"], y=y[t])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        print(f"[caller graph] replay {r}", flush=True)
        if r:
            inp = _rewrite(dev, inp, s, 310 + r, False)
        state.copy_(dev["state"])
        graph.replay()
        torch.cuda.synchronize()
        yg, sg = y.clone(), state.clone()
        state_e = dev["state"].clone()
        y_e = _eager(dev, state_e, False, torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(yg, y_e) and torch.equal(sg, state_e)
        yo, so = _oracle(inp, False)
        assert rel_err(yg.cpu().numpy(), yo) < TOL["bf16"] and rel_err(sg.cpu().numpy(), so) < TOL["bf16"]
        _unrelated_work()
