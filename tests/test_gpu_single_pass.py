"""GPU tests of the single-pass prefill (grids of many rounds) against the fp64 oracle.

The single-pass path forms every chunk's state, hands the entering states from chunk to
chunk through device memory (a look-back over the previous chunks' published states) and
writes y in one launch after a GEMM1 launch.  Its chunk and entering states stay fp32, so
it is checked against the oracle (y with the configured D, y with D = 0, the final state,
bar 2e-3 for bf16 inputs), not bit for bit against the other paths.  Every case that can
runs twice on one workspace with new inputs: the ticket counter and the status words must
start from zero on every call.  The give-up report is forced from the host (a wait bound of
zero polls), so every kernel still ends normally.
"""
from __future__ import annotations

import numpy as np
import pytest

from mamba_ssd_scan_amd import ssd, synth
from oracle import gated
from tests import gpu_helpers as gh
from tests.util import TOL, rel_err

pytestmark = pytest.mark.gpu

Q = 256
SP = ssd.PATH_SINGLE_PASS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


def _sub(inp, heads, H, G):
    """The problem restricted to some heads (each keeping its own group of B and C)."""
    sub = dict(inp)
    for k in ("x", "dt"):
        sub[k] = np.ascontiguousarray(inp[k][:, :, heads])
    sub["A"], sub["D"] = inp["A"][heads], inp["D"][heads]
    sub["h0"] = None if inp["h0"] is None else np.ascontiguousarray(inp["h0"][:, heads])
    grp = [h // (H // G) for h in heads]
    sub["B"], sub["C"] = np.ascontiguousarray(inp["B"][:, :, grp]), np.ascontiguousarray(inp["C"][:, :, grp])
    return sub


def _check_heads(inp, y, y0, fin, heads, H, G, tol, label):
    """y, y(D = 0) and the final state of the given heads against the oracle."""
    sub = _sub(inp, heads, H, G)
    yo, ho = gh.oracle_prefill(sub)
    yo0, _ = gh.oracle_prefill(sub, D=None)
    errs = dict(y=rel_err(y.cpu().numpy()[:, :, heads], yo), y_D0=rel_err(y0.cpu().numpy()[:, :, heads], yo0))
    if fin is not None:
        errs["state"] = rel_err(fin.cpu().numpy()[:, heads], ho)
    print(f"[single pass] {label} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert np.isfinite(v) and v < tol, (label, k, v)
    return errs


def _run(g, ws, *, path=SP, D="use", final=True, spin_limit=None):
    return ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"] if D == "use" else D, g["h0"], chunk=Q,
                       final_state="new" if final else None, workspace=ws, path=path, spin_limit=spin_limit)


# (B, L, H, N, G, initial state, final state, dt mode)
CASES = [
    (1, 256, 4, 128, 1, True, True, "softplus"),        # one chunk: no exchange at all
    (1, 2 * 256 + 17, 6, 64, 2, True, True, "weak"),    # 3 chunks, ragged, two groups
    (2, 9 * 256 - 3, 8, 128, 1, False, True, "weak"),   # 9 chunks, no initial state
    (3, 5 * 256, 10, 64, 5, True, False, "softplus"),   # no final state, five groups
    (1, 40 * 256 + 100, 12, 128, 3, True, True, "weak"),  # 41 chunks: long chains, ragged
    (4, 1100, 20, 128, 4, True, True, "strong"),        # decays underflow to zero
    (2, 17 * 256, 24, 128, 1, True, True, "weak"),      # 816 items: several rounds
]


@pytest.mark.parametrize("B,L,H,N,G,init,final,mode", CASES)
def test_single_pass_matches_oracle(B, L, H, N, G, init, final, mode):
    torch = gh.torch()
    ws = ssd.alloc_workspace(B, L, H, 64, N, G, Q)
    ci = CASES.index((B, L, H, N, G, init, final, mode))
    for call in range(2):
        inp = synth.random_prefill(np.random.Generator(np.random.PCG64(3100 + 10 * ci + call)), B, L, H, 64, N, G,
                                   "bf16", init_state=init, dt_mode=mode)
        print(f"[single pass] B={B} L={L} H={H} N={N} G={G} init={init} final={final} {mode} call {call}",
              flush=True)
        g = gh.upload(inp)
        y, fin = _run(g, ws, final=final)
        assert ssd.prefill_check(ws) == ssd.SSD_OK
        y0, _ = _run(g, ws, D=None, final=final)
        assert ssd.prefill_check(ws) == ssd.SSD_OK
        torch.cuda.synchronize()
        if not final:
            assert fin is None
        heads = list(range(H)) if B * L * H <= 300000 else [0, H // 3, H - 1]
        _check_heads(inp, y, y0, fin, heads, H, G, TOL["bf16"], f"B={B} L={L} H={H} N={N} call {call}")


def test_full_size_2p7b_layer():
    """The 2.7B-shaped layer at 16384 tokens (64 chunks x 80 heads, random initial state) on the
    single pass and on the library's own path (three launches for this shape), both against the
    oracle on sampled heads."""
    torch = gh.torch()
    s = synth.WORKLOADS[3]
    inp = synth.prefill_inputs(s, synth.SEED_BASE + 3)
    g = gh.upload(inp)
    ws = ssd.alloc_workspace(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk)
    for path in (SP, ssd.PATH_AUTO):
        y, fin = _run(g, ws, path=path)
        assert ssd.prefill_check(ws) == ssd.SSD_OK
        y0, _ = _run(g, ws, path=path, D=None)
        torch.cuda.synchronize()
        _check_heads(inp, y, y0, fin, [0, 37, 79], s.nheads, s.ngroups, TOL["bf16"], f"2.7B L=16384 path {path}")


@pytest.mark.parametrize("path", [SP, ssd.PATH_STAGED])
def test_long_weak_decay_stress(path):
    """64 chunks with a long memory (dt ~ U(0, 0.02), A in [-0.05, 0]) and a random initial
    state, the regime where the rounding of every chunk's state carries furthest: the single
    pass (fp32 states between chunks) and the three-launch path (fp16 chunk and entering
    states) both within the bf16 bar of the oracle on sampled heads."""
    torch = gh.torch()
    B, L, H, N, G = 1, 16384, 80, 128, 1
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(3300)), B, L, H, 64, N, G, "bf16",
                               init_state=True, dt_mode="weak")
    g = gh.upload(inp)
    ws = ssd.alloc_workspace(B, L, H, 64, N, G, Q)
    y, fin = _run(g, ws, path=path)
    y0, _ = _run(g, ws, path=path, D=None)
    torch.cuda.synchronize()
    _check_heads(inp, y, y0, fin, [0, 41, 79], H, G, TOL["bf16"], f"weak decay L=16384 path {path}")


def test_give_up_is_reported():
    """A wait bound of zero polls makes every wait between workgroups give up at once: the
    launch still ends, and ssd_prefill_check reports SSD_ERR_SYNC; the next call on the same
    workspace clears the report.  The same for the one-round path; the three-launch path has no
    such waits."""
    torch = gh.torch()
    B, L, H, N, G = 1, 8 * 256, 8, 128, 1
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(3400)), B, L, H, 64, N, G, "bf16",
                               dt_mode="weak")
    g = gh.upload(inp)
    ws = ssd.alloc_workspace(B, L, H, 64, N, G, Q)
    print("[give up] single pass, zero polls", flush=True)
    _run(g, ws, spin_limit=0)
    assert ssd.prefill_check(ws) == ssd.SSD_ERR_SYNC
    y, fin = _run(g, ws)
    assert ssd.prefill_check(ws) == ssd.SSD_OK
    y0, _ = _run(g, ws, D=None)
    assert ssd.prefill_check(ws) == ssd.SSD_OK
    _check_heads(inp, y, y0, fin, list(range(H)), H, G, TOL["bf16"], "after a give-up")

    # one-round path (the 130M-shaped layer fits it on a 256-CU device)
    s1 = synth.WORKLOADS[1]
    inp1 = synth.prefill_inputs(s1, synth.SEED_BASE + 1)
    g1 = gh.upload(inp1)
    ws1 = ssd.alloc_workspace(s1.batch, s1.seqlen, s1.nheads, s1.headdim, s1.dstate, s1.ngroups, s1.chunk)
    try:
        print("[give up] one-round path, zero polls", flush=True)
        _run(g1, ws1, path=ssd.PATH_ONE_ROUND, spin_limit=0)
    except ssd.SsdError as e:
        assert e.status == ssd.SSD_ERR_UNSUPPORTED
        pytest.skip("the one-round path does not apply on this device")
    assert ssd.prefill_check(ws1) == ssd.SSD_ERR_SYNC
    _run(g1, ws1, path=ssd.PATH_ONE_ROUND)
    assert ssd.prefill_check(ws1) == ssd.SSD_OK
    _run(g1, ws1, path=ssd.PATH_ONE_ROUND, spin_limit=0)
    _run(g1, ws1, path=ssd.PATH_STAGED, spin_limit=0)  # no waits: the report is clear
    assert ssd.prefill_check(ws1) == ssd.SSD_OK
    torch.cuda.synchronize()


@pytest.mark.parametrize("y16", [False, True])
def test_single_pass_options(y16):
    """dt = softplus(dt + bias), the z gate and (y16) a bf16 y on the single pass, against the
    fp64 oracle of the options."""
    torch = gh.torch()
    B, L, H, N, G = 2, 6 * 256 + 40, 8, 128, 2
    rng = np.random.Generator(np.random.PCG64(3500 + y16))
    inp = synth.random_prefill(rng, B, L, H, 64, N, G, "bf16", init_state=True)
    opt = synth.option_inputs(rng, inp)
    g = gh.upload(inp)
    dtr = synth.to_torch(opt["dt_raw"], "bf16")
    z = synth.to_torch(opt["z"], "bf16")
    bias = torch.from_numpy(np.ascontiguousarray(opt["dt_bias"], np.float32)).cuda()
    ws = ssd.alloc_workspace(B, L, H, 64, N, G, Q)
    yd = torch.bfloat16 if y16 else torch.float32
    kw = dict(dt_bias=bias, dt_softplus=True, z=z, y_dtype=yd, chunk=Q, workspace=ws, path=SP)
    y, fin = ssd.prefill_ex(g["x"], dtr, g["A"], g["B"], g["C"], g["D"], g["h0"], **kw)
    assert ssd.prefill_check(ws) == ssd.SSD_OK
    torch.cuda.synchronize()
    ok = dict(dt_bias=opt["dt_bias"], dt_softplus=True, z=opt["z"])
    yo, ho = gated.prefill(inp["x"], opt["dt_raw"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], **ok)
    tol = TOL["bf16"] + (2.0 ** -8 if y16 else 0.0)
    ey, es = rel_err(y.float().cpu().numpy(), yo), rel_err(fin.cpu().numpy(), ho)
    print(f"[single pass options] y16={y16} y={ey:.2e} state={es:.2e}", flush=True)
    assert ey < tol and es < TOL["bf16"]
    if y16:
        # bf16 y is the round-to-nearest-even of the same kernel's fp32 y
        y32, _ = ssd.prefill_ex(g["x"], dtr, g["A"], g["B"], g["C"], g["D"], g["h0"],
                                **dict(kw, y_dtype=torch.float32))
        torch.cuda.synchronize()
        assert torch.equal(y, y32.to(torch.bfloat16))


def test_single_pass_strided_inputs():
    """x, B and C read in place from a layer's [x | B | C] rows and dt from wider rows give the
    dense single pass's result bit for bit."""
    torch = gh.torch()
    B, L, H, N, G = 1, 7 * 256 + 5, 8, 128, 1
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(3600)), B, L, H, 64, N, G, "bf16")
    g = gh.upload(inp)
    hp, gn = H * 64, G * N
    xbc = torch.zeros((B, L, hp + 2 * gn + 8), dtype=torch.bfloat16, device="cuda")
    xbc[..., :hp] = g["x"].reshape(B, L, hp)
    xbc[..., hp:hp + gn] = g["B"].reshape(B, L, gn)
    xbc[..., hp + gn:hp + 2 * gn] = g["C"].reshape(B, L, gn)
    dtw = torch.zeros((B, L, H + 5), dtype=torch.bfloat16, device="cuda")
    dtw[..., :H] = g["dt"]
    xv = xbc[..., :hp].view(B, L, H, 64)
    bv = xbc[..., hp:hp + gn].view(B, L, G, N)
    cv = xbc[..., hp + gn:hp + 2 * gn].view(B, L, G, N)
    ws = ssd.alloc_workspace(B, L, H, 64, N, G, Q)
    y, fin = ssd.prefill(xv, dtw[..., :H], g["A"], bv, cv, g["D"], g["h0"], chunk=Q, workspace=ws, path=SP)
    yd, find = _run(g, ws)
    torch.cuda.synchronize()
    assert torch.equal(y, yd) and torch.equal(fin, find)


def test_single_pass_in_a_callers_graph():
    """The single pass captured by a caller's graph: its counters are cleared by its first
    launch (no memset), so every replay starts from zero.  Inputs are rewritten between
    replays, with eager work and synchronisations in between; every replay equals an eager
    call bit for bit."""
    torch = gh.torch()
    B, L, H, N, G = 1, 12 * 256, 16, 128, 1
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(3700)), B, L, H, 64, N, G, "bf16")
    g = gh.upload(inp)
    ws = ssd.alloc_workspace(B, L, H, 64, N, G, Q)
    y = torch.empty((B, L, H, 64), dtype=torch.float32, device="cuda")
    fin = torch.empty((B, H, 64, N), dtype=torch.float32, device="cuda")
    run = lambda: ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q, y=y,
                              final_state=fin, workspace=ws, path=SP)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        print(f"[single pass graph] replay {r}", flush=True)
        new = synth.random_prefill(np.random.Generator(np.random.PCG64(3701 + r)), B, L, H, 64, N, G, "bf16")
        nd = gh.upload(new)
        for k in ("x", "dt", "B", "C", "A", "D", "h0"):
            g[k].copy_(nd[k])
        graph.replay()
        torch.cuda.synchronize()
        yg, fg = y.clone(), fin.clone()
        ye, fe = ssd.prefill(nd["x"], nd["dt"], nd["A"], nd["B"], nd["C"], nd["D"], nd["h0"], chunk=Q, path=SP)
        torch.cuda.synchronize()
        assert torch.equal(yg, ye) and torch.equal(fg, fe), f"replay {r} differs from the eager prefill"
        (torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")).sum().item()


def test_prefill_on_a_side_stream_keeps_its_workspace():
    """A prefill enqueued on a stream other than the current one, with the workspace and outputs
    allocated by the binding: the memory belongs to that stream, so work queued right after on
    the same stream cannot be handed the workspace while the kernels still use it.  The result
    equals a call on the current stream bit for bit."""
    torch = gh.torch()
    B, L, H, N, G = 1, 20 * 256, 24, 128, 1
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(3800)), B, L, H, 64, N, G, "bf16")
    g = gh.upload(inp)
    yref, fref = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    y, fin = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q, stream=side)
    with torch.cuda.stream(side):
        # allocations on the side stream right after the call, filled with garbage
        junk = [torch.full((1 << 22,), float("nan"), device="cuda") for _ in range(8)]
    side.synchronize()
    del junk
    assert torch.equal(y, yref) and torch.equal(fin, fref)
