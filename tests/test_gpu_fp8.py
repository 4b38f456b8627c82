"""GPU tests of fp8 e4m3 input storage (x, B and C as OCP e4m3 codes, dt and z bf16).

The inputs the oracle consumes are the exact e4m3 values (synth rounds the draws to e4m3 and
the GPU receives their codes), so the oracle comparison keeps the bf16 inputs' bar: every
matrix-core operand computed from the inputs is fp16, as with bf16 inputs.  Covered: each
prefill path and kernel family (two heads per chunk-state workgroup with the one-round and
the pipelined chunk scan, the one-head chunk state with the persistent scan, padded sizes),
the options, inputs read in place from wider rows, the forced paths, the decode step and
graph, the full 2.7B-shaped layer on sampled heads, and NaN codes.
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


def _rng(k):
    return np.random.Generator(np.random.PCG64(6100 + k))


# (B, L, H, P, N, G, Q, dt_mode): the kernels each shape takes, for fp8 as for bf16
CASES = [
    (1, 1000, 8, 64, 128, 1, 256, "weak"),       # two-head chunk state, one-round scan with Step-3
    (1, 24 * 256 + 7, 24, 64, 128, 1, 256, "weak"),  # 600 items: two-head chunk state, pipelined scan
    (2, 1000, 6, 64, 128, 3, 256, "softplus"),   # three groups (two heads each), ragged last chunk
    (2, 700, 6, 64, 64, 2, 64, "weak"),          # one-head chunk state, persistent scan
    (2, 333, 4, 128, 128, 2, 128, "strong"),     # P = 128, decays underflow
    (1, 500, 4, 48, 80, 1, 64, "softplus"),      # unbuilt sizes: padded copies (1-byte elements)
]


@pytest.mark.parametrize("B,L,H,P,N,G,Q,mode", CASES)
def test_fp8_prefill_matches_oracle(B, L, H, P, N, G, Q, mode):
    inp = synth.random_prefill(_rng(L + H), B, L, H, P, N, G, "fp8", dt_mode=mode)
    assert inp["x"].dtype == np.float32 and np.array_equal(synth.e4m3_round(inp["x"]), inp["x"])
    gh.check_prefill(inp, Q, label=f"fp8 B={B} L={L} H={H} P={P} N={N} G={G} Q={Q} {mode}")


def test_fp8_paths_agree_bit_for_bit():
    """A one-round shape: the library's path, the three launches and the one-head chunk state
    give the same bits; the single pass does not take fp8 inputs."""
    torch = gh.torch()
    inp = synth.random_prefill(_rng(1), 1, 1500, 8, 64, 128, 1, "fp8", dt_mode="weak")
    g = gh.upload(inp)
    outs = {}
    for path in (ssd.PATH_AUTO, ssd.PATH_STAGED, ssd.PATH_ONE_ROUND, ssd.PATH_STAGED_ONE_HEAD):
        try:
            outs[path] = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=256, path=path)
        except ssd.SsdError as e:
            assert path == ssd.PATH_ONE_ROUND and e.status == ssd.SSD_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    y0, f0 = outs[ssd.PATH_AUTO]
    for path, (y, f) in outs.items():
        assert torch.equal(y, y0) and torch.equal(f, f0), path
    with pytest.raises(ssd.SsdError, match="UNSUPPORTED"):
        ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=256, path=ssd.PATH_SINGLE_PASS)


@pytest.mark.parametrize("Q,N,y16,L,H,G", [(256, 128, False, 700, 4, 1), (64, 64, True, 700, 4, 1),
                                          # 720 items: the pipelined chunk scan with the gate and bf16 y
                                          (256, 128, True, 2100, 40, 4)])
def test_fp8_prefill_options(Q, N, y16, L, H, G):
    """dt = softplus(dt + bias) and the gate y * silu(z) with bf16 dt and z beside e4m3 x, B
    and C; bf16 y within the fp32-y bar plus its own rounding (2^-8)."""
    torch = gh.torch()
    rng = _rng(2 + Q)
    inp = synth.random_prefill(rng, 2, L, H, 64, N, G, "fp8")
    opt = synth.option_inputs(rng, inp)
    g = gh.upload(inp)
    dtr = synth.to_torch(opt["dt_raw"], "bf16")
    z = synth.to_torch(opt["z"], "bf16")
    bias = torch.from_numpy(opt["dt_bias"]).cuda()
    yd = torch.bfloat16 if y16 else torch.float32
    y, fin = ssd.prefill_ex(g["x"], dtr, g["A"], g["B"], g["C"], g["D"], g["h0"], dt_bias=bias, dt_softplus=True,
                            z=z, y_dtype=yd, chunk=Q)
    torch.cuda.synchronize()
    kw = dict(dt_bias=opt["dt_bias"], dt_softplus=True, z=opt["z"])
    yo, ho = gated.prefill(inp["x"], opt["dt_raw"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], **kw)
    ey, es = rel_err(y.float().cpu().numpy(), yo), rel_err(fin.cpu().numpy(), ho)
    print(f"[fp8 options] Q={Q} N={N} L={L} H={H} G={G} y16={y16} y={ey:.2e} state={es:.2e}", flush=True)
    assert ey < TOL["fp8"] + (2.0 ** -8 if y16 else 0.0) and es < TOL["fp8"]
    with pytest.raises(TypeError):  # dt beside e4m3 inputs is bf16
        ssd.prefill(g["x"], g["x"][..., 0].contiguous(), g["A"], g["B"], g["C"], chunk=Q)


def test_fp8_inputs_read_in_place_from_wider_rows():
    """x, B and C as views into one [x | B | C] row per token (e4m3), dt into another (bf16):
    the same bits as dense copies."""
    torch = gh.torch()
    B, L, H, P, N, G, Q = 2, 900, 4, 64, 128, 1, 256
    inp = synth.random_prefill(_rng(3), B, L, H, P, N, G, "fp8", dt_mode="weak")
    g = gh.upload(inp)
    hp, gn = H * P, G * N
    codes = torch.zeros((B, L, hp + 2 * gn + 16), dtype=torch.uint8, device="cuda")
    codes[..., :hp] = g["x"].view(torch.uint8).reshape(B, L, hp)
    codes[..., hp:hp + gn] = g["B"].view(torch.uint8).reshape(B, L, gn)
    codes[..., hp + gn:hp + 2 * gn] = g["C"].view(torch.uint8).reshape(B, L, gn)
    rows = codes.view(torch.float8_e4m3fn)
    drows = torch.zeros((B, L, H + 5), dtype=torch.bfloat16, device="cuda")
    drows[..., 2:2 + H] = g["dt"]
    xv = rows[..., :hp].unflatten(-1, (H, P))
    bv = rows[..., hp:hp + gn].unflatten(-1, (G, N))
    cv = rows[..., hp + gn:hp + 2 * gn].unflatten(-1, (G, N))
    dv = drows[..., 2:2 + H]
    y1, f1 = ssd.prefill(xv, dv, g["A"], bv, cv, g["D"], g["h0"], chunk=Q)
    y0, f0 = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


def test_fp8_decode_step_and_graph():
    """Decode tokens with e4m3 x, B and C against the oracle, eager and as one decode graph."""
    torch = gh.torch()
    s = synth.DecodeShape(3, 6, 64, 128, 2, 12, "fp8")
    inp = synth.decode_inputs(s, 6200)
    xs, Bs, Cs = (synth.to_torch(inp[k], "fp8") for k in ("x", "B", "C"))
    dts = synth.to_torch(inp["dt"], "bf16")
    A, D = torch.from_numpy(inp["A"]).cuda(), torch.from_numpy(inp["D"]).cuda()
    st = torch.from_numpy(inp["state"]).cuda()
    st_g = st.clone()
    st_o = inp["state"].astype(np.float64).copy()
    worst = 0.0
    ys = []
    for t in range(s.steps):
        y = ssd.step(st, xs[t], dts[t], A, Bs[t], Cs[t], D)
        yo = ref.step(st_o, inp["x"][t], inp["dt"][t], inp["A"], inp["B"][t], inp["C"][t], inp["D"])
        torch.cuda.synchronize()
        worst = max(worst, rel_err(y.cpu().numpy(), yo))
        ys.append(y.clone())
    es = rel_err(st.cpu().numpy(), st_o)
    graph = ssd.DecodeGraph(st_g, xs, dts, A, Bs, Cs, D)
    yg = graph.launch()
    torch.cuda.synchronize()
    graph.close()
    print(f"[fp8 decode] y={worst:.2e} state={es:.2e}", flush=True)
    assert worst < TOL["fp8"] and es < TOL["fp8"]
    assert torch.equal(st_g, st) and torch.equal(yg, torch.stack(ys))


def test_fp8_full_size_2p7b_layer_sampled_heads():
    """The 2.7B-shaped 16384-token layer with e4m3 inputs (the launch configuration the
    benchmark's fp8 variant times); the oracle recomputes three heads."""
    torch = gh.torch()
    s = synth.PrefillShape(1, 16384, 80, 64, 128, 1, 256, "fp8", "randn")
    full = synth.prefill_inputs(s, synth.SEED_BASE + 3)
    g = gh.upload(full)
    y, hT = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=s.chunk)
    y0, _ = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], None, g["h0"], chunk=s.chunk, final_state=None)
    torch.cuda.synchronize()
    heads = [0, 41, 79]
    sub = synth.select_heads(full, heads, s.ngroups, s.nheads)
    yo, ho = gh.oracle_prefill(sub)
    yo0, _ = gh.oracle_prefill(sub, D=None)
    errs = dict(y=rel_err(y[:, :, heads].cpu().numpy(), yo), y_D0=rel_err(y0[:, :, heads].cpu().numpy(), yo0),
                state=rel_err(hT[:, heads].cpu().numpy(), ho))
    print("[fp8 full 2.7B] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert all(v < TOL["fp8"] for v in errs.values()), errs
    assert torch.isfinite(y).all().item()


def test_fp8_nan_codes_propagate():
    """A NaN code (0x7f, 0xff) in x widens to NaN: y is NaN in that channel from that token on,
    finite in every other channel of the head, in every earlier chunk and in the other head.
    Tokens of the same chunk before the NaN token may be NaN too: the chunk's masked product
    weighs the NaN token with a zero (0 * NaN is NaN), as the blocked matrix form does.  Every
    finite code widens exactly (head 1 cycles through all of them, checked against the oracle)."""
    torch = gh.torch()
    B, L, H, P, N, Q = 1, 512, 2, 64, 64, 64
    inp = synth.random_prefill(_rng(5), B, L, H, P, N, 1, "fp8", dt_mode="weak")
    finite = np.array([synth.e4m3_value(c) for c in range(256) if c not in (0x7F, 0xFF)], np.float32)
    inp["x"][0, :, 1, :] = np.resize(finite, (L, P))  # every finite code, up to +-448
    g = gh.upload(inp)
    codes = g["x"].view(torch.uint8)
    t0, p0 = 300, 5
    codes[0, t0, 0, p0] = 0x7F
    y, hT = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q)
    torch.cuda.synchronize()
    yc = y.cpu().numpy()
    assert np.isnan(yc[0, t0:, 0, p0]).all()
    assert np.isfinite(yc[0, :(t0 // Q) * Q, 0]).all()
    assert np.isfinite(np.delete(yc[0, :, 0], p0, axis=1)).all()
    assert np.isfinite(yc[0, :, 1]).all()
    hc = hT.cpu().numpy()
    assert np.isnan(hc[0, 0, p0]).all() and np.isfinite(np.delete(hc[0, 0], p0, axis=0)).all()
    sub = synth.select_heads(inp, [1], 1, H)
    yo, ho = gh.oracle_prefill(sub)
    e = rel_err(yc[:, :, [1]], yo)
    print(f"[fp8 codes] head with every finite code: y={e:.2e}", flush=True)
    assert e < TOL["fp8"]
