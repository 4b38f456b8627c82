"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Error metric: normwise max relative error (tests/util.py) on y with the
configured D, on y with D = 0 (the skip term would otherwise hide errors in
the SSD part) and on the final state.  Bar: 2e-3 for bf16 inputs, 1e-4 for
fp32 inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

from mamba_ssd_scan_amd import ssd, synth
from oracle import chunked, ref
from tests import gpu_helpers as gh
from tests.util import TOL, rel_err

pytestmark = pytest.mark.gpu


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


# --------------------------------------------------------------------------- decode

@pytest.mark.parametrize("dtype,P,N,G", [("bf16", 64, 128, 1), ("f32", 64, 64, 2), ("bf16", 32, 32, 4),
                                         ("bf16", 128, 64, 1)])
def test_step_matches_oracle(dtype, P, N, G):
    torch = gh.torch()
    B, H, S = 3, 8, 12
    inp = synth.random_prefill(rng(1), B, S, H, P, N, G, dtype)
    g = gh.upload(inp)
    st = g["h0"].clone()
    st_o = inp["h0"].astype(np.float64).copy()
    worst = 0.0
    for t in range(S):
        y = ssd.step(st, g["x"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"], g["B"][:, t].contiguous(),
                     g["C"][:, t].contiguous(), g["D"])
        yo = ref.step(st_o, inp["x"][:, t], inp["dt"][:, t], inp["A"], inp["B"][:, t], inp["C"][:, t], inp["D"])
        torch.cuda.synchronize()
        worst = max(worst, rel_err(y.cpu().numpy(), yo))
    e_state = rel_err(st.cpu().numpy(), st_o)
    print(f"[step] {dtype} P={P} N={N} G={G} y={worst:.2e} state={e_state:.2e}", flush=True)
    assert worst < TOL[dtype] and e_state < TOL[dtype]


def test_step_without_skip_term():
    torch = gh.torch()
    inp = synth.random_prefill(rng(2), 2, 1, 4, 64, 128, 1, "bf16")
    g = gh.upload(inp)
    st = g["h0"].clone()
    y = ssd.step(st, g["x"][:, 0].contiguous(), g["dt"][:, 0].contiguous(), g["A"], g["B"][:, 0].contiguous(),
                 g["C"][:, 0].contiguous(), None)
    st_o = inp["h0"].astype(np.float64).copy()
    yo = ref.step(st_o, inp["x"][:, 0], inp["dt"][:, 0], inp["A"], inp["B"][:, 0], inp["C"][:, 0], None)
    torch.cuda.synchronize()
    assert rel_err(y.cpu().numpy(), yo) < 2e-3


# --------------------------------------------------------------------------- stages

def _stage_case(dtype="bf16", L=700, Q=128, P=64, N=128, G=1, H=4, B=2, mode="weak"):
    inp = synth.random_prefill(rng(3), B, L, H, P, N, G, dtype, dt_mode=mode)
    r = chunked.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"], Q=Q)
    return inp, r


@pytest.mark.parametrize("Q", [16, 64, 256])
def test_stage_cumsum(Q):
    torch = gh.torch()
    inp, r = _stage_case(Q=Q, L=611)
    g = gh.upload(inp)
    acum, dtc = ssd.chunk_cumsum(g["dt"], g["A"], chunk=Q)
    torch.cuda.synchronize()
    assert np.array_equal(dtc.cpu().numpy(), r["dt"].astype(np.float32))
    e = rel_err(acum.cpu().numpy(), r["acum"])
    print(f"[cumsum] Q={Q} acum={e:.2e}", flush=True)
    assert e < 1e-5


@pytest.mark.parametrize("dtype,Q,P,N", [("bf16", 128, 64, 128), ("bf16", 64, 32, 64), ("f32", 64, 64, 64),
                                         ("bf16", 16, 128, 32)])
def test_stage_chunk_state(dtype, Q, P, N):
    torch = gh.torch()
    inp, r = _stage_case(dtype=dtype, Q=Q, P=P, N=N)
    g = gh.upload(inp)
    acum = torch.from_numpy(r["acum"].astype(np.float32)).cuda()
    dtc = torch.from_numpy(r["dt"].astype(np.float32)).cuda()
    st = ssd.chunk_state(g["x"], g["B"], acum, dtc, chunk=Q)
    torch.cuda.synchronize()
    assert st.dtype == (torch.float16 if dtype == "bf16" else torch.float32)
    e = rel_err(st.float().cpu().numpy(), r["states"])
    print(f"[chunk_state] {dtype} Q={Q} P={P} N={N} err={e:.2e}", flush=True)
    # bf16 inputs store the fp32-accumulated state in fp16: half an ulp, 2^-11 of the element
    assert e < TOL[dtype] / 2 + (2.0 ** -11 if dtype == "bf16" else 0.0)


@pytest.mark.parametrize("sdtype", ["f32", "f16"])
def test_stage_state_passing(sdtype):
    """fp32 states: the carry itself (bar 1e-5).  fp16 states (bf16 inputs): the oracle's
    chunk states rounded to fp16 go in and the entering states come out rounded to fp16
    (each rounding half an ulp, 2^-11 of the element; the carry is fp32): bar 2^-10."""
    torch = gh.torch()
    inp, r = _stage_case(Q=64, L=1000)
    acum = torch.from_numpy(r["acum"].astype(np.float32)).cuda()
    npt = np.float32 if sdtype == "f32" else np.float16
    states = torch.from_numpy(r["states"].astype(npt)).cuda()
    h0 = torch.from_numpy(inp["h0"].astype(np.float32)).cuda()
    fin = ssd.state_passing(states, acum, h0, chunk=64)
    torch.cuda.synchronize()
    e1 = rel_err(states.float().cpu().numpy(), r["h_enter"])
    e2 = rel_err(fin.cpu().numpy(), r["final"])
    print(f"[state_passing] {sdtype} h_enter={e1:.2e} final={e2:.2e}", flush=True)
    bar = 1e-5 if sdtype == "f32" else 2.0 ** -10
    assert e1 < bar and e2 < bar


def decode_gemm1(cb, B, G, nc, Q):
    """Unpack the GEMM1 output into [B, G, nc, Q, Q] (NaN where the layout holds nothing).

    Layout: per (b, g, c), row tile t (rows 16t..16t+15) and 32-column step s <= t/2 are
    numbered t by t; each holds 64 lanes x 8 values, lane l = 16 lg + li carrying
    G[16t + li][32s + 4lg + r] at r and G[16t + li][32s + 16 + 4lg + r] at 4 + r.
    """
    nt = Q // 16
    steps = [(t, s) for t in range(nt) for s in range(t // 2 + 1)]
    arr = cb[: B * G * nc * len(steps) * 512].reshape(B, G, nc, len(steps), 64, 8)
    out = np.full((B, G, nc, Q, Q), np.nan)
    lane = np.arange(64)
    li, lg = lane % 16, lane // 16
    for k, (t, s) in enumerate(steps):
        for r in range(4):
            for half in range(2):
                j = 32 * s + 16 * half + 4 * lg + r
                ok = j < Q
                out[:, :, :, 16 * t + li[ok], j[ok]] = arr[:, :, :, k, lane[ok], 4 * half + r]
    return out


@pytest.mark.parametrize("dtype,Q,N,G,L", [("bf16", 256, 128, 1, 700), ("bf16", 64, 64, 2, 1000),
                                           ("f32", 64, 64, 1, 300), ("bf16", 32, 128, 1, 100),
                                           ("bf16", 16, 32, 4, 50), ("f32", 128, 32, 2, 129)])
def test_stage_chunk_gemm1(dtype, Q, N, G, L):
    """C.B^T of every chunk against the oracle's Step-1 GEMM1, on the causal triangle."""
    torch = gh.torch()
    inp, r = _stage_case(dtype=dtype, Q=Q, P=32, N=N, G=G, L=L, H=G)
    g = gh.upload(inp)
    cb = ssd.chunk_gemm1(g["B"], g["C"], chunk=Q)
    torch.cuda.synchronize()
    nc = -(-L // Q)
    raw = cb.cpu().numpy()
    # bf16 inputs: the products are stored as fp16 (the matrix-core operand type downstream)
    vals = raw.view(np.float16) if dtype == "bf16" else raw
    got = decode_gemm1(vals.astype(np.float64), inp["x"].shape[0], G, nc, Q)
    want = r["gemm1"]
    tok = np.arange(nc)[:, None] * Q + np.arange(Q)[None, :]          # [nc, Q] global token
    keep = np.tril(np.ones((Q, Q), bool))[None] & (tok < L)[:, :, None]  # j <= i, row in sequence
    e = np.abs(got - want)[:, :, keep].max() / np.abs(want[:, :, keep]).max()
    print(f"[chunk_gemm1] {dtype} Q={Q} N={N} G={G} L={L} err={e:.2e}", flush=True)
    # fp32 accumulation of exact products; bf16 inputs add the fp16 rounding of the stored
    # value, at most 2^-11 of the element and so of max|G|
    bound = 2.0 ** -11 if dtype == "bf16" else TOL[dtype] / 20
    assert np.isfinite(got[:, :, keep]).all() and e < bound


@pytest.mark.parametrize("dtype,Q,P,N,G", [("bf16", 256, 64, 128, 1), ("bf16", 64, 64, 64, 2),
                                           ("f32", 64, 64, 64, 1), ("bf16", 32, 128, 128, 1),
                                           ("bf16", 16, 32, 32, 4), ("bf16", 128, 128, 64, 1),
                                           ("f32", 256, 32, 128, 1)])
def test_stage_chunk_scan(dtype, Q, P, N, G):
    torch = gh.torch()
    inp, r = _stage_case(dtype=dtype, Q=Q, P=P, N=N, G=G)
    g = gh.upload(inp)
    f = lambda a: torch.from_numpy(a.astype(np.float32)).cuda()
    for D in (g["D"], None):
        cb = ssd.chunk_gemm1(g["B"], g["C"], chunk=Q)
        # bf16 inputs take the entering states in fp16, the precision the kernel feeds them to
        # the matrix cores in (the same rounding it would otherwise apply itself)
        hq = f(r["h_enter"]) if dtype == "f32" else torch.from_numpy(r["h_enter"].astype(np.float16)).cuda()
        y = ssd.chunk_scan(g["x"], g["C"], cb, f(r["acum"]), f(r["dt"]), hq, D, chunk=Q)
        torch.cuda.synchronize()
        yo = r["y"] if D is not None else chunked.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], None,
                                                          inp["h0"], Q=Q)["y"]
        e = rel_err(y.cpu().numpy(), yo)
        print(f"[chunk_scan] {dtype} Q={Q} P={P} N={N} G={G} D={'y' if D is not None else 0} err={e:.2e}", flush=True)
        assert e < TOL[dtype] / 2


# --------------------------------------------------------------------------- prefill

@pytest.mark.parametrize("case", [
    # (dtype, B, L, H, P, N, G, Q, dt_mode, init)
    ("bf16", 2, 1000, 6, 64, 128, 3, 256, "softplus", True),   # ragged last chunk, G > 1
    ("bf16", 1, 777, 4, 64, 64, 1, 64, "weak", True),          # long memory: state passing matters
    ("bf16", 2, 333, 4, 128, 128, 2, 128, "weak", False),
    ("bf16", 1, 300, 2, 32, 32, 1, 16, "softplus", True),
    ("bf16", 1, 129, 4, 64, 128, 1, 32, "strong", True),       # decays underflow to zero
    ("f32", 1, 500, 4, 64, 64, 2, 64, "weak", True),
    ("f32", 2, 260, 3, 32, 128, 1, 128, "softplus", True),
    ("bf16", 3, 1, 4, 64, 64, 1, 64, "softplus", True),         # one token
    ("bf16", 1, 64, 4, 64, 64, 1, 64, "weak", True),            # exactly one chunk
    # 720 items (more than two per CU): two-head chunk state and the pipelined scan, with
    # four groups, two sequences and a ragged last chunk
    ("bf16", 2, 2100, 40, 64, 128, 4, 256, "softplus", True),
])
def test_prefill_matches_oracle(case):
    dtype, B, L, H, P, N, G, Q, mode, init = case
    inp = synth.random_prefill(rng(4), B, L, H, P, N, G, dtype, dt_mode=mode, init_state=init)
    gh.check_prefill(inp, Q, label=str(case))


def test_prefill_every_chunk_length_gives_the_same_result():
    inp = synth.random_prefill(rng(5), 1, 600, 4, 64, 128, 1, "bf16", dt_mode="weak")
    ys = {}
    for Q in (16, 32, 64, 128, 256):
        gh.check_prefill(inp, Q, label="Q-invariance")
        ys[Q] = gh.gpu_prefill(inp, Q)[0]
    for Q in ys:
        assert rel_err(ys[Q], ys[256]) < 2e-3


def test_config0_tiny_f32():
    s = synth.WORKLOADS[0]
    inp = synth.prefill_inputs(s, synth.SEED_BASE + 0)
    gh.check_prefill(inp, s.chunk, tol=1e-4, label="config0")


def test_seqlen_zero_copies_state():
    torch = gh.torch()
    inp = synth.random_prefill(rng(6), 2, 0, 4, 64, 64, 1, "bf16")
    y, hT = gh.gpu_prefill(inp, 64)
    assert y.shape == (2, 0, 4, 64) and np.array_equal(hT, inp["h0"])
    y, hT = gh.gpu_prefill(inp, 64, h0=None)
    assert np.array_equal(hT, np.zeros_like(inp["h0"]))


def test_final_state_may_alias_initial_state():
    torch = gh.torch()
    inp = synth.random_prefill(rng(7), 2, 300, 4, 64, 128, 1, "bf16", dt_mode="weak")
    g = gh.upload(inp)
    st = g["h0"].clone()
    y, hT = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], st, chunk=64, final_state=st)
    torch.cuda.synchronize()
    yo, ho = gh.oracle_prefill(inp)
    assert hT is st
    assert rel_err(st.cpu().numpy(), ho) < 2e-3 and rel_err(y.cpu().numpy(), yo) < 2e-3


def test_prefill_is_bitwise_deterministic():
    inp = synth.random_prefill(rng(8), 2, 900, 8, 64, 128, 1, "bf16")
    a = gh.gpu_prefill(inp, 256)
    b = gh.gpu_prefill(inp, 256)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_prefill_then_steps_equals_longer_prefill():
    """The final state is the decode cache: prefill(L) + k steps == prefill(L + k)."""
    torch = gh.torch()
    L0, k = 500, 6
    inp = synth.random_prefill(rng(9), 2, L0 + k, 4, 64, 128, 1, "bf16", dt_mode="weak")
    g = gh.upload(inp)
    _, st = ssd.prefill(g["x"][:, :L0].contiguous(), g["dt"][:, :L0].contiguous(), g["A"],
                        g["B"][:, :L0].contiguous(), g["C"][:, :L0].contiguous(), g["D"], g["h0"], chunk=128)
    ys = [ssd.step(st, g["x"][:, t].contiguous(), g["dt"][:, t].contiguous(), g["A"], g["B"][:, t].contiguous(),
                   g["C"][:, t].contiguous(), g["D"]) for t in range(L0, L0 + k)]
    torch.cuda.synchronize()
    yo, ho = gh.oracle_prefill(inp)
    for i, t in enumerate(range(L0, L0 + k)):
        assert rel_err(ys[i].cpu().numpy(), yo[:, t]) < 2e-3
    assert rel_err(st.cpu().numpy(), ho) < 2e-3


# --------------------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("cfg,heads", [(1, [0, 9, 23]), (2, [0, 17, 31]), (3, [0, 41, 79])])
def test_full_size_workload_sampled_heads(cfg, heads):
    """Full workload shape on the GPU (the launch configuration the benchmark
    times); the oracle recomputes a sample of heads (heads are independent)."""
    torch = gh.torch()
    s = synth.WORKLOADS[cfg]
    full = synth.prefill_inputs(s, synth.SEED_BASE + cfg)
    g = gh.upload(full)
    y, hT = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=s.chunk)
    y0, _ = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], None, g["h0"], chunk=s.chunk, final_state=None)
    torch.cuda.synchronize()
    bsel = slice(0, 2) if s.batch > 2 else slice(None)
    sub = synth.select_heads(full, heads, s.ngroups, s.nheads)
    for k in ("x", "dt", "B", "C"):
        sub[k] = sub[k][bsel]
    if sub["h0"] is not None:
        sub["h0"] = sub["h0"][bsel]
    yo, ho = gh.oracle_prefill(sub)
    yo0, _ = gh.oracle_prefill(sub, D=None)
    yg = y[bsel][:, :, heads].cpu().numpy()
    y0g = y0[bsel][:, :, heads].cpu().numpy()
    hg = hT[bsel][:, heads].cpu().numpy()
    errs = dict(y=rel_err(yg, yo), y_D0=rel_err(y0g, yo0), state=rel_err(hg, ho))
    print(f"[full cfg{cfg}] heads={heads} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v < TOL["bf16"], (k, v)
    assert torch.isfinite(y).all().item()


@pytest.mark.parametrize("cfg,heads,seed", [(1, [2, 11, 22], 1000), (2, [3, 20, 30], 1000), (3, [5, 38, 77], 1000),
                                           (3, [1, 40, 78], 2000)])
def test_full_size_workload_other_draws(cfg, heads, seed):
    """The full workloads again with other seeded draws and other heads sampled, so that the
    bar is not met by one draw alone."""
    torch = gh.torch()
    s = synth.WORKLOADS[cfg]
    full = synth.prefill_inputs(s, synth.SEED_BASE + cfg + seed)
    g = gh.upload(full)
    y, hT = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=s.chunk)
    y0, _ = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], None, g["h0"], chunk=s.chunk, final_state=None)
    torch.cuda.synchronize()
    bsel = slice(0, 2) if s.batch > 2 else slice(None)
    sub = synth.select_heads(full, heads, s.ngroups, s.nheads)
    for k in ("x", "dt", "B", "C"):
        sub[k] = sub[k][bsel]
    if sub["h0"] is not None:
        sub["h0"] = sub["h0"][bsel]
    yo, ho = gh.oracle_prefill(sub)
    yo0, _ = gh.oracle_prefill(sub, D=None)
    errs = dict(y=rel_err(y[bsel][:, :, heads].cpu().numpy(), yo),
                y_D0=rel_err(y0[bsel][:, :, heads].cpu().numpy(), yo0),
                state=rel_err(hT[bsel][:, heads].cpu().numpy(), ho))
    print(f"[full cfg{cfg} seed+{seed}] heads={heads} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for k, v in errs.items():
        assert v < TOL["bf16"], (k, v)


@pytest.mark.parametrize("L", [8192, 16384])
def test_130m_long_prefill_either_side_of_the_streaming_bound(L):
    """The 130M layer at 8192 and 16384 tokens: X, twice the states and y come to ~100 MB and
    ~200 MB, on either side of the bound past which the prefill streams X past the Infinity
    Cache; both run the three-launch path with the pipelined chunk scan (more than 16 chunks).
    Sampled heads against the oracle."""
    torch = gh.torch()
    s = synth.PrefillShape(1, L, 24, 64, 128, 1, 256, "bf16", "randn")
    full = synth.prefill_inputs(s, synth.SEED_BASE + 50 + L)
    g = gh.upload(full)
    heads = [0, 13, 23]
    y, hT = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=s.chunk)
    y0, _ = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], None, g["h0"], chunk=s.chunk, final_state=None)
    torch.cuda.synchronize()
    sub = synth.select_heads(full, heads, s.ngroups, s.nheads)
    yo, ho = gh.oracle_prefill(sub)
    yo0, _ = gh.oracle_prefill(sub, D=None)
    errs = dict(y=rel_err(y[:, :, heads].cpu().numpy(), yo), y_D0=rel_err(y0[:, :, heads].cpu().numpy(), yo0),
                state=rel_err(hT[:, heads].cpu().numpy(), ho))
    print(f"[130M L={L}] " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for k, v in errs.items():
        assert v < TOL["bf16"], (k, v)


def test_full_size_decode_sampled():
    """Decode at the full batch/head shape for 64 tokens; oracle on a sample of (b, h)."""
    torch = gh.torch()
    s = synth.WORKLOADS[4]
    S = 64
    inp = synth.decode_inputs(s, synth.SEED_BASE + 4, steps=S)
    T = torch
    st = T.from_numpy(inp["state"]).cuda()
    xs, dts = synth.to_torch(inp["x"], "bf16"), synth.to_torch(inp["dt"], "bf16")
    Bs, Cs = synth.to_torch(inp["B"], "bf16"), synth.to_torch(inp["C"], "bf16")
    A = T.from_numpy(inp["A"]).cuda()
    D = T.from_numpy(inp["D"]).cuda()
    bs, hs = [0, 17, 63], [0, 33, 79]
    st_o = inp["state"][bs][:, hs].astype(np.float64).copy()
    worst = 0.0
    for t in range(S):
        y = ssd.step(st, xs[t], dts[t], A, Bs[t], Cs[t], D)
        yo = ref.step(st_o, inp["x"][t][bs][:, hs], inp["dt"][t][bs][:, hs], inp["A"][hs], inp["B"][t][bs],
                      inp["C"][t][bs], inp["D"][hs])
        if t % 8 == 7 or t == S - 1:
            torch.cuda.synchronize()
            worst = max(worst, rel_err(y[bs][:, hs].cpu().numpy(), yo))
    torch.cuda.synchronize()
    e_state = rel_err(st[bs][:, hs].cpu().numpy(), st_o)
    print(f"[full decode] steps={S} y={worst:.2e} state={e_state:.2e}", flush=True)
    assert worst < 2e-3 and e_state < 2e-3
