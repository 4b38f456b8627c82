"""GPU tests of the prefill reading its inputs in place from wider token rows
(ssd_prefill_strided, reached through views in ssd.prefill / ssd.prefill_ex).

A Mamba-2 layer holds x, B and C side by side in the convolved rows [x | B | C], and the
gate and the step sizes in the input-projection rows [z | x | B | C | dt]
("Mamba-Family State-Space Model Kernels on a Programmable CGLA", Sec. III-A).  Here the
same inputs are laid out that way, with padding channels filled with NaN and the
projection's own x, B and C channels too, so that a read of any element other than the
input's own shows up in the output.  Where an input sits does not change the arithmetic,
so y and the final state must equal those of the call on dense copies bit for bit.
"""
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


def _layer_rows(g, opt_z, pad_xbc):
    """The inputs of g laid out as a layer holds them: returns views x, B, C (of the [x|B|C|pad]
    rows) and z, dt (of the [z|x|B|C|dt|pad] rows)."""
    torch = gh.torch()
    x, Bm, Cm, dt = g["x"], g["B"], g["C"], g["dt"]
    b, l, h, p = x.shape
    gn = Bm.shape[2] * Bm.shape[3]
    hp = h * p
    nan = float("nan")
    xbc = torch.full((b, l, hp + 2 * gn + pad_xbc), nan, dtype=x.dtype, device=x.device)
    xbc[..., :hp] = x.reshape(b, l, hp)
    xbc[..., hp:hp + gn] = Bm.reshape(b, l, gn)
    xbc[..., hp + gn:hp + 2 * gn] = Cm.reshape(b, l, gn)
    zin = torch.full((b, l, 2 * hp + 2 * gn + h + 3), nan, dtype=x.dtype, device=x.device)
    if opt_z is not None:
        zin[..., :hp] = opt_z.reshape(b, l, hp)
    zin[..., 2 * hp + 2 * gn:2 * hp + 2 * gn + h] = dt
    v = dict(x=xbc[..., :hp].unflatten(-1, (h, p)),
             B=xbc[..., hp:hp + gn].unflatten(-1, tuple(Bm.shape[2:])),
             C=xbc[..., hp + gn:hp + 2 * gn].unflatten(-1, tuple(Cm.shape[2:])),
             dt=zin[..., 2 * hp + 2 * gn:2 * hp + 2 * gn + h],
             z=zin[..., :hp].unflatten(-1, (h, p)) if opt_z is not None else None)
    return v, (xbc, zin)


# (dtype, B, L, H, P, N, G, Q, gate and softplus): the paths of the prefill
CASES = [
    ("bf16", 1, 4096, 24, 64, 128, 1, 256, False),   # two launches: two-head chunk state, one-round scan with Step-3
    ("bf16", 1, 4096, 24, 64, 128, 1, 256, True),
    ("bf16", 1, 21 * 256 - 5, 24, 64, 128, 1, 256, True),  # three launches, one-round scan without Step-3
    ("bf16", 2, 6000, 40, 64, 128, 1, 256, False),   # many rounds: two-head chunk state, persistent scan
    ("bf16", 2, 3000, 16, 64, 64, 2, 128, True),     # single-head chunk state, persistent scan (staged loads)
    ("bf16", 1, 700, 6, 128, 32, 3, 64, False),      # odd heads per group, P = 128
    ("f32", 2, 700, 8, 64, 64, 1, 64, True),         # fp32 inputs
    ("f32", 1, 333, 4, 32, 128, 2, 32, False),
    ("bf16", 3, 1, 4, 64, 64, 1, 64, True),          # one token per sequence: batches one row apart
]


@pytest.mark.parametrize("dtype,B,L,H,P,N,G,Q,opts", CASES)
def test_strided_inputs_equal_dense_inputs(dtype, B, L, H, P, N, G, Q, opts):
    torch = gh.torch()
    rng = np.random.Generator(np.random.PCG64(1200 + L + H))
    inp = synth.random_prefill(rng, B, L, H, P, N, G, dtype)
    g = gh.upload(inp)
    kw = {}
    z = None
    if opts:
        opt = synth.option_inputs(rng, inp)
        z = synth.to_torch(opt["z"], dtype)
        g["dt"] = synth.to_torch(opt["dt_raw"], dtype)
        kw = dict(dt_bias=torch.from_numpy(opt["dt_bias"]).cuda(), dt_softplus=True, z=z)
    print(f"[strided] {dtype} B={B} L={L} H={H} P={P} N={N} G={G} Q={Q} opts={opts}", flush=True)
    y, fin = ssd.prefill_ex(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q, **kw)
    v, keep = _layer_rows(g, z, pad_xbc=8)
    assert not v["x"].is_contiguous() and not v["dt"].is_contiguous()
    kws = dict(kw)
    if opts:
        kws["z"] = v["z"]
    ys, fins = ssd.prefill_ex(v["x"], v["dt"], g["A"], v["B"], v["C"], g["D"], g["h0"], chunk=Q, **kws)
    torch.cuda.synchronize()
    assert torch.isfinite(ys).all(), "a read outside the inputs' own channels reached y"
    assert torch.equal(y, ys) and torch.equal(fin, fins)
    if not opts:  # the plain entry point takes views too
        yp, finp = ssd.prefill(v["x"], v["dt"], g["A"], v["B"], v["C"], g["D"], g["h0"], chunk=Q)
        torch.cuda.synchronize()
        assert torch.equal(y, yp) and torch.equal(fin, finp)


def test_views_the_kernels_cannot_read_are_refused():
    torch = gh.torch()
    rng = np.random.Generator(np.random.PCG64(1300))
    inp = synth.random_prefill(rng, 2, 300, 4, 64, 64, 1, "bf16")
    g = gh.upload(inp)
    v, keep = _layer_rows(g, None, pad_xbc=8)
    xt = g["x"].transpose(2, 3)  # one token's values not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        ssd.prefill(xt, g["dt"], g["A"], g["B"], g["C"], chunk=64)
    with pytest.raises(ValueError, match="same token stride"):
        ssd.prefill(g["x"], g["dt"], g["A"], v["B"], g["C"], chunk=64)
    xs = keep[0][:, :150][..., :256].unflatten(-1, (4, 64))  # the first 150 tokens: batches 300 tokens apart
    with pytest.raises(ValueError, match="batches"):
        ssd.prefill(xs, g["dt"][:, :150], g["A"], g["B"][:, :150], g["C"][:, :150], chunk=64)
    # a row that is not a whole number of 16 bytes is refused by the library
    odd = torch.zeros((2, 300, 256 + 4), dtype=torch.bfloat16, device="cuda")[..., :256].unflatten(-1, (4, 64))
    with pytest.raises(ssd.SsdError, match="INVALID"):
        ssd.prefill(odd, g["dt"], g["A"], g["B"], g["C"], chunk=64)


@pytest.mark.parametrize("dtype,B,H,P,N,G,opts", [("bf16", 64, 80, 64, 128, 1, True), ("bf16", 3, 8, 64, 64, 2, False),
                                                  ("f32", 5, 4, 32, 128, 2, True), ("bf16", 1, 24, 64, 128, 1, True)])
def test_strided_decode_inputs_equal_dense_inputs(dtype, B, H, P, N, G, opts):
    """A decode token read in place from the rows of each batch entry (ssd_step_strided)
    equals the step on dense copies bit for bit, state and y."""
    torch = gh.torch()
    rng = np.random.Generator(np.random.PCG64(1400 + B + H))
    inp = synth.random_prefill(rng, B, 1, H, P, N, G, dtype, init_state=True)
    g = gh.upload(inp)
    kw, z = {}, None
    if opts:
        opt = synth.option_inputs(rng, inp)
        z = synth.to_torch(opt["z"], dtype)
        g["dt"] = synth.to_torch(opt["dt_raw"], dtype)
        kw = dict(dt_bias=torch.from_numpy(opt["dt_bias"]).cuda(), dt_softplus=True, z=z[:, 0])
    print(f"[strided decode] {dtype} B={B} H={H} P={P} N={N} G={G} opts={opts}", flush=True)
    s0 = g["h0"].clone()
    y = ssd.step_ex(s0, g["x"][:, 0].contiguous(), g["dt"][:, 0].contiguous(), g["A"], g["B"][:, 0].contiguous(),
                    g["C"][:, 0].contiguous(), g["D"], **kw)
    v, keep = _layer_rows(g, z, pad_xbc=8)
    assert not v["x"][:, 0].is_contiguous() or B == 1
    kws = dict(kw)
    if opts:
        kws["z"] = v["z"][:, 0]
    s1 = g["h0"].clone()
    ys = ssd.step_ex(s1, v["x"][:, 0], v["dt"][:, 0], g["A"], v["B"][:, 0], v["C"][:, 0], g["D"], **kws)
    torch.cuda.synchronize()
    assert torch.isfinite(ys).all(), "a read outside the inputs' own channels reached y"
    assert torch.equal(y, ys) and torch.equal(s0, s1)
    if not opts:
        s2 = g["h0"].clone()
        yp = ssd.step(s2, v["x"][:, 0], v["dt"][:, 0], g["A"], v["B"][:, 0], v["C"][:, 0], g["D"])
        torch.cuda.synchronize()
        assert torch.equal(y, yp) and torch.equal(s0, s2)


def test_strided_inputs_on_the_staged_path():
    """Strided inputs through the forced three-launch prefill (one head per chunk-state
    workgroup, the standalone state passing) equal the default two-launch prefill on the
    same views bit for bit."""
    torch = gh.torch()
    rng = np.random.Generator(np.random.PCG64(1600))
    inp = synth.random_prefill(rng, 1, 4096, 24, 64, 128, 1, "bf16", dt_mode="weak")
    g = gh.upload(inp)
    v, keep = _layer_rows(g, None, pad_xbc=8)
    y, fin = ssd.prefill(v["x"], v["dt"], g["A"], v["B"], v["C"], g["D"], g["h0"], chunk=256)
    ys, fins = ssd.prefill(v["x"], v["dt"], g["A"], v["B"], v["C"], g["D"], g["h0"], chunk=256,
                           path=ssd.PATH_STAGED_ONE_HEAD)
    torch.cuda.synchronize()
    assert torch.isfinite(ys).all()
    assert torch.equal(y, ys) and torch.equal(fin, fins)
