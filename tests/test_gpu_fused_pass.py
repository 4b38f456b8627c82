"""GPU tests of the prefill whose chunk scan runs the chunk recurrence itself.

When every (b, h, chunk) item of a bf16 problem with 256-token chunks and
headdim 64 fits the GPU at once, ssd_prefill runs two launches: chunk state,
then the chunk scan with the inter-chunk recurrence (Step-3) inside it, each
workgroup walking the recurrence for its share of the head's state and waiting
for the head's other chunks (with between one and two items per compute unit,
some items are split over two workgroups of one 16-row tile per wavefront).  The recurrence's arithmetic is the standalone
state-passing kernel's, so the two-launch prefill must equal the three-launch
one (ssd_prefill_forced with SSD_PATH_STAGED_ONE_HEAD) bit for bit, and the fp64 oracle within the bf16
bar.  The forced three-launch path also keeps one head per chunk-state
workgroup, so the same comparison covers the two-heads-per-workgroup chunk-state
kernel the default path uses (on one-round grids here, on grids of many rounds in the last
test).  Every case runs twice on one workspace with different inputs: the
per-head counters must start from zero on every call.
"""
from __future__ import annotations

import numpy as np
import pytest

from mamba_ssd_scan_amd import ssd, synth
from tests import gpu_helpers as gh
from tests.util import TOL, rel_err

pytestmark = pytest.mark.gpu

Q = 256


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ssd.lib()


def _fits(B, L, H):
    """Whether the library takes the one-round path: items <= 2 per compute unit."""
    torch = gh.torch()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    return B * H * ssd.nchunks(L, Q) <= 2 * ncu


def _two_launch_path(B, L, H):
    """The path these tests compare with the one-head three-launch prefill bit for bit: the
    one-round path where it applies (at most 16 chunks), else the three-launch path with two
    heads per chunk-state workgroup."""
    return ssd.PATH_ONE_ROUND if _fits(B, L, H) and ssd.nchunks(L, Q) <= 16 else ssd.PATH_STAGED


def _prefill(g, final, ws, staged, path=None):
    """ssd_prefill on the library's path, or on the three-launch one with one head per
    chunk-state workgroup (staged)."""
    if path is None:
        path = ssd.PATH_STAGED_ONE_HEAD if staged else ssd.PATH_AUTO
    return ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q,
                       final_state="new" if final else None, workspace=ws, path=path)


# (B, L, H, N, G, with initial state, with final state, dt mode)
CASES = [
    (1, 4096, 24, 128, 1, True, True, "softplus"),   # the 130M layer at 4096 tokens: 16 chunks x 24 heads
    (2, 700, 8, 64, 2, True, True, "weak"),          # 3 chunks, ragged last chunk, long memory
    (1, 256, 4, 32, 1, False, True, "softplus"),     # one chunk: the whole state in one workgroup
    (3, 1000, 6, 128, 3, False, False, "weak"),      # no initial, no final state
    (1, 21 * 256 - 5, 24, 128, 1, True, True, "weak"),  # 21 chunks: the three-launch path on both sides
    (2, 15 * 256 + 77, 16, 128, 2, True, True, "weak"),  # 16 chunks, ragged, 512 items
    (4, 1100, 20, 128, 4, True, True, "weak"),           # 5 chunks, ragged
    (1, 12 * 256 - 100, 25, 64, 5, True, True, "weak"),  # 300 items: 40 of them split in halves
    (1, 14 * 256, 32, 128, 1, False, True, "softplus"),  # 448 items: 64 split
    (2, 5 * 256, 40, 64, 1, True, True, "softplus"),    # 5 chunks x 80 head-items
]


@pytest.mark.parametrize("B,L,H,N,G,init,final,mode", CASES)
def test_fused_pass_equals_stages_and_oracle(B, L, H, N, G, init, final, mode):
    torch = gh.torch()
    if not _fits(B, L, H):
        pytest.skip("problem does not fit this device in one round")
    ws = ssd.alloc_workspace(B, L, H, 64, N, G, Q)
    ci = CASES.index((B, L, H, N, G, init, final, mode))
    for call in range(2):
        seed = 700 + 10 * ci + call
        inp = synth.random_prefill(np.random.Generator(np.random.PCG64(seed)), B, L, H, 64, N, G, "bf16",
                                   init_state=init, dt_mode=mode)
        print(f"[fused pass] B={B} L={L} H={H} N={N} G={G} init={init} final={final} {mode} call {call}", flush=True)
        g = gh.upload(inp)
        y, fin = _prefill(g, final, ws, staged=False, path=_two_launch_path(B, L, H))
        torch.cuda.synchronize()
        ys, fins = _prefill(g, final, ssd.alloc_workspace(B, L, H, 64, N, G, Q), staged=True)
        torch.cuda.synchronize()
        assert torch.equal(y, ys), "two-launch prefill y differs from the three-launch prefill"
        if final:
            assert torch.equal(fin, fins), "two-launch prefill final state differs from the three-launch prefill"
        else:
            assert fin is None
        # oracle: sampled heads at the large shapes, every head at the small ones
        heads = [0, H // 2, H - 1] if B * L * H > 20000 else list(range(H))
        sub = dict(inp)
        for k in ("x", "dt"):
            sub[k] = inp[k][:, :, heads]
        sub["A"], sub["D"] = inp["A"][heads], inp["D"][heads]
        sub["h0"] = None if inp["h0"] is None else inp["h0"][:, heads]
        # the heads keep their groups: expand B and C to one group per kept head
        grp = [h // (H // G) for h in heads]
        sub["B"], sub["C"] = inp["B"][:, :, grp], inp["C"][:, :, grp]
        yo, ho = gh.oracle_prefill(sub)
        ey = rel_err(y.cpu().numpy()[:, :, heads], yo)
        msg = f"    y err {ey:.2e}"
        assert ey < TOL["bf16"], msg
        if final:
            es = rel_err(fin.cpu().numpy()[:, heads], ho)
            msg += f" state err {es:.2e}"
            assert es < TOL["bf16"], msg
        print(msg, flush=True)


@pytest.mark.parametrize("B,L,H,N,G", [(1, 4096, 24, 128, 1), (2, 700, 8, 64, 2), (3, 2000, 10, 32, 5)])
def test_chunk_scan_passing_entry_point(B, L, H, N, G):
    """ssd_chunk_scan_passing against ssd_state_passing + ssd_chunk_scan on the same chunk states."""
    torch = gh.torch()
    if not _fits(B, L, H):
        pytest.skip("problem does not fit this device in one round")
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(790 + L)), B, L, H, 64, N, G, "bf16",
                               dt_mode="weak")
    print(f"[chunk_scan_passing] B={B} L={L} H={H} N={N} G={G}", flush=True)
    g = gh.upload(inp)
    acum, dtc = ssd.chunk_cumsum(g["dt"], g["A"], chunk=Q)
    st = ssd.chunk_state(g["x"], g["B"], acum, dtc, chunk=Q)
    cb = ssd.chunk_gemm1(g["B"], g["C"], chunk=Q)
    st2 = st.clone()
    fin = ssd.state_passing(st, acum, g["h0"], chunk=Q)
    y = ssd.chunk_scan(g["x"], g["C"], cb, acum, dtc, st, g["D"], chunk=Q)
    sync = ssd.alloc_sync(B, H)
    for call in range(2):
        st3 = st2.clone()
        sync.zero_()
        y2, fin2 = ssd.chunk_scan_passing(g["x"], g["C"], cb, acum, dtc, st3, sync, g["D"], g["h0"], chunk=Q)
        torch.cuda.synchronize()
        assert torch.equal(y, y2) and torch.equal(fin, fin2), call
        assert torch.equal(st, st3), "entering states differ"
        nc = ssd.nchunks(L, Q)
        assert torch.all(sync.view(B * H, -1)[:, 0] == nc)


def test_chunk_scan_passing_rejects_unsupported_shapes():
    torch = gh.torch()
    x = torch.zeros((1, 4096, 24, 64), dtype=torch.bfloat16, device="cuda")
    C = torch.zeros((1, 4096, 1, 128), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((1, 24, 16, 64, 128), dtype=torch.float16, device="cuda")
    acum = torch.zeros((1, 24, 16, 256), dtype=torch.float32, device="cuda")
    cb = torch.zeros(ssd.chunk_gemm1_size(1, 4096, 1, 128) // 4 + 4, dtype=torch.float32, device="cuda")
    sync = ssd.alloc_sync(1, 24)
    with pytest.raises(ssd.SsdError, match="UNSUPPORTED"):
        ssd.chunk_scan_passing(x, C, cb, acum, acum, st, sync, chunk=128)   # Q = 128
    big = torch.cuda.get_device_properties(0).multi_processor_count * 2 // 24 + 1  # heads x 1 chunk > 2 per CU
    xb = torch.zeros((big, 256, 24, 64), dtype=torch.bfloat16, device="cuda")
    Cb = torch.zeros((big, 256, 1, 128), dtype=torch.bfloat16, device="cuda")
    stb = torch.zeros((big, 24, 1, 64, 128), dtype=torch.float16, device="cuda")
    ab = torch.zeros((big, 24, 1, 256), dtype=torch.float32, device="cuda")
    cbb = torch.zeros(ssd.chunk_gemm1_size(big, 256, 1, 256) // 4 + 4, dtype=torch.float32, device="cuda")
    with pytest.raises(ssd.SsdError, match="UNSUPPORTED"):
        ssd.chunk_scan_passing(xb, Cb, cbb, ab, ab, stb, ssd.alloc_sync(big, 24), chunk=256)


def test_prefill_in_a_callers_graph():
    """ssd_prefill captured by a caller's graph (torch.cuda.CUDAGraph) on the two-launch path:
    the per-head counters are zeroed by the chunk-state launch, not by a memset, so every replay
    starts from zero.  Inputs are rewritten between replays, with eager work and
    synchronisations in between; every replay must equal an eager call bit for bit."""
    torch = gh.torch()
    B, L, H, N, G = 1, 4096, 24, 128, 1
    if not _fits(B, L, H):
        pytest.skip("problem does not fit this device in one round")
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(880)), B, L, H, 64, N, G, "bf16", dt_mode="weak")
    g = gh.upload(inp)
    ws = ssd.alloc_workspace(B, L, H, 64, N, G, Q)
    y = torch.empty((B, L, H, 64), dtype=torch.float32, device="cuda")
    fin = torch.empty((B, H, 64, N), dtype=torch.float32, device="cuda")
    run = lambda: ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=Q, y=y,
                              final_state=fin, workspace=ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm the library on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        print(f"[prefill graph] replay {r}", flush=True)
        new = synth.random_prefill(np.random.Generator(np.random.PCG64(881 + r)), B, L, H, 64, N, G, "bf16",
                                   dt_mode="weak")
        nd = gh.upload(new)
        for k in ("x", "dt", "B", "C", "A", "D", "h0"):
            g[k].copy_(nd[k])
        graph.replay()
        torch.cuda.synchronize()
        yg, fg = y.clone(), fin.clone()
        ye, fe = ssd.prefill(nd["x"], nd["dt"], nd["A"], nd["B"], nd["C"], nd["D"], nd["h0"], chunk=Q)
        torch.cuda.synchronize()
        assert torch.equal(yg, ye) and torch.equal(fg, fe), f"replay {r} differs from the eager prefill"
        (torch.randn(256, 256, device="cuda") @ torch.randn(256, 256, device="cuda")).sum().item()


@pytest.mark.parametrize("B,L,H,N,G", [
    (1, 16384, 80, 128, 1),      # the 2.7B layer at 16384 tokens: 64 chunks, 2816 workgroups
    (2, 9 * 256 + 31, 12, 64, 3),  # ragged, two heads per group
    (3, 3000, 8, 32, 1),
])
def test_two_head_chunk_state_on_grids_of_many_rounds(B, L, H, N, G):
    """The two-heads-per-workgroup chunk state also runs where its grid takes several rounds
    (it needs no co-residency); the three-launch prefill with it equals the one that keeps one
    head per chunk-state workgroup, bit for bit."""
    torch = gh.torch()
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(950 + H)), B, L, H, 64, N, G, "bf16",
                               init_state=True, dt_mode="weak")
    print(f"[two-head chunk state, many rounds] B={B} L={L} H={H} N={N} G={G}", flush=True)
    g = gh.upload(inp)
    y, fin = _prefill(g, True, ssd.alloc_workspace(B, L, H, 64, N, G, Q), staged=False, path=ssd.PATH_STAGED)
    ys, fins = _prefill(g, True, ssd.alloc_workspace(B, L, H, 64, N, G, Q), staged=True)
    torch.cuda.synchronize()
    assert torch.equal(y, ys) and torch.equal(fin, fins)
