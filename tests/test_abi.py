"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and rejects invalid arguments before any HIP call (no kernel is launched)."""
from __future__ import annotations

import os
import re

import pytest

from mamba_ssd_scan_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

F, BF, F8 = ssd.SSD_F32, ssd.SSD_BF16, ssd.SSD_FP8_E4M3
INV, UNS, WS = ssd.SSD_ERR_INVALID_ARG, ssd.SSD_ERR_UNSUPPORTED, ssd.SSD_ERR_WORKSPACE
P0 = 0x100000  # fake, aligned "device" addresses: only used on calls that must be rejected


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = ssd.lib()
    names = declared_functions()
    assert set(names) == set(ssd.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    for s in (0, -1, -2, -3, -4, -5, 99):
        assert isinstance(ssd.status_string(s), str) and ssd.status_string(s)
    assert "SYNC" in ssd.status_string(ssd.SSD_ERR_SYNC)
    assert ssd.lib().ssd_version() >> 16 == 4


def gemm1_steps(q):
    """32-column steps on or below the diagonal of a chunk of q tokens, over its 16-row tiles."""
    return sum(t // 2 + 1 for t in range(q // 16))


def test_gemm1_steps_closed_form():
    # the count the kernels use in closed form: T(2m) = m(m+1), T(2m+1) = (m+1)^2
    assert [gemm1_steps(q) for q in (16, 32, 64, 128, 256)] == [1, 2, 6, 20, 72]


FUSED_DEPTH = 2  # look-back depth of the single-pass prefill: 2 * depth ring slots of each kind per (b, h)


def test_workspace_size_formula():
    L = ssd.lib()
    al = lambda v: (v + 255) // 256 * 256
    for (b, l, h, p, n, g, q) in [(1, 4096, 24, 64, 128, 1, 256), (8, 2048, 32, 64, 64, 1, 64),
                                  (2, 1000, 6, 32, 128, 3, 128), (1, 1, 1, 32, 32, 1, 16),
                                  (1, 16384, 80, 64, 128, 1, 256), (3, 3000, 8, 64, 64, 2, 256)]:
        nc = -(-l // q)
        bhq = b * h * nc * q * 4
        cb = 4 * b * g * nc * gemm1_steps(q) * 512
        # control block, dA_cum, dt_c, states, GEMM1 products, one counter per (b, h)
        want = al(al(al(al(al(256 + bhq) + bhq) + 4 * b * h * nc * p * n) + cb) + 256 * b * h)
        if q == 256 and p == 64 and n in (64, 128):
            # single pass: control block, status words, ring slots, fp16 GEMM1 products
            fused = al(al(al(256 + b * h * 256) + b * h * 4 * FUSED_DEPTH * p * n * 4) + cb // 2)
            want = max(want, fused)
        assert L.ssd_prefill_workspace_size(b, l, h, p, n, g, q) == want, (b, l, h, p, n, g, q)
        assert L.ssd_chunk_gemm1_size(b, l, g, q) == cb
    assert L.ssd_prefill_workspace_size(1, 4096, 24, 64, 128, 1, 48) == 0   # bad chunk
    assert L.ssd_prefill_workspace_size(1, 4096, 24, 40, 128, 1, 64) == 0   # headdim not a multiple of 16
    assert L.ssd_prefill_workspace_size(1, 4096, 24, 272, 128, 1, 64) == 0  # headdim past 256
    assert L.ssd_prefill_workspace_size(1, 4096, 24, 64, 8, 1, 64) == 0     # dstate below 16
    assert L.ssd_prefill_workspace_size(1, 4096, 24, 64, 128, 5, 64) == 0   # H % G


def _native_ws(b, l, h, p, n, g, q):
    al = lambda v: (v + 255) // 256 * 256
    nc = -(-l // q)
    bhq = b * h * nc * q * 4
    cb = 4 * b * g * nc * gemm1_steps(q) * 512
    want = al(al(al(al(al(256 + bhq) + bhq) + 4 * b * h * nc * p * n) + cb) + 256 * b * h)
    if q == 256 and p == 64 and n in (64, 128):
        want = max(want, al(al(al(256 + b * h * 256) + b * h * 4 * FUSED_DEPTH * p * n * 4) + cb // 2))
    return want


@pytest.mark.parametrize("p,n", [(16, 16), (48, 80), (96, 256), (16, 128), (128, 16), (144, 64), (256, 256)])
def test_workspace_size_of_padded_shapes(p, n):
    """P and N that the kernels are not built for run padded to the next built size (P over
    128 as two heads of half the channels); the workspace holds the padded problem's own
    workspace, then padded copies of x, z, B, C, dt, A, D, the bias, the initial state, y and
    the final state (4 bytes per element, each region 256-byte aligned)."""
    L = ssd.lib()
    al = lambda v: (v + 255) // 256 * 256
    b, l, h, g, q = 2, 1000, 6, 3, 128
    pp = 32 if p <= 32 else 64 if p <= 64 else 128 if p <= 128 else 256
    nn = 32 if n <= 32 else 64 if n <= 64 else 128 if n <= 128 else 256
    split = 2 if pp == 256 else 1
    hk, pk = h * split, pp // split
    tok = b * l
    xel, bel, sel = tok * hk * pk, tok * g * nn, b * hk * pk * nn
    off = _native_ws(b, l, hk, pk, nn, g, q)
    for nbytes in (4 * xel, 4 * xel, 4 * bel, 4 * bel, 4 * tok * hk, 4 * hk, 4 * hk, 4 * hk, 4 * sel, 4 * xel, 4 * sel):
        off = al(al(off) + nbytes)
    assert L.ssd_prefill_workspace_size(b, l, h, p, n, g, q) == off


def test_forced_path_and_check_reject_before_any_hip_call():
    L = ssd.lib()
    args = [P0, P0, P0, P0, P0, None, None, 0, None, None, None, P0, BF, F, 1, 300, 4, 64, 64, 1, 64, 0, 0, 0, 0,
            P0, 1 << 30, None]
    assert L.ssd_prefill_forced(*args, 5, -1) == INV      # no such path
    assert L.ssd_prefill_forced(*args, -1, -1) == INV
    bad = list(args)
    bad[12] = 7                                            # bad dtype, any path
    assert L.ssd_prefill_forced(*bad, ssd.PATH_STAGED, -1) == INV
    assert L.ssd_prefill_check(None, 1 << 20, None) == WS
    assert L.ssd_prefill_check(P0 + 16, 1 << 20, None) == WS  # misaligned
    assert L.ssd_prefill_check(P0, 255, None) == WS           # smaller than the control block


def test_timed_prefill_rejects_before_any_hip_call():
    import ctypes
    L = ssd.lib()
    args = [P0, P0, P0, P0, P0, None, None, 0, None, None, None, P0, BF, F, 1, 300, 4, 64, 64, 1, 64, 0, 0, 0, 0,
            P0, 1 << 30, None, ssd.PATH_AUTO, -1]
    ev = (ctypes.c_void_p * 2)(P0, P0)
    null_in = (ctypes.c_void_p * 2)(P0, None)
    n = ctypes.c_int(-7)
    assert L.ssd_prefill_timed(*args, ev, ev, None, -1, ctypes.byref(n)) == INV   # negative capacity
    assert L.ssd_prefill_timed(*args, None, ev, None, 2, ctypes.byref(n)) == INV  # no start events
    assert L.ssd_prefill_timed(*args, ev, None, None, 2, ctypes.byref(n)) == INV  # no stop events
    assert L.ssd_prefill_timed(*args, ev, null_in, None, 2, ctypes.byref(n)) == INV  # a NULL event
    assert n.value == -7                                    # untouched by a rejected call
    bad = list(args)
    bad[-2] = 9                                             # no such path: the prefill's own check
    assert L.ssd_prefill_timed(*bad, ev, ev, None, 2, ctypes.byref(n)) == INV
    assert n.value == 0                                     # nothing launched


def _prefill(**kw):
    a = dict(x=P0, dt=P0, A=P0, B=P0, C=P0, D=None, h0=None, hT=None, y=P0, dtype=BF, batch=1, seqlen=300,
             nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64, ws=P0, wsb=1 << 30, stream=None)
    a.update(kw)
    return ssd.lib().ssd_prefill(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["h0"], a["hT"], a["y"],
                                 a["dtype"], a["batch"], a["seqlen"], a["nheads"], a["headdim"], a["dstate"],
                                 a["ngroups"], a["chunk"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), INV), (dict(batch=0), INV), (dict(seqlen=-1), INV), (dict(nheads=0), INV),
    (dict(nheads=6, ngroups=4), INV), (dict(headdim=40), UNS), (dict(headdim=272), UNS), (dict(dstate=8), UNS),
    (dict(dstate=272), UNS), (dict(headdim=0), INV), (dict(chunk=48), UNS), (dict(chunk=512), UNS), (dict(chunk=0), INV),
    (dict(batch=70000), UNS), (dict(x=None), INV), (dict(dt=None), INV), (dict(A=None), INV), (dict(B=None), INV),
    (dict(C=None), INV), (dict(y=None), INV), (dict(x=P0 + 2), INV), (dict(B=P0 + 8), INV), (dict(C=P0 + 4), INV),
    (dict(y=P0 + 4), INV), (dict(dt=P0 + 1), INV), (dict(h0=P0 + 4), INV), (dict(hT=P0 + 8), INV),
    (dict(D=P0 + 2), INV), (dict(ws=None), WS), (dict(wsb=1024), WS), (dict(ws=P0 + 128), WS),
])
def test_prefill_rejects_before_launch(kw, code):
    assert _prefill(**kw) == code


def test_step_rejects_before_launch():
    L = ssd.lib()
    def st(**kw):
        a = dict(state=P0, x=P0, dt=P0, A=P0, B=P0, C=P0, D=None, y=P0, dtype=BF, batch=2, nheads=4, headdim=64,
                 dstate=128, ngroups=1, stream=None)
        a.update(kw)
        return L.ssd_step(a["state"], a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["y"], a["dtype"], a["batch"],
                          a["nheads"], a["headdim"], a["dstate"], a["ngroups"], a["stream"])
    assert st(state=None) == INV
    assert st(state=P0 + 4) == INV
    assert st(x=None) == INV
    assert st(y=None) == INV
    assert st(dtype=3) == INV
    assert st(headdim=40) == UNS
    assert st(dstate=40) == UNS
    assert st(dstate=272) == UNS
    assert st(nheads=3, ngroups=2) == INV
    assert st(batch=0) == INV
    assert st(x=P0 + 1) == INV


def test_option_entry_points_reject_before_launch():
    L = ssd.lib()
    base = dict(x=P0, dt=P0, A=P0, B=P0, C=P0, D=None, bias=None, sp=1, z=None, h0=None, hT=None, y=P0, dtype=BF,
                ydtype=F, batch=1, seqlen=300, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64, ws=P0,
                wsb=1 << 30, stream=None)

    def pf(**kw):
        a = dict(base, **kw)
        return L.ssd_prefill_ex(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["bias"], a["sp"], a["z"],
                                a["h0"], a["hT"], a["y"], a["dtype"], a["ydtype"], a["batch"], a["seqlen"],
                                a["nheads"], a["headdim"], a["dstate"], a["ngroups"], a["chunk"], a["ws"],
                                a["wsb"], a["stream"])
    assert pf(ydtype=5) == INV                 # bad y dtype
    assert pf(dtype=5) == INV
    assert pf(bias=P0 + 2) == INV              # misaligned dt_bias
    assert pf(z=P0 + 1) == INV                 # misaligned z (bf16 needs 2-byte alignment)
    assert pf(chunk=48) == UNS
    assert pf(ws=None) == WS
    assert pf(dtype=F8, ws=None) == WS         # fp8 x, B, C with bf16 dt: accepted up to the workspace
    assert pf(dtype=F8, ydtype=F8) == INV      # y is never fp8
    assert pf(dtype=F8, x=P0 + 8, ws=None) == INV   # fp8 rows are read 16 bytes at a time
    assert pf(dtype=F8, dt=P0 + 1, ws=None) == INV  # dt beside fp8 inputs is bf16
    assert pf(dtype=F8, z=P0 + 1) == INV       # so is z
    assert pf(x=None) == INV
    assert pf(seqlen=0, y=None) == 0               # empty sequence, no final state: nothing to launch
    def st(**kw):
        a = dict(state=P0, x=P0, dt=P0, A=P0, B=P0, C=P0, D=None, bias=None, sp=0, z=None, y=P0, dtype=BF, ydtype=F,
                 batch=2, nheads=4, headdim=64, dstate=64, ngroups=1, stream=None)
        a.update(kw)
        return L.ssd_step_ex(a["state"], a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["bias"], a["sp"],
                             a["z"], a["y"], a["dtype"], a["ydtype"], a["batch"], a["nheads"], a["headdim"],
                             a["dstate"], a["ngroups"], a["stream"])
    assert st(ydtype=9) == INV
    assert st(y=None) == INV
    assert st(y=P0 + 2) == INV                 # fp32 y must be 4-byte aligned
    assert st(z=P0 + 1) == INV
    assert st(headdim=24) == UNS
    assert st(dtype=F8, ydtype=F8) == INV
    assert st(dtype=F8, dt=P0 + 1) == INV      # bf16 dt beside fp8 x, B, C


def test_strided_prefill_checks_token_strides_before_launch():
    """ssd_prefill_strided: strides below the dense row, rows not a whole number of 16 bytes,
    and chunks past 32-bit offsets are refused before anything is launched; accepted strides
    reach the workspace check (no workspace here)."""
    L = ssd.lib()
    base = dict(x=P0, dt=P0, A=P0, B=P0, C=P0, D=None, bias=None, sp=1, z=None, h0=None, hT=None, y=P0, dtype=BF,
                ydtype=F, batch=1, seqlen=300, nheads=4, headdim=64, dstate=64, ngroups=1, chunk=64,
                sx=0, sb=0, sd=0, sz=0, ws=None, wsb=1 << 30, stream=None)

    def pf(**kw):
        a = dict(base, **kw)
        return L.ssd_prefill_strided(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["bias"], a["sp"], a["z"],
                                     a["h0"], a["hT"], a["y"], a["dtype"], a["ydtype"], a["batch"], a["seqlen"],
                                     a["nheads"], a["headdim"], a["dstate"], a["ngroups"], a["chunk"], a["sx"],
                                     a["sb"], a["sd"], a["sz"], a["ws"], a["wsb"], a["stream"])
    assert pf() == WS                                   # all dense (0)
    assert pf(sx=256, sb=64, sd=4, sz=256) == WS        # the dense strides spelled out
    assert pf(sx=256 + 2 * 64 + 8, sb=256 + 2 * 64 + 8, sd=13, sz=1000) == WS  # wider token rows
    assert pf(sx=255) == INV                            # below H * P
    assert pf(sb=56) == INV                             # below G * N
    assert pf(sd=3) == INV                              # below H
    assert pf(sz=200) == INV                            # below H * P
    assert pf(sx=-256) == INV
    assert pf(sx=260) == INV                            # 520 bytes: not a multiple of 16
    assert pf(sb=68) == INV
    assert pf(dtype=F, sx=260) == WS                    # fp32: 1040 bytes
    assert pf(dtype=F, sx=258) == INV
    assert pf(dtype=F8, sx=272, sb=80) == WS            # fp8: rows of 272 and 80 bytes
    assert pf(dtype=F8, sx=264) == INV                  # 264 bytes: not a multiple of 16
    assert pf(dtype=F8, sb=72) == INV
    assert pf(sx=1 << 24) == UNS                        # 64 tokens x 2 bytes x 2^24 = 2^31 bytes per chunk
    assert pf(sd=1 << 24) == UNS
    assert L.ssd_prefill_ex(P0, P0, P0, P0, P0, None, None, 1, None, None, None, P0, BF, F, 1, 300, 4, 64, 64, 1, 64,
                            None, 1 << 30, None) == WS  # the dense call is the strided one with zeros


def test_strided_step_checks_batch_strides_before_launch():
    L = ssd.lib()

    def st(**kw):
        a = dict(state=P0, x=P0, dt=P0, A=P0, B=P0, C=P0, D=None, bias=None, sp=0, z=None, y=P0, dtype=BF, ydtype=F,
                 batch=2, nheads=4, headdim=64, dstate=64, ngroups=1, sx=0, sb=0, sd=0, sz=0, stream=None)
        a.update(kw)
        return L.ssd_step_strided(a["state"], a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["bias"], a["sp"],
                                  a["z"], a["y"], a["dtype"], a["ydtype"], a["batch"], a["nheads"], a["headdim"],
                                  a["dstate"], a["ngroups"], a["sx"], a["sb"], a["sd"], a["sz"], a["stream"])
    assert st(sx=255) == INV        # below H * P
    assert st(sb=63) == INV         # below G * N
    assert st(sd=3) == INV          # below H
    assert st(sz=255) == INV        # below H * P
    assert st(sx=-1) == INV
    assert st(sx=1 << 31) == UNS    # past 32-bit element offsets
    assert st(x=None, sx=300) == INV
    assert st(headdim=40, sx=300) == UNS


def test_decode_graph_rejects_before_capture():
    """ssd_decode_graph_create validates everything before any HIP call and leaves *out NULL."""
    import ctypes
    L = ssd.lib()

    def mk(**kw):
        a = dict(n=8, state=P0, x=P0, dt=P0, A=P0, B=P0, C=P0, D=None, bias=None, sp=0, z=None, y=P0, dtype=BF,
                 ydtype=F, batch=2, nheads=4, headdim=64, dstate=64, ngroups=1)
        a.update(kw)
        h = ctypes.c_void_p(P0)  # must come back NULL
        rc = L.ssd_decode_graph_create(ctypes.byref(h), a["n"], a["state"], a["x"], a["dt"], a["A"], a["B"], a["C"],
                                       a["D"], a["bias"], a["sp"], a["z"], a["y"], a["dtype"], a["ydtype"],
                                       a["batch"], a["nheads"], a["headdim"], a["dstate"], a["ngroups"])
        assert h.value is None, "handle must be NULL after a rejected create"
        return rc
    assert mk(n=0) == INV
    assert mk(n=65537) == INV                   # above SSD_DECODE_GRAPH_MAX_STEPS
    assert mk(state=None) == INV
    assert mk(state=P0 + 4) == INV              # the state needs 16-byte alignment
    assert mk(z=P0 + 1) == INV
    assert mk(ydtype=3) == INV
    assert mk(headdim=40) == UNS
    assert mk(nheads=6, ngroups=4) == INV
    assert L.ssd_decode_graph_create(None, 8, P0, P0, P0, P0, P0, P0, None, None, 0, None, P0, BF, F, 2, 4, 64, 64,
                                     1) == INV
    assert L.ssd_decode_graph_launch(None, None) == INV
    assert L.ssd_decode_graph_steps(None) == 0
    assert L.ssd_decode_graph_destroy(None) == 0
    m = re.search(r"#define SSD_DECODE_GRAPH_MAX_STEPS (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == 65536


def test_stage_entry_points_reject_before_launch():
    L = ssd.lib()
    assert L.ssd_chunk_cumsum(None, P0, P0, P0, BF, 1, 100, 4, 64, None) == INV
    assert L.ssd_chunk_cumsum(P0, P0, P0, P0, BF, 1, 100, 4, 100, None) == UNS
    assert L.ssd_chunk_cumsum(P0, P0, P0 + 4, P0, BF, 1, 100, 4, 64, None) == INV
    assert L.ssd_chunk_state(P0, P0, P0, P0, None, BF, 1, 100, 4, 64, 64, 1, 64, None) == INV
    assert L.ssd_chunk_state(P0, P0, P0, P0, P0, BF, 1, 100, 4, 64, 96, 1, 64, None) == UNS
    assert L.ssd_state_passing(None, P0, None, None, BF, 1, 4, 64, 64, 3, 64, None) == INV
    assert L.ssd_state_passing(P0, P0, None, None, BF, 1, 4, 64, 64, -1, 64, None) == INV
    assert L.ssd_state_passing(P0, P0, P0 + 4, None, F, 1, 4, 64, 64, 3, 64, None) == INV
    assert L.ssd_state_passing(P0, P0, None, None, 7, 1, 4, 64, 64, 3, 64, None) == INV   # bad state dtype
    assert L.ssd_chunk_gemm1(None, P0, P0, BF, 1, 100, 64, 1, 64, None) == INV
    assert L.ssd_chunk_gemm1(P0, P0, P0 + 4, BF, 1, 100, 64, 1, 64, None) == INV
    assert L.ssd_chunk_gemm1(P0, P0, P0, BF, 1, 100, 96, 1, 64, None) == UNS
    assert L.ssd_chunk_gemm1(P0, P0, P0, BF, 1, 100, 64, 1, 48, None) == UNS
    assert L.ssd_chunk_gemm1(P0, P0, P0, 7, 1, 100, 64, 1, 64, None) == INV
    assert L.ssd_chunk_gemm1(None, None, None, BF, 1, 0, 64, 1, 64, None) == 0   # empty sequence: no-op
    assert L.ssd_chunk_gemm1_size(1, 100, 1, 48) == 0
    assert L.ssd_chunk_scan(P0, P0, P0, P0, P0, None, None, P0, BF, 1, 100, 4, 64, 64, 1, 64, None) == INV
    assert L.ssd_chunk_scan(P0, P0, None, P0, P0, P0, None, P0, BF, 1, 100, 4, 64, 64, 1, 64, None) == INV
    assert L.ssd_chunk_scan(P0, P0, P0, P0, P0, P0, None, P0 + 4, BF, 1, 100, 4, 64, 64, 1, 64, None) == INV
    assert L.ssd_chunk_scan(P0, P0, P0, P0, P0, P0, None, P0, F, 1, 100, 4, 64, 64, 3, 64, None) == INV
    # ssd_chunk_scan_passing(x, C, cb, acum, dtc, states, init, final, D, y, sync, dtype, B, L, H, P, N, G, Q, s)
    sp = lambda *a: L.ssd_chunk_scan_passing(*a)
    assert sp(P0, P0, P0, P0, P0, None, None, None, None, P0, P0, BF, 1, 4096, 24, 64, 128, 1, 256, None) == INV
    assert sp(P0, P0, P0, P0, P0, P0, None, None, None, P0, None, BF, 1, 4096, 24, 64, 128, 1, 256, None) == INV
    assert sp(P0, P0, P0, P0, P0, P0, None, None, None, P0, P0 + 4, BF, 1, 4096, 24, 64, 128, 1, 256, None) == INV
    assert sp(P0, P0, P0, P0, P0, P0, P0 + 8, None, None, P0, P0, BF, 1, 4096, 24, 64, 128, 1, 256, None) == INV
    # shapes the one-round path does not take: fp32, another chunk length or headdim, > 16 chunks
    assert sp(P0, P0, P0, P0, P0, P0, None, None, None, P0, P0, F, 1, 4096, 24, 64, 128, 1, 256, None) == UNS
    assert sp(P0, P0, P0, P0, P0, P0, None, None, None, P0, P0, BF, 1, 4096, 24, 64, 128, 1, 128, None) == UNS
    assert sp(P0, P0, P0, P0, P0, P0, None, None, None, P0, P0, BF, 1, 4096, 24, 32, 128, 1, 256, None) == UNS
    assert sp(P0, P0, P0, P0, P0, P0, None, None, None, P0, P0, BF, 1, 4097, 24, 64, 128, 1, 256, None) == UNS


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The package never imports the oracle and has no CPU compute path."""
    pkg = os.path.join(ROOT, "mamba_ssd_scan_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.replace("Oracle", "").lower() or f == "synth.py", f
