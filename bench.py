"""Benchmark of the SSD layer core on one MI355X.

One step = one full chunked prefill (every prefill stage: cumulative decay, chunk states,
inter-chunk state passing, intra-chunk + off-diagonal output) over the Mamba-2-2.7B-shaped
long-context layer (batch 1, 16384 tokens, 80 heads, headdim 64, d_state 128, chunk 256,
bf16 inputs, fp32 state and output, random initial state), with inputs resident in HBM.
The timed steps run back to back, rotating over copies of the buffers that together span
over 1 GiB (4x the 256 MiB Infinity Cache), so that no step finds its data in that cache
from the step before; one marker pair brackets the block.  Each step goes through
ssd_prefill_timed, which binds HIP events to every kernel launch itself (the kernel's own
start and end, no marker between launches): the per-kernel durations and the roofline come
from them.  The 130M- and 370M-shaped layers are timed the same way and reported under
"workloads"; the same 2.7B-shaped step with x, B and C stored as fp8 e4m3 under
"fp8_inputs"; the decode update (batch 64, 80 heads, 1024 tokens) under "decode".

Prints ONE JSON line.  The oracle (fp64 CPU recurrence) is timed on the host's cores on the
same workload as "cpu_baseline".
"""
from __future__ import annotations

import argparse
import dataclasses
import gc
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mamba_ssd_scan_amd import ssd, synth  # noqa: E402

METRIC = "SSD tokens/s + % roofline (prefill MFMA TFLOPS, decode-step HBM GB/s)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16/fp16 matrix, published
PREFILL_WORKLOAD = 3              # the headline step: the 2.7B-shaped 16384-token layer
EXTRA_WORKLOADS = (1, 2)          # also timed, each with its own roofline
DECODE_WORKLOAD = 4
PROFILE_DIR = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "chunk_scan_kernel": "ssd_chunk_scan.hip", "chunk_scan_pipe_kernel": "ssd_chunk_scan.hip",
    "chunk_state_kernel": "ssd_chunk_state.hip",
    "state_passing_kernel": "ssd_state_passing.hip", "chunk_cumsum_kernel": "ssd_cumsum.hip",
    "step_kernel": "ssd_step.hip", "step_heads_kernel": "ssd_step.hip", "chunk_gemm1_kernel": "ssd_chunk_gemm1.hip",
    "chunk_scan_small_kernel": "ssd_chunk_scan_small.hip", "chunk_state_pair_kernel": "ssd_chunk_state_pair.hip",
    "chunk_fused_kernel": "ssd_prefill_fused.hip", "fused_prep_kernel": "ssd_prefill_fused.hip",
}


def scan_kernel_name(s, ncu=None) -> str:
    """The chunk-scan kernel the library launches for this shape: the one-round kernel when
    every (b, h, chunk) item fits at two per compute unit (bf16 or fp8, 256-token chunks,
    P = 64), else the pipelined persistent one (bf16 or fp8, 256-token chunks, P = 64, N = 128) or the
    persistent one (the same rule as the library's launcher).  ncu: compute units (default:
    the current device's)."""
    if ncu is None:
        import torch
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
    nitems = s.batch * s.nheads * -(-s.seqlen // s.chunk)
    small = s.dtype in ("bf16", "fp8") and s.chunk == 256 and s.headdim == 64 and nitems <= 2 * ncu
    if small:
        return "chunk_scan_small_kernel"
    pipe = s.dtype in ("bf16", "fp8") and s.chunk == 256 and s.headdim == 64 and s.dstate == 128
    return "chunk_scan_pipe_kernel" if pipe else "chunk_scan_kernel"


def passing_in_scan(s, ncu=None) -> bool:
    """Whether ssd_prefill runs Step-3 inside the one-round chunk scan (two launches): the
    one-round kernel's shapes with at most 16 chunks (the same rule as the library)."""
    return scan_kernel_name(s, ncu) == "chunk_scan_small_kernel" and -(-s.seqlen // s.chunk) <= 16


def chunk_state_pair(s) -> bool:
    """Whether ssd_prefill's first launch (cumulative decay, chunk states and GEMM1) takes two
    heads of a group per workgroup: bf16 or fp8, 256-token chunks, P = 64 and an even number of heads
    per group (the same rule as the library)."""
    return s.dtype in ("bf16", "fp8") and s.chunk == 256 and s.headdim == 64 and (s.nheads // s.ngroups) % 2 == 0


def step_kernels(s, ncu=None) -> list:
    """The kernels one ssd_prefill launches, in order.  The first is the fused launch
    (cumulative decay + chunk states + GEMM1): chunk_state_pair_kernel, or chunk_state_kernel's
    fused instantiation."""
    first = "chunk_state_pair_kernel" if chunk_state_pair(s) else "chunk_state_kernel"
    if passing_in_scan(s, ncu):
        return [first, "chunk_scan_small_kernel"]
    return [first, "state_passing_kernel", scan_kernel_name(s, ncu)]


# ---------------------------------------------------------------------------- algorithmic work

def alg_counts(s: synth.PrefillShape, ncu=None) -> dict:
    """Algorithmic bytes and flops per launch of each prefill kernel.

    Bytes: every tensor a kernel must read or write, once.  Flops: the
    causal triangle of the intra-chunk products is counted (Q(Q+1)/2 pairs per
    chunk), C.B^T once per group, multiply-add = 2 flops.
    """
    B, L, H, P, N, G, Q = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk
    ib = {"bf16": 2, "fp8": 1, "f32": 4}[s.dtype]   # x, B and C
    db = 4 if s.dtype == "f32" else 2               # dt (bf16 beside fp8 inputs)
    hb = 4 if s.dtype == "f32" else 2               # intermediates: fp16 for bf16 and fp8 inputs
    nc = -(-L // Q)
    x = B * L * H * P * ib
    dt = B * L * H * db
    bc = B * L * G * N * ib            # one of B or C
    y = B * L * H * P * 4
    chunk_tab = 2 * B * H * nc * Q * 4  # dA_cum + dt regrouped per chunk
    states = B * H * nc * P * N * hb   # chunk / entering states
    hen = states
    st = B * H * P * N * 4
    h0 = st if s.init_state != "zero" else 0
    tri = Q * (Q + 1)                  # 2 flops x Q(Q+1)/2 pairs
    # C.B^T products as the GEMM1 kernel stores them: per (b, g, chunk), 512 values per
    # 32-column step of each 16-row tile (the steps on or below the diagonal), fp16 for
    # bf16 and fp8 inputs and fp32 for fp32 inputs
    cb = B * G * nc * sum(t // 2 + 1 for t in range(Q // 16)) * 512 * hb
    k = {
        "chunk_cumsum_kernel": dict(bytes=dt + chunk_tab, flops=2 * B * L * H),
        "chunk_state_kernel": dict(bytes=x + bc + chunk_tab + states, flops=2 * B * H * L * P * N),
        "state_passing_kernel": dict(bytes=2 * states + B * H * nc * 4 + h0 + st, flops=2 * B * H * nc * P * N),
        "chunk_gemm1_kernel": dict(bytes=2 * bc + cb, flops=B * nc * G * N * tri),
        "chunk_scan_kernel": dict(bytes=x + bc + cb + chunk_tab + hen + y,
                                  flops=B * nc * H * P * tri + 2 * B * H * L * P * N),
    }
    k["chunk_scan_small_kernel"] = dict(k["chunk_scan_kernel"])
    k["chunk_scan_pipe_kernel"] = dict(k["chunk_scan_kernel"])
    # the prefill's fused first launch: dt in, dA_cum / dt_c and the chunk states out, and
    # the GEMM1 products (B and C in, cb out); x and B are read once
    k["chunk_state_pair_kernel"] = dict(bytes=x + dt + 2 * bc + chunk_tab + states + cb,
                                        flops=2 * B * H * L * P * N + B * nc * G * N * tri + 2 * B * L * H)
    if passing_in_scan(s, ncu):
        # Step-3 inside the chunk scan: the chunk states, the initial and the final state
        # instead of the entering states (which it writes and reads back itself)
        k["chunk_scan_small_kernel"] = dict(bytes=x + bc + cb + chunk_tab + states + h0 + st + y,
                                            flops=k["chunk_scan_kernel"]["flops"] + 2 * B * H * nc * P * N)
    fused_bytes = x + dt + 2 * bc + y + st + h0
    fused_flops = B * nc * (G * N * tri + H * P * tri) + 4 * B * H * L * P * N
    # the method's own tensors each kernel reads or writes (inputs, y, the initial and final
    # states), without the intermediates of this implementation (decay tables, chunk and
    # entering states, GEMM1 products): what a kernel would move if nothing else existed
    method = {
        "chunk_cumsum_kernel": dt,
        "chunk_state_kernel": x + bc,
        "chunk_state_pair_kernel": x + dt + 2 * bc,
        "state_passing_kernel": h0 + st,
        "chunk_gemm1_kernel": 2 * bc,
        "chunk_scan_kernel": x + bc + y,
        "chunk_scan_pipe_kernel": x + bc + y,
        "chunk_scan_small_kernel": x + bc + y + (h0 + st if passing_in_scan(s, ncu) else 0),
    }
    for name, b in method.items():
        k[name]["method_bytes"] = b
    return dict(kernels=k, fused_bytes=fused_bytes, fused_flops=fused_flops)


def decode_bytes_per_step(s: synth.DecodeShape) -> int:
    ib = 2 if s.dtype == "bf16" else 4
    B, H, P, N, G = s.batch, s.nheads, s.headdim, s.dstate, s.ngroups
    return 2 * B * H * P * N * 4 + B * H * P * ib + B * H * ib + 2 * B * G * N * ib + B * H * P * 4


def source_hash(kernel: str) -> str:
    """Hash of the kernel's source file and the shared device header."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "ssd_common.h"):
        h.update(open(os.path.join(ROOT, "mamba_ssd_scan_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_summary(path: str) -> dict:
    """`key: value` lines of a profile summary (other lines ignored)."""
    out = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#", "|")):
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None.

    The summary is used only if it was taken on the current kernel source.
    """
    path = os.path.join(PROFILE_DIR, f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    try:
        d = read_summary(path)
        if d.get("source_sha256_16") != source_hash(kernel):
            return None
        return float(d["hbm_bytes_per_launch"])
    except (OSError, ValueError, KeyError):
        return None


# ---------------------------------------------------------------------------- GPU timing

class Flusher:
    """Evicts the Infinity Cache (256 MiB) and the L2s with a 512 MiB read."""

    def __init__(self, torch, mib=512):
        self.buf = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.zeros(1, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.sink += self.buf.sum()


def settle_clocks(torch, flush, seconds=0.3):
    """Untimed eviction reads for a fixed time, so that the timed work does not start
    while the GPU is still raising its clocks after the set-up (inputs, buffers)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            flush()
        torch.cuda.synchronize()


CACHE_SPAN = 1 << 30  # bytes a rotation of buffer sets spans: 4x the 256 MiB Infinity Cache


def lead_flushes(torch, flush, host_us, steps):
    """Evictions to queue ahead of a timed block so that the host, which enqueues the block's
    calls at ``host_us`` each, stays ahead of the GPU for all ``steps`` of them (an interval
    also counts any time the GPU waits for the host)."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    flush()
    b.record()
    torch.cuda.synchronize()
    per = max(a.elapsed_time(b) * 1e3, 1.0)
    return int(min(400, max(8, 2.0 * steps * host_us / per)))


def host_us_per_call(torch, fn, n=8):
    """Host time to enqueue one call of fn (mean of n, after one untimed call)."""
    fn()
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    us = (time.perf_counter() - t0) * 1e6 / n
    torch.cuda.synchronize()
    return us


def time_block(torch, fns, steps, flush):
    """Mean time (us) of ``steps`` calls in a row, fns[k % len(fns)](), between one marker
    pair: the step time of a caller that runs them back to back.  Evictions queued before the
    block keep the host ahead; Python's garbage collector is off during the block."""
    k = [0]

    def one():
        fns[k[0] % len(fns)]()
        k[0] += 1
    lead = lead_flushes(torch, flush, host_us_per_call(torch, one), steps)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gc_on = gc.isenabled()
    gc.disable()
    try:
        torch.cuda.synchronize()
        for _ in range(lead):
            flush()
        a.record(stream)
        for _ in range(steps):
            one()
        b.record(stream)
        torch.cuda.synchronize()
    finally:
        if gc_on:
            gc.enable()
    return a.elapsed_time(b) * 1e3 / steps


def time_steps(torch, calls, steps, flush, pairs=8):
    """``steps`` prefills in a row, calls[k % len(calls)](events_k), each through
    ssd_prefill_timed: every kernel launch is bound to an event pair of its own (HIP's
    launch-with-events extension, the kernel's own start and end), so the kernels'
    durations and the gaps between them are read with no marker between launches.  One
    marker pair brackets the block; block / steps is the step time back to back.

    Returns the block's step time, each step's span (first kernel's start to last kernel's
    end), per launch position its kernel name and durations, and the gaps inside a step
    and between steps (us)."""
    evs = [ssd.LaunchEvents(pairs) for _ in range(steps)]
    k = [0]

    def one(ev=None):
        calls[k[0] % len(calls)](ev if ev is not None else evs[0])
        k[0] += 1
    lead = lead_flushes(torch, flush, host_us_per_call(torch, one), steps)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gc_on = gc.isenabled()
    gc.disable()
    try:
        torch.cuda.synchronize()
        k[0] = 0
        t0 = time.perf_counter()
        for _ in range(lead):
            flush()
        a.record(stream)
        for i in range(steps):
            one(evs[i])
        b.record(stream)
        host = time.perf_counter() - t0
        torch.cuda.synchronize()
    finally:
        if gc_on:
            gc.enable()
    n = len(evs[0].names)
    names = evs[0].names
    if any(e.names != names for e in evs):
        raise RuntimeError("the timed steps did not all make the same launches")
    per = [e.durations_ms() for e in evs]
    dur = [[p[j] * 1e3 for p in per] for j in range(n)]
    span = [e.span_ms() * 1e3 for e in evs]
    inner = [sum(e.gaps_ms()) * 1e3 for e in evs]
    between = [evs[i + 1].since_ms(evs[i]) * 1e3 for i in range(steps - 1)]
    return {"block_us_per_step": a.elapsed_time(b) * 1e3 / steps, "span_us": span, "names": names,
            "launch_us": dur, "gaps_in_step_us": inner, "gaps_between_steps_us": between,
            "host_enqueue_us_per_step": host * 1e6 / steps, "lead_evictions": lead}


def stats(v):
    v = sorted(v)
    return {"mean": sum(v) / len(v), "median": v[len(v) // 2], "min": v[0], "max": v[-1]}


def launch_cold(torch, fn, n, flush, before=None):
    """Profiling aid: n launches of fn, each after a 512 MiB eviction (nothing timed)."""
    for _ in range(n):
        if before is not None:
            before()
        flush()
        fn()
    torch.cuda.synchronize()


def prefill_buffers(torch, s, inp):
    g = {k: synth.to_torch(inp[k], s.dtype) for k in ("x", "B", "C")}
    g["dt"] = synth.to_torch(inp["dt"], synth.dt_dtype(s.dtype))
    g["A"] = torch.from_numpy(inp["A"]).cuda()
    g["D"] = torch.from_numpy(inp["D"]).cuda()
    g["h0"] = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).cuda()
    nc = -(-s.seqlen // s.chunk)
    g["y"] = torch.empty((s.batch, s.seqlen, s.nheads, s.headdim), dtype=torch.float32, device="cuda")
    g["final"] = torch.empty((s.batch, s.nheads, s.headdim, s.dstate), dtype=torch.float32, device="cuda")
    g["ws"] = ssd.alloc_workspace(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk)
    g["acum"] = torch.empty((s.batch, s.nheads, nc, s.chunk), dtype=torch.float32, device="cuda")
    g["dtc"] = torch.empty_like(g["acum"])
    # chunk states, then (in place) entering states: fp16 for bf16 inputs, fp32 otherwise
    g["states"] = torch.empty((s.batch, s.nheads, nc, s.headdim, s.dstate),
                              dtype=torch.float32 if s.dtype == "f32" else torch.float16, device="cuda")
    g["hen"] = g["states"]
    g["cb"] = torch.empty(ssd.chunk_gemm1_size(s.batch, s.seqlen, s.ngroups, s.chunk) // 4, dtype=torch.float32,
                          device="cuda")
    return g


def run_prefill(g, s):
    ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=s.chunk, y=g["y"],
                final_state=g["final"], workspace=g["ws"])


def plain_prefill(g, s, **kw):
    """The prefill with options (prefill_ex; a path through ssd_prefill_forced), untimed."""
    def run():
        ssd.prefill_ex(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=s.chunk,
                       y=g.get("y_out", g["y"]), final_state=g["final"], workspace=g["ws"], **kw)
    return run


def timed_prefill(g, s, **kw):
    """The same prefill through ssd_prefill_timed (every launch bound to an event pair)."""
    def run(ev):
        ssd.prefill_timed(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], events=ev, chunk=s.chunk,
                          y=g.get("y_out", g["y"]), final_state=g["final"], workspace=g["ws"], **kw)
    return run


def rotation(torch, g, s):
    """Buffer sets to rotate over: copies of the workload's inputs (same values, other
    addresses) with outputs and a workspace of their own, as many as span CACHE_SPAN bytes
    together (at least one), so that a step does not find its data in the Infinity Cache
    from the steps just before it."""
    per = alg_counts(s)["fused_bytes"] + g["ws"].numel() * g["ws"].element_size()
    r = max(1, min(32, -(-CACHE_SPAN // per)))
    sets = []
    for i in range(r):
        h = dict(g)
        if i:
            for k in ("x", "dt", "B", "C"):
                h[k] = g[k].clone()
            h["h0"] = None if g["h0"] is None else g["h0"].clone()
            h["y"], h["final"], h["ws"] = (torch.empty_like(g["y"]), torch.empty_like(g["final"]),
                                           torch.empty_like(g["ws"]))
        sets.append(h)
    return sets


def stage_fns(torch, g, s):
    """The launches of the prefill for this input type, each callable on its own."""
    Q = s.chunk
    pristine = {}

    def cumsum():
        ssd.chunk_cumsum(g["dt"], g["A"], chunk=Q, acum=g["acum"], dtc=g["dtc"])

    def cstate():
        ssd.chunk_state(g["x"], g["B"], g["acum"], g["dtc"], chunk=Q, states=g["states"])

    def passing():
        ssd.state_passing(g["states"], g["acum"], g["h0"], chunk=Q, final_state=g["final"])

    def restore_states():  # state passing works in place: restart from the chunk states every launch
        g["states"].copy_(pristine["states"])

    def gemm1():
        ssd.chunk_gemm1(g["B"], g["C"], chunk=Q, cb=g["cb"])

    def scan():
        ssd.chunk_scan(g["x"], g["C"], g["cb"], g["acum"], g["dtc"], g["hen"], g["D"], chunk=Q, y=g["y"])

    def scan_passing():
        ssd.chunk_scan_passing(g["x"], g["C"], g["cb"], g["acum"], g["dtc"], g["states"], g["sync"], g["D"],
                               g["h0"], chunk=Q, y=g["y"], final_state=g["final"])

    def restore_states_and_counters():  # Step-3 in the scan works in place on zeroed counters
        g["states"].copy_(pristine["states"])
        g["sync"].zero_()

    cumsum()
    cstate()
    torch.cuda.synchronize()
    pristine["states"] = g["states"].clone()
    passing()
    gemm1()
    torch.cuda.synchronize()
    out = {"chunk_cumsum_kernel": (cumsum, None), "chunk_state_kernel": (cstate, None),
           "state_passing_kernel": (passing, restore_states), "chunk_gemm1_kernel": (gemm1, None),
           scan_kernel_name(s): (scan, None)}
    if passing_in_scan(s):
        g["sync"] = ssd.alloc_sync(s.batch, s.nheads)
        out["chunk_scan_small_kernel"] = (scan_passing, restore_states_and_counters)
    return out


# ---------------------------------------------------------------------------- CPU baseline

def cpu_baseline(s, inp, min_seconds=10.0, max_reps=2000):
    from oracle import ref  # the oracle: test infrastructure, timed here as the CPU baseline
    # every core this process may run on, within the host's share for this GPU when the
    # environment states one (OMP_NUM_THREADS)
    cores = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit() and int(os.environ["OMP_NUM_THREADS"]) > 0:
        cores = min(cores, int(os.environ["OMP_NUM_THREADS"]))
    f64 = {k: (None if inp[k] is None else np.ascontiguousarray(inp[k], np.float64))
           for k in ("x", "dt", "A", "B", "C", "D", "h0")}
    ref.load()
    times = []
    while len(times) < max_reps and (sum(times) < min_seconds or not times):
        t0 = time.perf_counter()
        ref.prefill(f64["x"], f64["dt"], f64["A"], f64["B"], f64["C"], f64["D"], f64["h0"], nthreads=cores)
        times.append(time.perf_counter() - t0)
    tokens = s.batch * s.seqlen
    med = sorted(times)[len(times) // 2]
    return {"value": tokens / med, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "mean_tokens_per_s": tokens * len(times) / sum(times),
            "sample": f"the full workload ({s.batch}x{s.seqlen} tokens, all {s.nheads} heads), fp64 sequential "
                      f"recurrence, repeated {len(times)}x ({sum(times):.1f} s); value: the median repetition"}


# ---------------------------------------------------------------------------- decode

def bench_decode(torch, steps, flush):
    s = synth.WORKLOADS[DECODE_WORKLOAD]
    inp = synth.decode_inputs(s, synth.SEED_BASE + DECODE_WORKLOAD, steps=steps)
    xs, dts = synth.to_torch(inp["x"], s.dtype), synth.to_torch(inp["dt"], s.dtype)
    Bs, Cs = synth.to_torch(inp["B"], s.dtype), synth.to_torch(inp["C"], s.dtype)
    del inp["x"]
    A = torch.from_numpy(inp["A"]).cuda()
    D = torch.from_numpy(inp["D"]).cuda()
    state = torch.from_numpy(inp["state"]).cuda()
    y = torch.empty((s.batch, s.nheads, s.headdim), dtype=torch.float32, device="cuda")
    for t in range(min(8, steps)):  # warm-up
        ssd.step(state, xs[t], dts[t], A, Bs[t], Cs[t], D, y=y)
    torch.cuda.synchronize()
    # the timed tokens: back to back, each batch of sequences on a state of its own, rotating
    # over as many states as span CACHE_SPAN bytes (a step does not find its state in the
    # Infinity Cache from the step before)
    nst = max(1, -(-CACHE_SPAN // (state.numel() * 4)))
    states = [state] + [state.clone() for _ in range(nst - 1)]
    k = [0]

    def one():
        t = k[0] % steps
        ssd.step(states[k[0] % nst], xs[t], dts[t], A, Bs[t], Cs[t], D, y=y)
        k[0] += 1
    us_loop = time_block(torch, [one], steps, flush)
    # one state carried through every token (it can stay in the Infinity Cache between steps)
    k2 = [0]

    def same():
        t = k2[0] % steps
        ssd.step(state, xs[t], dts[t], A, Bs[t], Cs[t], D, y=y)
        k2[0] += 1
    us_same = time_block(torch, [same], steps, flush)
    del states[1:]
    # the same tokens as one HIP graph (ssd_decode_graph): one launch for all of them
    y_all = torch.empty((steps, s.batch, s.nheads, s.headdim), dtype=torch.float32, device="cuda")
    graph = ssd.DecodeGraph(state, xs, dts, A, Bs, Cs, D, y=y_all)
    graph.launch()
    torch.cuda.synchronize()
    us_graph = time_block(torch, [graph.launch], 3, flush) / steps
    graph.close()
    nbytes = decode_bytes_per_step(s)
    # the batch-64 x 80-head step runs one workgroup per head (step_heads_kernel)
    traffic = counter_traffic("step_heads_kernel", synth.WORKLOAD_NAMES[DECODE_WORKLOAD])
    return {
        "counter_traffic_bytes_per_step": traffic,
        "workload": synth.WORKLOAD_NAMES[DECODE_WORKLOAD], "steps": steps,
        "us_per_step": us_loop, "tokens_per_s": s.batch / (us_loop * 1e-6),
        "alg_bytes_per_step": nbytes, "gbps": nbytes / (us_loop * 1e-6) / 1e9,
        "hbm_frac": nbytes / (us_loop * 1e-6) / 1e9 / HBM_PEAK_GBS, "states_rotated": nst,
        "one_state_us_per_step": us_same, "one_state_gbps": nbytes / (us_same * 1e-6) / 1e9,
        "graph_us_per_step": us_graph, "graph_gbps": nbytes / (us_graph * 1e-6) / 1e9,
        "note": f"us_per_step: {steps} back-to-back ssd_step launches rotating over {nst} states (each "
                f"{state.numel() * 4 / 1e6:.0f} MB); one_state: the same launches on one state (it can stay in "
                "the 256 MiB Infinity Cache between steps); graph: the tokens as one ssd_decode_graph launch "
                "on one state (per-token outputs in their own slots)",
    }


def bench_layer_rows(torch, s, g, flush, steps):
    """The prefill with its inputs where a Mamba-2 layer holds them: x, B and C in the
    convolved [x | B | C] rows, dt in the input-projection [z | x | B | C | dt] rows.
    Read in place through token strides, against copying the four inputs out to dense
    tensors first (what a dense-only call needs)."""
    B, L, H, P, N, G = s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups
    hp, gn = H * P, G * N
    xbc = torch.empty((B, L, hp + 2 * gn), dtype=g["x"].dtype, device="cuda")
    zin = torch.empty((B, L, 2 * hp + 2 * gn + H), dtype=g["x"].dtype, device="cuda")
    xbc[..., :hp] = g["x"].reshape(B, L, hp)
    xbc[..., hp:hp + gn] = g["B"].reshape(B, L, gn)
    xbc[..., hp + gn:] = g["C"].reshape(B, L, gn)
    zin[..., 2 * hp + 2 * gn:] = g["dt"]
    v = dict(x=xbc[..., :hp].unflatten(-1, (H, P)), B=xbc[..., hp:hp + gn].unflatten(-1, (G, N)),
             C=xbc[..., hp + gn:].unflatten(-1, (G, N)), dt=zin[..., 2 * hp + 2 * gn:])
    ws = g["ws"]

    def in_place():
        ssd.prefill(v["x"], v["dt"], g["A"], v["B"], v["C"], g["D"], g["h0"], chunk=s.chunk, y=g["y"],
                    final_state=g["final"], workspace=ws)

    def copied():
        ssd.prefill(v["x"].contiguous(), v["dt"].contiguous(), g["A"], v["B"].contiguous(), v["C"].contiguous(),
                    g["D"], g["h0"], chunk=s.chunk, y=g["y"], final_state=g["final"], workspace=ws)
    for _ in range(3):
        in_place()
        copied()
    torch.cuda.synchronize()
    us_in = time_block(torch, [in_place], steps, flush)
    us_cp = time_block(torch, [copied], steps, flush)
    return {"in_place_us": us_in, "copy_then_dense_us": us_cp,
            "rows": f"x|B|C rows of {hp + 2 * gn} and z|x|B|C|dt rows of {2 * hp + 2 * gn + H} elements",
            "note": "back to back on one set of rows (a step's data exceeds the Infinity Cache); the copies "
                    "are torch's, outside the library"}


def bench_cached_vs_recompute(torch, flush, context=4096, ntok=256, reps=20):
    """Per generated token at a ``context``-token context, batch 1, for the five Mamba-2 shapes:
    cached decode (the state carried over; ``ntok`` tokens as one decode graph, and as eager
    ssd_step launches) against full-prefix recomputation (an ssd_prefill over context + 1 tokens,
    whose last output is the new token's).  Both warm, back to back."""
    out = {}
    for name, H in synth.MAMBA2_LADDER.items():
        s = synth.PrefillShape(1, context + 1, H, 64, 128, 1, 256, "bf16")
        inp = synth.prefill_inputs(s, synth.SEED_BASE + 100 + H)
        g = prefill_buffers(torch, s, inp)
        run_prefill(g, s)
        torch.cuda.synchronize()
        us_re = time_block(torch, [lambda: run_prefill(g, s)], reps, flush)
        ds = synth.DecodeShape(1, H, 64, 128, 1, ntok, "bf16")
        dinp = synth.decode_inputs(ds, synth.SEED_BASE + 200 + H)
        xs, dts = synth.to_torch(dinp["x"], "bf16"), synth.to_torch(dinp["dt"], "bf16")
        Bs, Cs = synth.to_torch(dinp["B"], "bf16"), synth.to_torch(dinp["C"], "bf16")
        state = g["final"].clone()  # the cached state after the prefix
        graph = ssd.DecodeGraph(state, xs, dts, g["A"], Bs, Cs, g["D"])
        graph.launch()
        torch.cuda.synchronize()
        us_graph = time_block(torch, [graph.launch], max(2, reps // 4), flush) / ntok
        graph.close()
        y1 = torch.empty((1, H, 64), dtype=torch.float32, device="cuda")
        k = [0]

        def eager():
            t = k[0] % ntok
            k[0] += 1
            ssd.step(state, xs[t], dts[t], g["A"], Bs[t], Cs[t], g["D"], y=y1)
        eager()
        torch.cuda.synchronize()
        us_eager = time_block(torch, [eager], ntok, flush)
        out[name] = {"nheads": H, "recompute_us": us_re, "cached_graph_us": us_graph, "cached_eager_us": us_eager,
                     "speedup_graph": us_re / us_graph, "speedup_eager": us_re / us_eager}
        del g, xs, dts, Bs, Cs, state
    return {"context": context, "batch": 1, "headdim": 64, "dstate": 128, "chunk": 256, "dtype": "bf16",
            "tokens_per_graph": ntok, "models": out,
            "note": "SSD layer core only (one layer, no projections): per-token time of cached decode vs an "
                    "ssd_prefill over the whole prefix plus the token; warm, back-to-back launches"}


# ---------------------------------------------------------------------------- main

def launch_counts(counts, j, name):
    """Algorithmic counts of launch j of a prefill: the first launch of the three- and two-launch
    paths is the fused one (cumulative decay, chunk states and GEMM1, counted under
    chunk_state_pair_kernel whichever instantiation runs it)."""
    if j == 0 and name in ("chunk_state_pair_kernel", "chunk_state_kernel"):
        return counts["kernels"]["chunk_state_pair_kernel"]
    return counts["kernels"].get(name)


def launch_table(t, counts):
    """Per launch position of a time_steps result: the kernel, its durations and its rates."""
    out = []
    for j, name in enumerate(t["names"]):
        st = stats(t["launch_us"][j])
        r = {"kernel": name, "us": st["mean"], "us_median": st["median"], "us_min": st["min"], "us_max": st["max"]}
        c = launch_counts(counts, j, name)
        if c is not None:
            sec = st["mean"] * 1e-6
            r.update({"method_bytes": c["method_bytes"], "alg_bytes_incl_intermediates": c["bytes"],
                      "alg_flops": c["flops"], "method_gbps": c["method_bytes"] / sec / 1e9,
                      "hbm_frac_method_bytes": c["method_bytes"] / sec / 1e9 / HBM_PEAK_GBS,
                      "tflops": c["flops"] / sec / 1e12})
        out.append(r)
    return out


def step_summary(us, t, s, counts):
    """The step figures: ``us`` per step of the plain block, the launches of a time_steps result."""
    tokens = s.batch * s.seqlen
    launches = launch_table(t, counts)
    fb, ff = counts["fused_bytes"], counts["fused_flops"]
    sp = stats(t["span_us"])
    return {
        "us_per_step": us, "tokens_per_s": tokens / (us * 1e-6),
        "timed_launch_us_per_step": t["block_us_per_step"],
        "span_us_mean": sp["mean"], "span_us_median": sp["median"], "span_us_min": sp["min"],
        "kernel_us_sum": sum(r["us"] for r in launches),
        "gaps_in_step_us": stats(t["gaps_in_step_us"])["mean"],
        "gap_between_steps_us": stats(t["gaps_between_steps_us"])["mean"] if t["gaps_between_steps_us"] else None,
        "gap_between_steps_us_max": max(t["gaps_between_steps_us"]) if t["gaps_between_steps_us"] else None,
        "host_enqueue_us_per_step": t["host_enqueue_us_per_step"], "lead_evictions": t["lead_evictions"],
        "method_bytes": fb, "alg_flops": ff,
        "method_gbps": fb / (us * 1e-6) / 1e9, "hbm_frac_method_bytes": fb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "alg_tflops": ff / (us * 1e-6) / 1e12, "alg_mfma_frac": ff / (us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "hbm_floor_us": fb / (HBM_PEAK_GBS * 1e9) * 1e6,
        "launches": launches,
    }


def roofline_of(step, s, wl):
    """The roofline object of a step: its longest launch, on the method's own bytes."""
    d = max((r for r in step["launches"] if "method_bytes" in r), key=lambda r: r["us"])
    dom = d["kernel"]
    return {"bound": "hbm", "achieved": d["method_gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": d["method_gbps"] / HBM_PEAK_GBS, "traffic": counter_traffic(dom, synth.WORKLOAD_NAMES[wl]),
            "kernel": dom,
            "variant": ("with Step-3 inside (two-launch prefill)" if dom == "chunk_scan_small_kernel"
                        and passing_in_scan(s) else "as ssd_prefill launches it"),
            "us_per_launch": d["us"], "us_per_launch_median": d["us_median"],
            "timing": "HIP events bound to the kernel's own launch in each timed step (ssd_prefill_timed), "
                      "mean over the steps",
            "method_bytes_per_launch": d["method_bytes"],
            "alg_bytes_incl_intermediates_per_launch": d["alg_bytes_incl_intermediates"],
            "alg_flops_per_launch": d["alg_flops"], "mfma_tflops": d["tflops"],
            "mfma_frac": d["tflops"] / MFMA_BF16_PEAK_TFLOPS,
            "intensity_flop_per_method_byte": d["alg_flops"] / d["method_bytes"]}


def bench_prefill_workload(torch, wl, steps, warmup, flush, dtype=None):
    """Timed prefill steps of one workload, every launch timed, and its roofline.

    The timed region is ``steps`` prefills back to back over a rotation of buffer sets, each
    through ssd_prefill_timed.  ``dtype`` stores the inputs in another type (the same draw,
    rounded to it).  Returns (record, inputs, buffer sets, wall seconds of the timed region)."""
    s = synth.WORKLOADS[wl]
    if dtype is not None:
        s = dataclasses.replace(s, dtype=dtype)
    inp = synth.prefill_inputs(s, synth.SEED_BASE + wl)
    g = prefill_buffers(torch, s, inp)
    sets = rotation(torch, g, s)
    plain = [lambda h=h: run_prefill(h, s) for h in sets]
    calls = [timed_prefill(h, s) for h in sets]
    settle_clocks(torch, flush)
    ev = ssd.LaunchEvents(8)
    for i in range(max(warmup, len(sets))):
        plain[i % len(plain)]()
        calls[i % len(calls)](ev)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` steps through ssd_prefill, bracketed by synchronisations
    t_wall = time.perf_counter()
    us = time_block(torch, plain, steps, flush)
    wall = time.perf_counter() - t_wall
    # ---- the same steps through ssd_prefill_timed: every kernel's own duration.  Events bound
    # to a launch put a few microseconds of dispatch between kernels (the block's step time
    # shows it), not into the kernels.
    t = time_steps(torch, calls, steps, flush)
    counts = alg_counts(s)
    step = step_summary(us, t, s, counts)
    step["buffer_sets"] = len(sets)
    roof = roofline_of(step, s, wl)
    if dtype is not None:  # the committed counter summaries are of the workload's own input type
        roof["traffic"] = None
    # on one buffer set: what stays in the Infinity Cache between steps helps
    step["one_buffer_set_us_per_step"] = time_block(torch, [lambda: run_prefill(g, s)], steps, flush)
    # bf16 y (the fp32 result rounded once): halves the largest stream
    if s.dtype == "bf16":
        bsets = [dict(h, y_out=torch.empty(h["y"].shape, dtype=torch.bfloat16, device="cuda")) for h in sets]
        ub = time_block(torch, [plain_prefill(h, s, y_dtype=torch.bfloat16) for h in bsets], steps, flush)
        tb = time_steps(torch, [timed_prefill(h, s, y_dtype=torch.bfloat16) for h in bsets], steps, flush)
        bb = counts["fused_bytes"] - s.batch * s.seqlen * s.nheads * s.headdim * 2
        step["bf16_y"] = {"us_per_step": ub, "tokens_per_s": s.batch * s.seqlen / (ub * 1e-6), "method_bytes": bb,
                          "hbm_frac_method_bytes": bb / (ub * 1e-6) / 1e9 / HBM_PEAK_GBS,
                          "launches": [{"kernel": n, "us": stats(v)["mean"]} for n, v in zip(tb["names"], tb["launch_us"])]}
        del bsets
    rec = {"workload": synth.WORKLOAD_NAMES[wl], "value": step["tokens_per_s"], "unit": "tokens/s",
           "roofline": roof, "prefill": step}
    return rec, inp, sets, wall


def bench_single_pass(torch, wl, sets, steps, flush):
    """The single-pass prefill (only selected on request) on the same workload and buffers."""
    s = synth.WORKLOADS[wl]
    calls = [timed_prefill(h, s, path=ssd.PATH_SINGLE_PASS) for h in sets]
    try:
        calls[0](ssd.LaunchEvents(8))
    except ssd.SsdError:
        return None
    torch.cuda.synchronize()
    us = time_block(torch, [plain_prefill(h, s, path=ssd.PATH_SINGLE_PASS) for h in sets], steps, flush)
    t = time_steps(torch, calls, steps, flush)
    return {"us_per_step": us, "tokens_per_s": s.batch * s.seqlen / (us * 1e-6),
            "launches": [{"kernel": n, "us": stats(v)["mean"]} for n, v in zip(t["names"], t["launch_us"])],
            "note": "ssd_prefill_forced's SSD_PATH_SINGLE_PASS; the library's own path is the step above"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=PREFILL_WORKLOAD, choices=[0, 1, 2, 3],
                    help="prefill workload timed as the step (default 3; 1 and 2 are also reported)")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other prefill workloads")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-input variant of the step")
    ap.add_argument("--only", choices=["prefill", "chunk_scan_kernel", "chunk_scan_pipe_kernel", "chunk_state_kernel", "state_passing_kernel",
                                       "chunk_cumsum_kernel", "chunk_gemm1_kernel", "chunk_scan_small_kernel",
                                       "single_pass", "step", "cached", "copy"],
                    help="profiling aid: launch only this work --steps times, print nothing else (prefill and "
                         "single_pass: back to back over the rotating buffer sets, as timed; a stage kernel: "
                         "through its entry point, each launch after a cache eviction)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the SSD core here is a single-GPU "
              f"library and no multi-GPU path is built.", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    ssd.lib()
    flush = Flusher(torch)
    for _ in range(3):  # load the eviction's reduction kernel before anything is timed
        flush()
    torch.cuda.synchronize()
    s = synth.WORKLOADS[args.workload]
    wname = synth.WORKLOAD_NAMES[args.workload]

    if args.only == "copy":  # plain copy of known size, to scale HBM counters
        src = torch.ones(256 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            flush()
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 4, "copy_bytes_written": dst.numel() * 4,
                          "launches": args.steps}))
        return 0
    if args.only == "step":
        print(json.dumps(bench_decode(torch, args.decode_steps, flush)))
        return 0
    if args.only == "cached":
        print(json.dumps(bench_cached_vs_recompute(torch, flush)))
        return 0
    if args.only is not None:
        inp = synth.prefill_inputs(s, synth.SEED_BASE + args.workload)
        g = prefill_buffers(torch, s, inp)
        settle_clocks(torch, flush)
        for _ in range(args.warmup):
            run_prefill(g, s)
        torch.cuda.synchronize()
        if args.only in ("prefill", "single_pass"):
            path = ssd.PATH_SINGLE_PASS if args.only == "single_pass" else ssd.PATH_AUTO
            sets = rotation(torch, g, s)
            for i in range(args.steps):
                h = sets[i % len(sets)]
                ssd.prefill(h["x"], h["dt"], h["A"], h["B"], h["C"], h["D"], h["h0"], chunk=s.chunk, y=h["y"],
                            final_state=h["final"], workspace=h["ws"], path=path)
            torch.cuda.synchronize()
        else:
            fn, before = stage_fns(torch, g, s)[args.only]
            launch_cold(torch, fn, args.steps, flush, before)
        return 0

    rec, inp, sets, wall = bench_prefill_workload(torch, args.workload, args.steps, args.warmup, flush)
    us_step = rec["prefill"]["us_per_step"]
    out = {
        "metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us_step / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": s.dtype, "data": "synthetic",
        "config": {"workload": wname, "batch": s.batch, "seqlen": s.seqlen, "nheads": s.nheads,
                   "headdim": s.headdim, "dstate": s.dstate, "ngroups": s.ngroups, "chunk": s.chunk,
                   "initial_state": s.init_state,
                   "timing": f"{args.steps} steps back to back over {len(sets)} rotating buffer set(s) of "
                             f"the inputs, outputs and workspace (together over 1 GiB, 4x the Infinity Cache), "
                             f"one marker pair around the block; every kernel launch bound to HIP events of "
                             f"its own (ssd_prefill_timed)",
                   "parallelism": "single GPU"},
        "roofline": rec["roofline"],
        "prefill": rec["prefill"],
        "timed_wall_s": wall,
    }
    sp = bench_single_pass(torch, args.workload, sets, args.steps, flush)
    if sp is not None:
        out["single_pass"] = sp
    out["layer_rows"] = bench_layer_rows(torch, s, sets[0], flush, args.steps)
    del sets
    if s.dtype == "bf16" and not args.no_fp8:
        # the same workload with x, B and C stored as fp8 e4m3 (dt bf16): the same kernels,
        # half the bytes of the largest inputs
        r8, _, g8, _ = bench_prefill_workload(torch, args.workload, args.steps, args.warmup, flush, dtype="fp8")
        p8 = r8["prefill"]
        out["fp8_inputs"] = {"us_per_step": p8["us_per_step"], "tokens_per_s": p8["tokens_per_s"],
                             "method_bytes": p8["method_bytes"], "hbm_frac_method_bytes": p8["hbm_frac_method_bytes"],
                             "kernel_us_sum": p8["kernel_us_sum"], "roofline": r8["roofline"],
                             "launches": p8["launches"]}
        del g8
    if not args.no_extra:
        out["workloads"] = {}
        for wl in EXTRA_WORKLOADS:
            if wl == args.workload:
                continue
            r, _, gx, _ = bench_prefill_workload(torch, wl, args.steps, args.warmup, flush)
            out["workloads"][r["workload"]] = r
            del gx
    if not args.no_decode:
        out["decode"] = bench_decode(torch, args.decode_steps, flush)
        out["cached_vs_recompute"] = bench_cached_vs_recompute(torch, flush)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(s, inp)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
