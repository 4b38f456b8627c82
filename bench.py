"""Benchmark of the SSD layer core on one MI355X.

One step = one full chunked prefill (every prefill stage: cumulative decay, chunk states,
inter-chunk state passing, intra-chunk + off-diagonal output) over the Mamba-2-2.7B-shaped
long-context layer (batch 1, 16384 tokens, 80 heads, headdim 64, d_state 128, chunk 256,
bf16 inputs, fp32 state and output, random initial state), with inputs resident in HBM.
Each timed step starts cold: a 512 MiB read evicts the 256 MiB Infinity Cache and the L2s
first, outside the timed events.  The 130M- and 370M-shaped layers are timed the same way
and reported under "workloads"; the decode update (batch 64, 80 heads, 1024 tokens) under
"decode".

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded on the stream
the kernels run on.  The oracle (fp64 CPU recurrence) is timed on the host's cores on the
same workload as "cpu_baseline".
"""
from __future__ import annotations

import argparse
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
    every (b, h, chunk) item fits at two per compute unit (bf16, 256-token chunks, P = 64),
    else the pipelined persistent one (bf16, 256-token chunks, P = 64, N = 128) or the
    persistent one (the same rule as the library's launcher).  ncu: compute units (default:
    the current device's)."""
    if ncu is None:
        import torch
        ncu = torch.cuda.get_device_properties(0).multi_processor_count
    nitems = s.batch * s.nheads * -(-s.seqlen // s.chunk)
    small = s.dtype == "bf16" and s.chunk == 256 and s.headdim == 64 and nitems <= 2 * ncu
    if small:
        return "chunk_scan_small_kernel"
    pipe = s.dtype == "bf16" and s.chunk == 256 and s.headdim == 64 and s.dstate == 128
    return "chunk_scan_pipe_kernel" if pipe else "chunk_scan_kernel"


def passing_in_scan(s, ncu=None) -> bool:
    """Whether ssd_prefill runs Step-3 inside the one-round chunk scan (two launches): the
    one-round kernel's shapes with at most 16 chunks (the same rule as the library)."""
    return scan_kernel_name(s, ncu) == "chunk_scan_small_kernel" and -(-s.seqlen // s.chunk) <= 16


def chunk_state_pair(s) -> bool:
    """Whether ssd_prefill's first launch (cumulative decay, chunk states and GEMM1) takes two
    heads of a group per workgroup: bf16, 256-token chunks, P = 64 and an even number of heads
    per group (the same rule as the library)."""
    return s.dtype == "bf16" and s.chunk == 256 and s.headdim == 64 and (s.nheads // s.ngroups) % 2 == 0


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
    ib = 2 if s.dtype == "bf16" else 4
    nc = -(-L // Q)
    x = B * L * H * P * ib
    dt = B * L * H * ib
    bc = B * L * G * N * ib            # one of B or C
    y = B * L * H * P * 4
    chunk_tab = 2 * B * H * nc * Q * 4  # dA_cum + dt regrouped per chunk
    states = B * H * nc * P * N * ib   # chunk / entering states: fp16 for bf16 inputs, fp32 otherwise
    hen = states
    st = B * H * P * N * 4
    h0 = st if s.init_state != "zero" else 0
    tri = Q * (Q + 1)                  # 2 flops x Q(Q+1)/2 pairs
    # C.B^T products as the GEMM1 kernel stores them: per (b, g, chunk), 512 values per
    # 32-column step of each 16-row tile (the steps on or below the diagonal), fp16 for
    # bf16 inputs and fp32 for fp32 inputs
    cb = B * G * nc * sum(t // 2 + 1 for t in range(Q // 16)) * 512 * (2 if s.dtype == "bf16" else 4)
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


def time_launches(torch, fn, n, flush=None, before=None):
    """Duration (us) of ``fn``: mean and min over n launches, from HIP events on the current stream.

    With ``flush``, every launch is preceded by the cache eviction.  A pair of
    events costs a few microseconds of dispatch and completion signalling, so
    the events bracket [eviction + fn] and, on interleaved iterations,
    [eviction] alone; the difference of the means is fn's duration with the
    event overhead cancelled (the eviction itself is outside the result).

    An interval also counts any time the GPU waits for the host to enqueue the next
    command, so the host must stay ahead: evictions are put in flight before the first
    timed launch (the GPU works through them while the loop enqueues), and Python's
    garbage collector, whose pauses can drain the queue, is off during the loop.
    (Without this a single stalled interval moved a 200-launch mean by over 100 us.)
    """
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    with_fn, alone = [], []
    gc_on = gc.isenabled()
    gc.disable()
    try:
        if flush is not None:
            for _ in range(8):
                flush()
        for _ in range(n):
            if before is not None:
                before()
            a, b = ev(), ev()
            a.record(stream)
            if flush is not None:
                flush()
            fn()
            b.record(stream)
            with_fn.append((a, b))
            if flush is not None:
                c, d = ev(), ev()
                c.record(stream)
                flush()
                d.record(stream)
                alone.append((c, d))
        torch.cuda.synchronize()
    finally:
        if gc_on:
            gc.enable()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in with_fn])
    if flush is None:
        return float(t.mean()), float(t.min()), float(np.median(t))
    f = np.array([c.elapsed_time(d) * 1e3 for c, d in alone])
    return float(t.mean() - f.mean()), float(t.min() - f.mean()), float(np.median(t) - np.median(f))


def prefill_buffers(torch, s, inp):
    g = {k: synth.to_torch(inp[k], s.dtype) for k in ("x", "dt", "B", "C")}
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
                              dtype=torch.float16 if s.dtype == "bf16" else torch.float32, device="cuda")
    g["hen"] = g["states"]
    g["cb"] = torch.empty(ssd.chunk_gemm1_size(s.batch, s.seqlen, s.ngroups, s.chunk) // 4, dtype=torch.float32,
                          device="cuda")
    return g


def run_prefill(g, s):
    ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=s.chunk, y=g["y"],
                final_state=g["final"], workspace=g["ws"])


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
    reps, total = 0, 0.0
    while reps < max_reps and (total < min_seconds or reps == 0):
        t0 = time.perf_counter()
        ref.prefill(f64["x"], f64["dt"], f64["A"], f64["B"], f64["C"], f64["D"], f64["h0"], nthreads=cores)
        total += time.perf_counter() - t0
        reps += 1
    tokens = s.batch * s.seqlen * reps
    return {"value": tokens / total, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full workload ({s.batch}x{s.seqlen} tokens, all {s.nheads} heads), fp64 sequential "
                      f"recurrence, repeated {reps}x ({total:.1f} s)"}


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
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for t in range(steps):
        ssd.step(state, xs[t], dts[t], A, Bs[t], Cs[t], D, y=y)
    b.record(stream)
    torch.cuda.synchronize()
    us_loop = a.elapsed_time(b) * 1e3 / steps
    # cold: flush before each step (64 sampled steps)
    k = [0]

    def one():
        t = k[0] % steps
        k[0] += 1
        ssd.step(state, xs[t], dts[t], A, Bs[t], Cs[t], D, y=y)

    us_cold = time_launches(torch, one, min(64, steps), flush=flush)[0]
    # the same tokens as one HIP graph (ssd_decode_graph): one launch for all of them
    y_all = torch.empty((steps, s.batch, s.nheads, s.headdim), dtype=torch.float32, device="cuda")
    graph = ssd.DecodeGraph(state, xs, dts, A, Bs, Cs, D, y=y_all)
    graph.launch()
    torch.cuda.synchronize()
    us_graph = time_back_to_back(torch, graph.launch, 3) / steps
    graph.close()
    nbytes = decode_bytes_per_step(s)
    # the batch-64 x 80-head step runs one workgroup per head (step_heads_kernel)
    traffic = counter_traffic("step_heads_kernel", synth.WORKLOAD_NAMES[DECODE_WORKLOAD])
    return {
        "counter_traffic_bytes_per_step": traffic,
        "workload": synth.WORKLOAD_NAMES[DECODE_WORKLOAD], "steps": steps,
        "us_per_step": us_loop, "tokens_per_s": s.batch / (us_loop * 1e-6),
        "alg_bytes_per_step": nbytes, "gbps": nbytes / (us_loop * 1e-6) / 1e9,
        "hbm_frac": nbytes / (us_loop * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "cold_us_per_step": us_cold, "cold_gbps": nbytes / (us_cold * 1e-6) / 1e9,
        "cold_hbm_frac": nbytes / (us_cold * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "graph_us_per_step": us_graph, "graph_gbps": nbytes / (us_graph * 1e-6) / 1e9,
        "note": "us_per_step: 1024 back-to-back ssd_step launches on one state (the 168 MB state can stay in "
                "the 256 MiB Infinity Cache between steps); cold: 512 MiB cache eviction before each step; "
                "graph: the 1024 tokens as one ssd_decode_graph launch (per-token outputs in their own slots)",
    }


def time_back_to_back(torch, fn, n):
    """Mean duration (us) of ``fn`` over n back-to-back launches between two events (warm caches)."""
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def bench_layer_rows(torch, s, g, flush, steps):
    """The prefill with its inputs where a Mamba-2 layer holds them: x, B and C in the
    convolved [x | B | C] rows, dt in the input-projection [z | x | B | C | dt] rows.
    Cold, like the step: read in place through token strides, against copying the four
    inputs out to dense tensors first (what a dense-only call needs)."""
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
    us_in = time_launches(torch, in_place, steps, flush=flush)[0]
    us_cp = time_launches(torch, copied, steps, flush=flush)[0]
    return {"in_place_us": us_in, "copy_then_dense_us": us_cp,
            "rows": f"x|B|C rows of {hp + 2 * gn} and z|x|B|C|dt rows of {2 * hp + 2 * gn + H} elements",
            "note": "cold, events on the launch stream; the copies are torch's, outside the library"}


def bench_cached_vs_recompute(torch, context=4096, ntok=256, reps=20):
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
        us_re = time_back_to_back(torch, lambda: run_prefill(g, s), reps)
        ds = synth.DecodeShape(1, H, 64, 128, 1, ntok, "bf16")
        dinp = synth.decode_inputs(ds, synth.SEED_BASE + 200 + H)
        xs, dts = synth.to_torch(dinp["x"], "bf16"), synth.to_torch(dinp["dt"], "bf16")
        Bs, Cs = synth.to_torch(dinp["B"], "bf16"), synth.to_torch(dinp["C"], "bf16")
        state = g["final"].clone()  # the cached state after the prefix
        graph = ssd.DecodeGraph(state, xs, dts, g["A"], Bs, Cs, g["D"])
        graph.launch()
        torch.cuda.synchronize()
        us_graph = time_back_to_back(torch, graph.launch, max(2, reps // 4)) / ntok
        graph.close()
        y1 = torch.empty((1, H, 64), dtype=torch.float32, device="cuda")
        k = [0]

        def eager():
            t = k[0] % ntok
            k[0] += 1
            ssd.step(state, xs[t], dts[t], g["A"], Bs[t], Cs[t], g["D"], y=y1)
        eager()
        torch.cuda.synchronize()
        us_eager = time_back_to_back(torch, eager, ntok)
        out[name] = {"nheads": H, "recompute_us": us_re, "cached_graph_us": us_graph, "cached_eager_us": us_eager,
                     "speedup_graph": us_re / us_graph, "speedup_eager": us_re / us_eager}
        del g, xs, dts, Bs, Cs, state
    return {"context": context, "batch": 1, "headdim": 64, "dstate": 128, "chunk": 256, "dtype": "bf16",
            "tokens_per_graph": ntok, "models": out,
            "note": "SSD layer core only (one layer, no projections): per-token time of cached decode vs an "
                    "ssd_prefill over the whole prefix plus the token; warm, back-to-back launches"}


# ---------------------------------------------------------------------------- main

def bench_prefill_workload(torch, wl, steps, warmup, flush, headline=False):
    """Cold prefill steps of one workload, its kernels one by one, and the rooflines.

    Returns (record, inputs, buffers, wall seconds of the timed steps)."""
    s = synth.WORKLOADS[wl]
    inp = synth.prefill_inputs(s, synth.SEED_BASE + wl)
    g = prefill_buffers(torch, s, inp)
    settle_clocks(torch, flush)
    for _ in range(warmup):
        run_prefill(g, s)
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` cold steps, bracketed by synchronisations
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    us_step, us_step_min, us_step_med = time_launches(torch, lambda: run_prefill(g, s), steps, flush=flush)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    tokens = s.batch * s.seqlen
    us_warm = time_back_to_back(torch, lambda: run_prefill(g, s), steps)

    # ---- per-kernel durations (cold), events on the launch stream
    counts = alg_counts(s)
    stages = stage_fns(torch, g, s)
    kernels = {}
    for name, (fn, before) in stages.items():
        us, us_min, us_med = time_launches(torch, fn, steps, flush=flush, before=before)
        c = counts["kernels"][name]
        kernels[name] = {"us": us, "us_min": us_min, "us_median": us_med, "method_bytes": c["method_bytes"],
                         "alg_bytes_incl_intermediates": c["bytes"], "alg_flops": c["flops"],
                         "method_gbps": c["method_bytes"] / (us * 1e-6) / 1e9, "tflops": c["flops"] / (us * 1e-6) / 1e12}
    # the step's longest launch among those timed on their own (the fused first launch has no
    # entry point of its own; its duration is in the kernel trace)
    dom = max((k for k in step_kernels(s) if k in kernels), key=lambda k: kernels[k]["us"])
    d = kernels[dom]
    roof = {"bound": "hbm", "achieved": d["method_gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": d["method_gbps"] / HBM_PEAK_GBS, "traffic": counter_traffic(dom, synth.WORKLOAD_NAMES[wl]),
            "kernel": dom,
            "variant": ("with Step-3 (ssd_chunk_scan_passing)" if dom == "chunk_scan_small_kernel"
                        and passing_in_scan(s) else "as launched by the stage entry point"),
            "us_per_launch": d["us"], "method_bytes_per_launch": d["method_bytes"],
            "alg_bytes_incl_intermediates_per_launch": d["alg_bytes_incl_intermediates"],
            "alg_flops_per_launch": d["alg_flops"], "mfma_tflops": d["tflops"],
            "mfma_frac": d["tflops"] / MFMA_BF16_PEAK_TFLOPS,
            "intensity_flop_per_method_byte": d["alg_flops"] / d["method_bytes"]}

    sec = us_step * 1e-6
    fb, ff = counts["fused_bytes"], counts["fused_flops"]
    prefill = {
        "us_per_step_cold": us_step, "us_per_step_cold_median": us_step_med, "us_per_step_cold_min": us_step_min,
        "us_per_step_warm": us_warm, "tokens_per_s": tokens / sec, "warm_tokens_per_s": tokens / (us_warm * 1e-6),
        "method_bytes": fb, "alg_flops": ff,
        "method_gbps": fb / sec / 1e9, "hbm_frac_method_bytes": fb / sec / 1e9 / HBM_PEAK_GBS,
        "alg_tflops": ff / sec / 1e12, "alg_mfma_frac": ff / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "hbm_floor_us": fb / (HBM_PEAK_GBS * 1e9) * 1e6,
        "step_launches": step_kernels(s),
        "kernel_us_sum": sum(kernels[k]["us"] for k in step_kernels(s) if k in kernels),
    }
    # bf16 y (the fp32 result rounded once): halves the largest stream
    if s.dtype == "bf16":
        yb = torch.empty((s.batch, s.seqlen, s.nheads, s.headdim), dtype=torch.bfloat16, device="cuda")
        fbf = lambda: ssd.prefill_ex(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], y_dtype=torch.bfloat16,
                                     chunk=s.chunk, y=yb, final_state=g["final"], workspace=g["ws"])
        for _ in range(3):
            fbf()
        torch.cuda.synchronize()
        ub = time_launches(torch, fbf, steps, flush=flush)
        bb = fb - s.batch * s.seqlen * s.nheads * s.headdim * 2
        prefill["bf16_y"] = {"us_per_step_cold": ub[0], "us_per_step_cold_median": ub[2],
                             "tokens_per_s": tokens / (ub[0] * 1e-6), "method_bytes": bb,
                             "hbm_frac_method_bytes": bb / (ub[0] * 1e-6) / 1e9 / HBM_PEAK_GBS}
    rec = {"workload": synth.WORKLOAD_NAMES[wl], "value": tokens / sec, "unit": "tokens/s",
           "roofline": roof, "prefill": prefill, "kernels": kernels}
    return rec, inp, g, wall


def bench_single_pass(torch, wl, g, steps, flush):
    """The single-pass prefill (only selected on request) on the same workload, cold."""
    s = synth.WORKLOADS[wl]
    ws = ssd.alloc_workspace(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk)
    f = lambda: ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], g["h0"], chunk=s.chunk, y=g["y"],
                            final_state=g["final"], workspace=ws, path=ssd.PATH_SINGLE_PASS)
    try:
        f()
    except ssd.SsdError:
        return None
    for _ in range(2):
        f()
    torch.cuda.synchronize()
    us = time_launches(torch, f, steps, flush=flush)
    return {"us_per_step_cold": us[0], "us_per_step_cold_median": us[2],
            "tokens_per_s": s.batch * s.seqlen / (us[0] * 1e-6),
            "note": "ssd_prefill_forced with SSD_PATH_SINGLE_PASS; the library's own path is the step above"}


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
    ap.add_argument("--only", choices=["prefill", "chunk_scan_kernel", "chunk_scan_pipe_kernel", "chunk_state_kernel", "state_passing_kernel",
                                       "chunk_cumsum_kernel", "chunk_gemm1_kernel", "chunk_scan_small_kernel",
                                       "single_pass", "step", "cached", "copy"],
                    help="profiling aid: launch only this work --steps times (cold), print nothing else")
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
        print(json.dumps(bench_cached_vs_recompute(torch)))
        return 0
    if args.only is not None:
        inp = synth.prefill_inputs(s, synth.SEED_BASE + args.workload)
        g = prefill_buffers(torch, s, inp)
        settle_clocks(torch, flush)
        for _ in range(args.warmup):
            run_prefill(g, s)
        torch.cuda.synchronize()
        if args.only == "prefill":
            time_launches(torch, lambda: run_prefill(g, s), args.steps, flush=flush)
        elif args.only == "single_pass":
            bench_single_pass(torch, args.workload, g, args.steps, flush)
        else:
            fn, before = stage_fns(torch, g, s)[args.only]
            time_launches(torch, fn, args.steps, flush=flush, before=before)
        return 0

    rec, inp, g, wall = bench_prefill_workload(torch, args.workload, args.steps, args.warmup, flush, headline=True)
    us_step = rec["prefill"]["us_per_step_cold"]
    out = {
        "metric": METRIC, "value": rec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": us_step / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": s.dtype, "data": "synthetic",
        "config": {"workload": wname, "batch": s.batch, "seqlen": s.seqlen, "nheads": s.nheads,
                   "headdim": s.headdim, "dstate": s.dstate, "ngroups": s.ngroups, "chunk": s.chunk,
                   "initial_state": s.init_state,
                   "cache": "cold (512 MiB eviction before each step, outside the events)",
                   "parallelism": "single GPU"},
        "roofline": rec["roofline"],
        "prefill": rec["prefill"],
        "kernels": rec["kernels"],
        "timed_wall_s": wall,
    }
    sp = bench_single_pass(torch, args.workload, g, args.steps, flush)
    if sp is not None:
        out["single_pass"] = sp
    out["layer_rows"] = bench_layer_rows(torch, s, g, flush, args.steps)
    del g
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
        out["cached_vs_recompute"] = bench_cached_vs_recompute(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(s, inp)
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
