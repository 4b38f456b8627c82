"""CPU tests of bench.py's host logic: which launches a prefill makes at a given compute-unit
count (the same rules as the library's launchers), the algorithmic byte counts the roofline
uses, and the refusal of more than one GPU."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench
from mamba_ssd_scan_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NCU = 256  # MI355X compute units


def _shape(B, L, H, G, Q=256, P=64, N=128, dtype="bf16"):
    return synth.PrefillShape(B, L, H, P, N, G, Q, dtype)


def test_launches_of_the_benchmarked_prefill():
    s = synth.WORKLOADS[1]  # 130M layer, 4096 tokens: 384 items, 16 chunks, 256 pair workgroups
    assert bench.scan_kernel_name(s, NCU) == "chunk_scan_small_kernel"
    assert bench.passing_in_scan(s, NCU)
    assert bench.chunk_state_pair(s)
    assert bench.step_kernels(s, NCU) == ["chunk_state_pair_kernel", "chunk_scan_small_kernel"]


@pytest.mark.parametrize("w,expect", [
    (0, ["chunk_state_kernel", "state_passing_kernel", "chunk_scan_kernel"]),  # fp32, Q = 64
    (2, ["chunk_state_kernel", "state_passing_kernel", "chunk_scan_kernel"]),  # Q = 64
    (3, ["chunk_state_pair_kernel", "state_passing_kernel", "chunk_scan_pipe_kernel"]),  # 5120 items
])
def test_launches_of_the_other_workloads(w, expect):
    assert bench.step_kernels(synth.WORKLOADS[w], NCU) == expect


def test_launch_rules_at_their_edges():
    # 21 chunks: one-round scan (21 x 24 = 504 items) but Step-3 stays a launch of its own
    s = _shape(1, 21 * 256 - 5, 24, 1)
    assert bench.step_kernels(s, NCU) == ["chunk_state_pair_kernel", "state_passing_kernel",
                                          "chunk_scan_small_kernel"]
    # 513 items: the persistent scan, pipelined at N = 128 and P = 64
    assert bench.scan_kernel_name(_shape(1, 19 * 256, 27, 1), NCU) == "chunk_scan_pipe_kernel"
    assert bench.scan_kernel_name(_shape(1, 19 * 256, 27, 1, N=64), NCU) == "chunk_scan_kernel"
    assert bench.scan_kernel_name(_shape(1, 19 * 256, 27, 1, P=128), NCU) == "chunk_scan_kernel"
    assert bench.scan_kernel_name(_shape(1, 16 * 256, 32, 1), NCU) == "chunk_scan_small_kernel"  # 512 items
    # an odd number of heads per group keeps one head per workgroup
    assert not bench.chunk_state_pair(_shape(1, 12 * 256 - 100, 25, 5))
    assert bench.chunk_state_pair(_shape(2, 700, 8, 2, N=64))
    assert bench.chunk_state_pair(_shape(1, 32 * 256, 32, 1))  # any number of rounds
    assert not bench.chunk_state_pair(_shape(1, 4096, 24, 1, Q=128))
    assert not bench.chunk_state_pair(_shape(1, 4096, 24, 1, dtype="f32"))


def test_algorithmic_bytes_of_the_benchmarked_prefill():
    k = bench.alg_counts(synth.WORKLOADS[1], NCU)["kernels"]
    x, dt, bc = 4096 * 24 * 64 * 2, 4096 * 24 * 2, 4096 * 128 * 2
    tab = 2 * 24 * 16 * 256 * 4          # dA_cum and dt per chunk
    states = 24 * 16 * 64 * 128 * 2      # fp16 chunk states
    cb = 16 * 72 * 512 * 2               # 72 stored 32-column steps per chunk, 512 fp16 values each
    y, st = 4096 * 24 * 64 * 4, 24 * 64 * 128 * 4
    assert k["chunk_state_pair_kernel"]["bytes"] == x + dt + 2 * bc + tab + states + cb == 23134208
    # Step-3 inside the scan: chunk states and the final state, no entering states (and no
    # initial state: this workload starts from zero)
    assert synth.WORKLOADS[1].init_state == "zero"
    assert k["chunk_scan_small_kernel"]["bytes"] == x + bc + cb + tab + states + st + y == 47841280


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_method_bytes_of_the_headline_prefill():
    """The 2.7B-shaped 16384-token layer: the method's own bytes per step (inputs, y, initial
    and final state) are the 519.6 MB of the roofline floor; the pipelined chunk scan's share is
    x + C + y, without the entering states and GEMM1 products it also reads."""
    s = synth.WORKLOADS[3]
    c = bench.alg_counts(s, NCU)
    L, H, P, N = 16384, 80, 64, 128
    x, dt, bc, y, st = L * H * P * 2, L * H * 2, L * N * 2, L * H * P * 4, H * P * N * 4
    assert c["fused_bytes"] == x + dt + 2 * bc + y + 2 * st == 519569408
    k = c["kernels"]
    assert k["chunk_scan_pipe_kernel"]["method_bytes"] == x + bc + y
    assert k["chunk_scan_pipe_kernel"]["bytes"] > k["chunk_scan_pipe_kernel"]["method_bytes"]
    assert k["chunk_state_pair_kernel"]["method_bytes"] == x + dt + 2 * bc
    assert k["state_passing_kernel"]["method_bytes"] == 2 * st
    assert bench.step_kernels(s, NCU)[-1] == "chunk_scan_pipe_kernel"


def test_fp8_inputs_take_the_same_launches_and_count_one_byte_per_value():
    """x, B and C in fp8 e4m3 (dt in bf16): the same kernels as bf16 inputs, and method bytes
    of one byte per x, B and C value (two per dt value)."""
    import dataclasses
    s = dataclasses.replace(synth.WORKLOADS[3], dtype="fp8")
    assert bench.step_kernels(s, NCU) == ["chunk_state_pair_kernel", "state_passing_kernel", "chunk_scan_pipe_kernel"]
    s1 = dataclasses.replace(synth.WORKLOADS[1], dtype="fp8")
    assert bench.step_kernels(s1, NCU) == ["chunk_state_pair_kernel", "chunk_scan_small_kernel"]
    L, H, P, N = 16384, 80, 64, 128
    x, dt, bc, y, st = L * H * P, L * H * 2, L * N, L * H * P * 4, H * P * N * 4
    c = bench.alg_counts(s, NCU)
    assert c["fused_bytes"] == x + dt + 2 * bc + y + 2 * st == 431489024
    # the intermediates stay fp16, as for bf16 inputs
    assert c["kernels"]["state_passing_kernel"]["bytes"] == bench.alg_counts(synth.WORKLOADS[3], NCU)["kernels"][
        "state_passing_kernel"]["bytes"]
