"""Seeded synthetic inputs for the SSD layer core.

This module only draws random numbers and rounds them to the storage
precision; it holds none of the state-space arithmetic.  Both the GPU path
and the CPU oracle consume the arrays it returns, so the oracle sees exactly
the values the GPU sees (bf16 values are carried as the fp32 numbers they
represent, which upcast to fp64 without error).

Recipe (Mamba-2 shaped inputs; the three pages give no dataset for the SSD
core, so every workload is synthetic):

* x ~ N(0, 1)                                    [B, L, H, P]
* B, C ~ N(0, 1) / sqrt(N)                       [B, L, G, N]
* dt = softplus(N(-3, 1))  (positive step size)  [B, L, H]
* A_h = -exp(U(log 1, log 16))  (decay rate)     [H]     fp32
* D ~ N(0, 1)  (skip gain)                       [H]     fp32
* initial state: zeros, or N(0, 0.1^2)           [B, H, P, N] fp32

Draw order is x, B, C, dt, A, D, state, from numpy's PCG64 seeded with
``20260000 + config index`` for the named workloads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

SEED_BASE = 20260000


@dataclasses.dataclass(frozen=True)
class PrefillShape:
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str  # "bf16", "f32" or "fp8" (x, B, C in e4m3, dt in bf16): storage of the inputs
    init_state: str = "zero"  # "zero" or "randn" (std 0.1)


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    steps: int
    dtype: str = "bf16"


# The five named workloads.  Index 0 is the tiny fp32 case, 1-3 are Mamba-2
# layer prefills (130M, 370M in the N=Q=64 setting, 2.7B long context) and 4
# is the batched single-token decode.
WORKLOADS = {
    0: PrefillShape(1, 256, 4, 64, 64, 1, 64, "f32"),
    1: PrefillShape(1, 4096, 24, 64, 128, 1, 256, "bf16"),
    2: PrefillShape(8, 2048, 32, 64, 64, 1, 64, "bf16"),
    3: PrefillShape(1, 16384, 80, 64, 128, 1, 256, "bf16", "randn"),
    4: DecodeShape(64, 80, 64, 128, 1, 1024, "bf16"),
}

# Head counts of the five Mamba-2 checkpoints (130M .. 2.7B) on which cached decode is
# compared with full-prefix recomputation at a 4096-token context ("Compiler-First
# State Space Duality and Portable O(1) Autoregressive Caching for Inference",
# abstract).  Every one has headdim 64, d_state 128 and one B/C group per layer;
# the head count is 2 * d_model / 64.
MAMBA2_LADDER = {"130m": 24, "370m": 32, "780m": 48, "1.3b": 64, "2.7b": 80}

WORKLOAD_NAMES = {
    0: "tiny-f32-prefill-b1-l256-h4-p64-n64-q64",
    1: "mamba2-130m-prefill-b1-l4096-h24-p64-n128-q256",
    2: "mamba2-370m-prefill-b8-l2048-h32-p64-n64-q64",
    3: "mamba2-2.7b-prefill-b1-l16384-h80-p64-n128-q256",
    4: "mamba2-2.7b-decode-b64-h80-p64-n128-x1024",
}


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # uint32 arithmetic wraps only for NaN bit patterns, which are restored below.
    with np.errstate(over="ignore"):
        rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    out = rounded.view(np.float32)
    nan = np.isnan(a)
    if nan.any():
        out = np.where(nan, a, out)
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


E4M3_MAX = 448.0


def e4m3_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest OCP fp8 e4m3 value (ties to even); returns fp32.

    e4m3: a sign, 4 exponent bits (bias 7), 3 mantissa bits; normals from 2^-6, subnormals
    in steps of 2^-9, largest finite 448.  Values that would round past 448 are refused."""
    a = np.asarray(a, dtype=np.float64)
    if np.any(np.abs(a) >= 464.0):  # 464 and up round past the largest finite value
        raise ValueError("value out of the e4m3 range")
    _, ex = np.frexp(a)                          # |a| in [2^(ex-1), 2^ex)
    k = np.maximum(ex - 1, -6)                   # the binade's exponent, subnormals at -6
    q = np.ldexp(1.0, k - 3)                     # the spacing of e4m3 values there
    return (np.round(a / q) * q).astype(np.float32)  # np.round: half to even


def e4m3_codes(a: np.ndarray) -> np.ndarray:
    """The e4m3 codes (uint8) of fp32 values that are already e4m3-representable."""
    a = np.asarray(a, dtype=np.float64)
    sign = (np.signbit(a)).astype(np.uint8) << 7
    m = np.abs(a)
    _, ex = np.frexp(m)
    k = ex - 1
    normal = m >= 2.0 ** -6
    e = np.where(normal, k + 7, 0)
    mant = np.where(normal, m / np.ldexp(1.0, k) - 1.0, m / 2.0 ** -9) * np.where(normal, 8.0, 1.0)
    return (sign | (e.astype(np.uint8) << 3) | np.rint(mant).astype(np.uint8)).astype(np.uint8)


def e4m3_value(code) -> float:
    """The value of one e4m3 code (NaN for 0x7f and 0xff)."""
    code = int(code)
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    return s * (m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7))


def softplus(z: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), z).astype(np.float32)


def _store(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(a)
    if dtype == "fp8":
        return e4m3_round(a)
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def dt_dtype(dtype: str) -> str:
    """Storage of dt and z beside inputs of ``dtype`` (bf16 beside fp8 x, B and C)."""
    return "bf16" if dtype == "fp8" else dtype


def prefill_inputs(shape: PrefillShape, seed: int, *, heads: Optional[np.ndarray] = None) -> dict:
    """Draw one prefill problem.  All arrays are fp32 holding exact values.

    ``heads`` optionally selects a subset of heads after drawing the full
    problem (the draw is identical either way), so large workloads can be
    checked head by head on the CPU.
    """
    s = shape
    rng = np.random.Generator(np.random.PCG64(seed))
    f = np.float32
    x = rng.standard_normal((s.batch, s.seqlen, s.nheads, s.headdim), dtype=f)
    Bm = rng.standard_normal((s.batch, s.seqlen, s.ngroups, s.dstate), dtype=f) / f(math.sqrt(s.dstate))
    Cm = rng.standard_normal((s.batch, s.seqlen, s.ngroups, s.dstate), dtype=f) / f(math.sqrt(s.dstate))
    dt = softplus(rng.normal(-3.0, 1.0, size=(s.batch, s.seqlen, s.nheads)).astype(f))
    A = -np.exp(rng.uniform(math.log(1.0), math.log(16.0), size=(s.nheads,))).astype(f)
    D = rng.standard_normal((s.nheads,), dtype=f)
    if s.init_state == "randn":
        h0 = (0.1 * rng.standard_normal((s.batch, s.nheads, s.headdim, s.dstate), dtype=f)).astype(f)
    elif s.init_state == "zero":
        h0 = None
    else:
        raise ValueError(s.init_state)
    out = dict(
        x=_store(x, s.dtype),
        dt=_store(dt, dt_dtype(s.dtype)),
        A=A,
        B=_store(Bm, s.dtype),
        C=_store(Cm, s.dtype),
        D=D,
        h0=h0,
        dtype=s.dtype,
    )
    if heads is not None:
        out = select_heads(out, heads, s.ngroups, s.nheads)
    return out


def select_heads(inp: dict, heads, ngroups: int, nheads: int) -> dict:
    """Restrict a prefill problem to a subset of heads (groups kept whole)."""
    heads = np.asarray(heads)
    hpg = nheads // ngroups
    groups = np.unique(heads // hpg)
    if len(groups) != 1 and ngroups != 1:
        raise ValueError("head subset must lie in one group")
    g = groups[0] if ngroups != 1 else 0
    out = dict(inp)
    out["x"] = np.ascontiguousarray(inp["x"][:, :, heads, :])
    out["dt"] = np.ascontiguousarray(inp["dt"][:, :, heads])
    out["A"] = np.ascontiguousarray(inp["A"][heads])
    out["D"] = np.ascontiguousarray(inp["D"][heads])
    out["B"] = np.ascontiguousarray(inp["B"][:, :, g:g + 1, :])
    out["C"] = np.ascontiguousarray(inp["C"][:, :, g:g + 1, :])
    if inp.get("h0") is not None:
        out["h0"] = np.ascontiguousarray(inp["h0"][:, heads])
    return out


def random_prefill(rng: np.random.Generator, batch, seqlen, nheads, headdim, dstate, ngroups,
                   dtype="f32", *, init_state=True, A_range=(1.0, 16.0), dt_mode="softplus",
                   D_zero=False) -> dict:
    """Small random problem for tests, with optional stress distributions.

    ``dt_mode``: "softplus" (the workload recipe), "weak" (dt ~ U(0, 0.02)
    with A in [-0.05, 0]: long memory, exercises chunk-to-chunk passing),
    "strong" (dt*A around -50: decays underflow to zero).
    """
    f = np.float32
    x = rng.standard_normal((batch, seqlen, nheads, headdim), dtype=f)
    Bm = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=f) / f(math.sqrt(dstate))
    Cm = rng.standard_normal((batch, seqlen, ngroups, dstate), dtype=f) / f(math.sqrt(dstate))
    if dt_mode == "softplus":
        dt = softplus(rng.normal(-3.0, 1.0, size=(batch, seqlen, nheads)).astype(f))
        A = -np.exp(rng.uniform(math.log(A_range[0]), math.log(A_range[1]), size=(nheads,))).astype(f)
    elif dt_mode == "weak":
        dt = rng.uniform(0.0, 0.02, size=(batch, seqlen, nheads)).astype(f)
        A = -rng.uniform(0.0, 0.05, size=(nheads,)).astype(f)
    elif dt_mode == "strong":
        dt = rng.uniform(2.0, 4.0, size=(batch, seqlen, nheads)).astype(f)
        A = -rng.uniform(12.0, 16.0, size=(nheads,)).astype(f)
    else:
        raise ValueError(dt_mode)
    D = np.zeros((nheads,), f) if D_zero else rng.standard_normal((nheads,), dtype=f)
    h0 = (0.1 * rng.standard_normal((batch, nheads, headdim, dstate), dtype=f)).astype(f) if init_state else None
    return dict(x=_store(x, dtype), dt=_store(dt, dt_dtype(dtype)), A=A, B=_store(Bm, dtype), C=_store(Cm, dtype),
                D=D, h0=h0, dtype=dtype)


def option_inputs(rng: np.random.Generator, inp: dict) -> dict:
    """Raw in-projection channels for the option entry points, shaped like ``inp``.

    dt_raw ~ N(-3, 1) (the pre-softplus step-size channel, so that the effective
    step size has the recipe's distribution when dt_bias is small), dt_bias [H] ~
    N(0, 0.5^2) fp32, z ~ N(0, 1) laid out like x; dt_raw and z in inp's storage dtype.
    """
    f = np.float32
    d = inp["dtype"]
    H = inp["A"].shape[0]
    dt_raw = rng.normal(-3.0, 1.0, size=inp["dt"].shape).astype(f)
    bias = (0.5 * rng.standard_normal((H,))).astype(f)
    z = rng.standard_normal(inp["x"].shape, dtype=f)
    return dict(dt_raw=_store(dt_raw, dt_dtype(d)), dt_bias=bias, z=_store(z, dt_dtype(d)))


def decode_inputs(shape: DecodeShape, seed: int, steps: Optional[int] = None) -> dict:
    """Per-step decode inputs for ``steps`` tokens plus the starting state.

    Arrays carry a leading step axis: x [S, B, H, P], dt [S, B, H],
    B/C [S, B, G, N]; state [B, H, P, N] ~ N(0, 0.1^2) fp32.
    """
    s = shape
    S = s.steps if steps is None else steps
    rng = np.random.Generator(np.random.PCG64(seed))
    f = np.float32
    x = rng.standard_normal((S, s.batch, s.nheads, s.headdim), dtype=f)
    Bm = rng.standard_normal((S, s.batch, s.ngroups, s.dstate), dtype=f) / f(math.sqrt(s.dstate))
    Cm = rng.standard_normal((S, s.batch, s.ngroups, s.dstate), dtype=f) / f(math.sqrt(s.dstate))
    dt = softplus(rng.normal(-3.0, 1.0, size=(S, s.batch, s.nheads)).astype(f))
    A = -np.exp(rng.uniform(math.log(1.0), math.log(16.0), size=(s.nheads,))).astype(f)
    D = rng.standard_normal((s.nheads,), dtype=f)
    state = (0.1 * rng.standard_normal((s.batch, s.nheads, s.headdim, s.dstate), dtype=f)).astype(f)
    return dict(x=_store(x, s.dtype), dt=_store(dt, dt_dtype(s.dtype)), A=A, B=_store(Bm, s.dtype),
                C=_store(Cm, s.dtype), D=D, state=state, dtype=s.dtype)


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    """Copy an fp32 array holding exact values to a torch tensor of ``dtype``.

    ``dtype`` "bf16" moves the bf16 bit patterns (no re-rounding), "fp8" the e4m3
    codes (torch.float8_e4m3fn), "f32" the fp32 values.
    """
    import torch
    if dtype == "fp8":
        return torch.from_numpy(e4m3_codes(a)).to(device).view(torch.float8_e4m3fn)
    if dtype == "bf16":
        bits = bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
    raise ValueError(dtype)
