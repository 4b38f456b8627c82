"""Helpers for the GPU parity tests: upload synthetic inputs, run the HIP
path through the C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

from mamba_ssd_scan_amd import ssd, synth
from oracle import ref
from tests.util import TOL, rel_err


def torch():
    import torch as t
    return t


def upload(inp: dict) -> dict:
    T = torch()
    d = inp["dtype"]
    out = {k: synth.to_torch(inp[k], d) for k in ("x", "B", "C")}
    out["dt"] = synth.to_torch(inp["dt"], synth.dt_dtype(d))
    out["A"] = T.from_numpy(np.ascontiguousarray(inp["A"], np.float32)).cuda()
    out["D"] = None if inp.get("D") is None else T.from_numpy(np.ascontiguousarray(inp["D"], np.float32)).cuda()
    out["h0"] = None if inp.get("h0") is None else T.from_numpy(np.ascontiguousarray(inp["h0"], np.float32)).cuda()
    return out


def gpu_prefill(inp: dict, Q: int, *, D="use", h0="use"):
    T = torch()
    g = upload(inp)
    Dd = g["D"] if D == "use" else D
    H0 = g["h0"] if h0 == "use" else h0
    y, hT = ssd.prefill(g["x"], g["dt"], g["A"], g["B"], g["C"], Dd, H0, chunk=Q)
    T.cuda.synchronize()
    return y.cpu().numpy(), hT.cpu().numpy()


def oracle_prefill(inp: dict, *, D="use"):
    return ref.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"] if D == "use" else D, inp["h0"])


def check_prefill(inp: dict, Q: int, tol: float = None, label: str = ""):
    """y (with D), y (D = 0) and the final state within the tolerance of the input dtype."""
    tol = TOL[inp["dtype"]] if tol is None else tol
    y, hT = gpu_prefill(inp, Q)
    yo, ho = oracle_prefill(inp)
    y0, _ = gpu_prefill(inp, Q, D=None)
    yo0, _ = oracle_prefill(inp, D=None)
    errs = dict(y=rel_err(y, yo), y_D0=rel_err(y0, yo0), state=rel_err(hT, ho))
    print(f"[parity] {label} Q={Q} dtype={inp['dtype']} " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
          flush=True)
    for k, v in errs.items():
        assert np.isfinite(v) and v < tol, (label, k, v, tol)
    return errs
