"""Write tests/golden/oracle_regression.json from the fp64 oracle.

Calls only ``oracle/`` (and the seeded input generator).  The fixture guards
the oracle against accidental drift (a rebuild with other flags, an edit):
the regression test re-runs the same case and demands bitwise equality.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from mamba_ssd_scan_amd import synth  # noqa: E402
from oracle import ref  # noqa: E402

CASE = dict(seed=424242, batch=1, seqlen=9, nheads=2, headdim=3, dstate=4, ngroups=1)


def compute():
    c = CASE
    inp = synth.random_prefill(np.random.Generator(np.random.PCG64(c["seed"])), c["batch"], c["seqlen"],
                               c["nheads"], c["headdim"], c["dstate"], c["ngroups"], "f32")
    return inp, ref.prefill(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"])


if __name__ == "__main__":
    _, (y, hT) = compute()
    out = dict(what="fp64 oracle output on a seeded random case; regression guard, written by make_golden.py",
               case=CASE, y=[float.hex(float(v)) for v in y.ravel()],
               final_state=[float.hex(float(v)) for v in hT.ravel()])
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json"), "w") as f:
        json.dump(out, f, indent=1)
