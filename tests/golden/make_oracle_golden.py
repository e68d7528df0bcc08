"""Writes oracle_small.json: fp64 oracle outputs for a small seeded problem.

Calls only the oracle (and the shared seeded input generator).  The pages print
no worked numeric example for Lizard attention, so this file is a regression
anchor for the oracle itself (its correctness is pinned by the closed-form and
library-routine tests), not a value taken from the pages.

    python tests/golden/make_oracle_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from linearized_attention_amd.synthetic import make_fwd_inputs  # noqa: E402

CASE = dict(B=1, Hq=2, Hkv=1, L=70, d=8, W=5, M=2, dtype="f32", seed=2024, gate="uniform:-3")


def compute():
    inp = make_fwd_inputs(**CASE)
    y, yg, yw = oracle.lizard_fwd(*inp.tensors(), W=inp.W, M=inp.M, mix=inp.mix,
                                  scale=inp.scale, return_branches=True)
    idx = [(h, t) for h in range(2) for t in (0, 1, 4, 5, 31, 63, 64, 69)]
    return {
        "case": CASE,
        "mix": inp.mix,
        "scale": inp.scale,
        "samples": [{"head": h, "token": t, "y": y[0, h, t].tolist(),
                     "y_gla": yg[0, h, t].tolist(), "y_win": yw[0, h, t].tolist()}
                    for (h, t) in idx],
        "norms": {"y": float(np.linalg.norm(y)), "y_gla": float(np.linalg.norm(yg)),
                  "y_win": float(np.linalg.norm(yw))},
    }


if __name__ == "__main__":
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.json")
    with open(out, "w") as f:
        json.dump(compute(), f, indent=1)
    print("wrote", out)
