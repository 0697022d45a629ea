"""Writes downproj_gate_bias.json: the gate bias b_g of the mixed-gate
down_proj workload (K=14336, N=4096, r=64, token counts 64 and 512).

The workload asks for a bias that puts about 70% of the tokens below the skip
threshold tau = 0.05.  Reading: with z0 = X . w_g (float64, from the oracle)
sorted ascending and j = ceil(0.7 M), b_g = logit(0.05) - (z0_(j) + z0_(j+1))/2,
so exactly j tokens have g < 0.05 and no token sits near the threshold.
The value is rounded to float32 (the type of the bias argument).

Calls only the oracle and the seeded input generator.  Run from the repo root:
    python tests/golden/make_gate_bias.py
"""
import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402

TAU = 0.05


def compute():
    spec = workloads.WORKLOADS[4]
    X, W, A, B, w_g = workloads.draw((0, 4), max(spec["ms"]), spec["K"], spec["N"], spec["r"],
                                     spec["outliers"])
    out, margins = {}, {}
    for M in spec["ms"]:
        z0 = np.sort(oracle.gate_logits(X[:M], w_g, 0.0))
        j = math.ceil(0.7 * M)
        t = 0.5 * (z0[j - 1] + z0[j])
        b = float(np.float32(math.log(TAU / (1.0 - TAU)) - t))
        out[str(M)] = b
        margins[str(M)] = float(0.5 * (z0[j] - z0[j - 1]))
    return out, margins


def main():
    b, margins = compute()
    doc = {
        "workload": "mixed-gate down_proj, K=14336, N=4096, r=64, seed 0",
        "tau": TAU,
        "b_g": b,
        "logit_margin": margins,
        "written_by": "tests/golden/make_gate_bias.py (oracle.gate_logits)",
    }
    path = os.path.join(HERE, "downproj_gate_bias.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=2)
        f.write("\n")
    print(json.dumps(doc, indent=2))


if __name__ == "__main__":
    main()
