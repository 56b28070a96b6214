"""Writes tests/golden/tiny_fp32_seed0.json from the oracle alone.

The paper prints no worked example for the Muon step, so this fixture is an
oracle-written regression anchor for the tiny fp32 workload (4 matrices of
64x128, grads then momentum drawn N(0,1) from numpy default_rng(0), lr 0.02,
beta 0.95, Nesterov, 5 quintic NS steps, params zero). Run:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import workloads  # noqa: E402


def main():
    w = workloads.WORKLOADS["tiny_fp32"]
    out = {"workload": w.description, "lr": w.lr, "beta": w.beta, "ns_steps": w.ns_steps,
           "scale_rule": "rms", "rms_target": 0.2, "matrices": []}
    for gi, j, r, c in w.matrices():
        g = workloads.grad(w, gi, j).as_f64()
        b = workloads.momentum(w, gi, j).astype(np.float64)
        p = workloads.params(w, gi, j).as_f64()
        p1, b1, o = oracle.muon_matrix_step(p, g, b, w.lr, w.beta, w.ns_steps)
        out["matrices"].append({
            "index": j,
            "p1_first_row_8": [float(v) for v in p1[0, :8]],
            "p1_frobenius": float(np.linalg.norm(p1)),
            "momentum1_first_row_8": [float(v) for v in b1[0, :8]],
            "o_singular_values_min_max": [float(v) for v in np.linalg.svd(o, compute_uv=False)[[-1, 0]]],
        })
    with open(os.path.join(HERE, "tiny_fp32_seed0.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
