"""Calibrate the Zipf gate-bias scale tau of the 256-expert bf16 workload.

The workload's gate bias is b[e] = -tau * ln(e + 1). This script finds, by
bisection on [0, 10], the tau for which the least-squares slope of
log(count_e) against log(e + 1) is -1 (Zipf exponent s = 1), with the counts
taken from the oracle's top-k selection on the first 8192 tokens of the
workload. It writes datagen/zipf_tau.json. Run: python tests/golden/calibrate_zipf_tau.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import datagen as dg  # noqa: E402
import oracle  # noqa: E402

ROWS = 8192


def zipf_slope(w, inp, tau):
    inp = dict(inp)
    inp["gate_bias"] = dg.gate_bias(w, tau)
    sel = oracle.gate(inp, w.k, rows=np.arange(ROWS))["topk_idx"]
    counts = np.bincount(sel.ravel(), minlength=w.n_experts)
    ranks = np.arange(1, w.n_experts + 1)
    ok = counts > 0
    slope = np.polyfit(np.log(ranks[ok]), np.log(counts[ok]), 1)[0]
    return slope, counts


def main():
    w = dg.WORKLOADS["zipf_bf16_n256"]
    inp = dg.make_inputs(dg.workload(w.name, tokens=ROWS), experts=False, gate_bias_tau=0.0)
    lo, hi = 0.0, 10.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        s, _ = zipf_slope(w, inp, mid)
        if s > -1.0:
            lo = mid
        else:
            hi = mid
    tau = 0.5 * (lo + hi)
    s, counts = zipf_slope(w, inp, tau)
    out = {"tau": round(tau, 6), "slope": round(float(s), 4), "rows": ROWS,
           "max_count": int(counts.max()), "min_count": int(counts.min()),
           "written_by": "tests/golden/calibrate_zipf_tau.py (oracle top-k selection)"}
    with open(os.path.join(ROOT, "datagen", "zipf_tau.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
