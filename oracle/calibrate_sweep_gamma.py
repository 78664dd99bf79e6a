"""Choose the routing scale gamma of each alpha / chunk-size point of the 16K sweep workload.

Uses only the oracle's Stage 0 and Stage 1 (on host-generated inputs of the sweep recipe, a
sample of query rows late enough to see many chunks) and bisects log(gamma) until the routed
fraction of candidate chunks meets the point's target. Writes tests/golden/sweep_gamma.json,
which the tests and the benchmark read as an input parameter.

    python -m oracle.calibrate_sweep_gamma
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle
import workloads as wl

OUT = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden",
                   "sweep_gamma.json")
# denser routing for the softer map, sparser for sparsemax: the sweep spans ~5% .. ~50%
TARGET = {1.25: 0.50, 1.5: 0.25, 2.0: 0.05}


def support_fraction(inp, kbar, w: wl.Workload, alpha, gamma, rows):
    st = oracle.block_entmax(inp["q"], kbar, n_kv=w.n_kv, block=w.block, alpha=alpha,
                             gamma=gamma, sigma=1e8, h_kv=w.h_kv, rows=rows)
    routed = (st["w"] > 0).sum()
    cand = sum(min((r % w.n_q) // w.block, w.n_kv // w.block) for r in rows) * w.h_kv
    return routed / max(1, cand)


def calibrate(alpha: float, block: int, rows_per_point: int = 48) -> dict:
    w = wl.sweep_workload(alpha, block, 1.0)
    inp = wl.make_inputs(w, "cpu")
    kbar = oracle.pool_keys(inp["k"], block)
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(np.arange(w.n_kv // 4, w.n_kv), size=rows_per_point, replace=False))
    lo, hi = math.log(1e-3), math.log(1e3)
    target = TARGET[alpha]
    for _ in range(30):  # support shrinks as gamma grows
        mid = 0.5 * (lo + hi)
        if support_fraction(inp, kbar, w, alpha, math.exp(mid), rows) > target:
            lo = mid
        else:
            hi = mid
    gamma = float(f"{math.exp(0.5 * (lo + hi)):.4g}")
    frac = support_fraction(inp, kbar, w, alpha, gamma, rows)
    return dict(alpha=alpha, block=block, gamma=gamma, target=target, measured=round(float(frac), 4))


def main():
    points = [calibrate(a, b) for a, b in wl.SWEEP_POINTS]
    for p in points:
        print(p)
    with open(OUT, "w") as f:
        json.dump(dict(about="gamma per (alpha, block) of the 16K sweep, chosen by "
                             "oracle/calibrate_sweep_gamma.py from the oracle's Stage 1 on a sample "
                             "of rows; 'measured' is the routed fraction of candidate chunks there",
                       points=points), f, indent=1)


if __name__ == "__main__":
    main()
