"""Calibrate the Zipf skew constant of the skewed decode-like workload.

TEST INFRASTRUCTURE (writes an input parameter, never an expected value).
Centroid norms are scaled by 1 + c * rank^(-s) (s = 1.2, ranks a seeded
permutation).  With K experts chosen per token one expert can take at most
1/K of all assignments, so an exact Zipf(1.2) load (top expert 65x the mean)
cannot occur; the constant c is bisected until the initial max/mean expert
load, routed by the oracle with zero bias, lies in [9.5, 10.5] ("hot experts
about 10x the mean").  Run:  python -m oracle.calibrate_skew
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from moe_workloads import CONFIGS, make_inputs, to_numpy_f32  # noqa: E402
from moe_workloads.generate import make_centroids, _SKEW_FILE  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402


def load_ratio(cfg, seed, c, u):
    E = to_numpy_f32(make_centroids(cfg, seed, skew_c=c))
    idx = O.select_topk(O.affinities(u, E), np.zeros(cfg.n_routed, np.float32), cfg.top_k)["idx"]
    counts = np.bincount(idx.ravel(), minlength=cfg.n_routed)
    return counts.max() / counts.mean(), counts


def main(name="skew_decode_d7168", seed=0):
    cfg = CONFIGS[name]
    u = to_numpy_f32(make_inputs(cfg.replace(zipf_s=None), seed, with_weights=False).u)  # u does not depend on the skew
    lo, hi = 0.0, 64.0
    for _ in range(60):
        c = 0.5 * (lo + hi)
        ratio, counts = load_ratio(cfg, seed, c, u)
        print(f"c={c:.6f} max/mean={ratio:.3f}", flush=True)
        if 9.5 <= ratio <= 10.5:
            break
        if ratio < 9.5:
            lo = c
        else:
            hi = c
    else:
        raise SystemExit("calibration did not converge")
    table = json.load(open(_SKEW_FILE)) if os.path.exists(_SKEW_FILE) else {}
    table[f"{name}/seed{seed}"] = {"c": c, "initial_max_over_mean": float(ratio),
                                   "initial_max": int(counts.max()), "mean": float(counts.mean()),
                                   "experts_touched": int((counts > 0).sum())}
    with open(_SKEW_FILE, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(table)


if __name__ == "__main__":
    main()
