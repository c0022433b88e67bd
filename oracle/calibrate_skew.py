"""Calibrate the router-bias scale of the skewed Qwen3-235B-shaped workload.

Run:  python -m oracle.calibrate_skew   (writes datagen/skew_qwen235.json)

The workload asks for expert popularity with a Zipf(1.2) shape and a hottest
expert near 4x the mean load.  A pure Zipf(1.2) over 128 experts would put the
hottest at ~35x the mean, which top-8 cannot reach (at most 16x), so the
reading is: Zipf fixes the shape of the bias, b_e = -beta * 1.2 * ln(r_e) with
r a seeded permutation of 1..E, and the 4x target fixes beta.  beta is found by
bisection on the realised maximum load routed by the oracle (the load is
monotone in beta to within routing noise).  The 4.01x busiest-rank load of the
UltraEP page (section 结果) is the skew this mirrors.

Test infrastructure: calls only oracle/ and datagen/.
"""
import json
import os

import numpy as np

from datagen import configs, gen
from oracle import moe_oracle as O


def max_over_mean(logits0: np.ndarray, bias_unit: np.ndarray, beta: float, k: int, E: int) -> float:
    l = logits0 + (np.float32(beta) * bias_unit)[None, :].astype(np.float32)
    p = O.softmax32(l)
    ids, _, _ = O.topk(p, k)
    c = np.bincount(ids.reshape(-1), minlength=E)
    return float(c.max() / (ids.size / E))


def main(seed: int = 0, target: float = gen.HOT_RATIO) -> dict:
    w = configs.QWEN235
    d = gen.generate(w, seed=seed, beta=0.0)
    logits0 = O.router_logits(d["x"], d["w_router"], None)
    unit = gen.zipf_bias(w.E, 1.0, w.cfg_id, seed)      # beta = 1
    lo, hi = 0.0, 2.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        if max_over_mean(logits0, unit, mid, w.k, w.E) < target:
            lo = mid
        else:
            hi = mid
    beta = hi
    ratio = max_over_mean(logits0, unit, beta, w.k, w.E)
    l = logits0 + (np.float32(beta) * unit)[None, :]
    ids, _, _ = O.topk(O.softmax32(l), w.k)
    c = np.bincount(ids.reshape(-1), minlength=w.E)
    res = {"beta": beta, "zipf_s": gen.ZIPF_S, "target_ratio": target, "ratio": ratio,
           "max_count": int(c.max()), "min_count": int(c.min()), "seed": seed,
           "note": "written by oracle/calibrate_skew.py (oracle routing only)"}
    with open(gen.SKEW_FILE, "w") as f:
        json.dump(res, f, indent=1)
    return res


if __name__ == "__main__":
    print(main())
