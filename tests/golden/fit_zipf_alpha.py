"""Fit the router-gain exponent of the Zipf-skewed Qwen prefill workload.

Row e of the router weight is scaled by rho_e**-alpha (rho_e a seeded random
rank).  This script bisects alpha until the least-squares slope of
log(per-expert load) against log(load rank) is -1 (Zipf, s = 1.0) for seed 0,
using only the oracle's routing, and writes tests/golden/zipf_alpha.json.
The fitted value is copied into workloads/gen.py (ZIPF_ALPHA).

    python tests/golden/fit_zipf_alpha.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle.formats import decode                      # noqa: E402
from oracle.moe import permute, router_logits, topk_softmax  # noqa: E402
from workloads import CONFIGS, router_inputs, to_bits  # noqa: E402


def zipf_slope(counts: np.ndarray) -> float:
    c = np.sort(counts[counts > 0])[::-1].astype(np.float64)
    r = np.arange(1, c.size + 1, dtype=np.float64)
    return float(np.polyfit(np.log(r), np.log(c), 1)[0])


def loads(cfg, alpha, seed=0):
    x, wr = router_inputs(cfg, seed, zipf_alpha=alpha)
    l = router_logits(decode(to_bits(x), cfg.act_dtype), decode(to_bits(wr), cfg.act_dtype))
    idx, _ = topk_softmax(l, cfg.k)
    return permute(idx, cfg.E)[0]


def main():
    cfg = CONFIGS["qwen_prefill"]
    lo, hi = 0.0, 1.0
    for _ in range(16):
        mid = 0.5 * (lo + hi)
        s = zipf_slope(loads(cfg, mid))
        print(f"alpha={mid:.5f} slope={s:.4f}", flush=True)
        if s > -1.0:
            lo = mid
        else:
            hi = mid
    alpha = round(0.5 * (lo + hi), 4)
    c = loads(cfg, alpha)
    out = {"alpha": alpha, "slope": zipf_slope(c), "max": int(c.max()), "min": int(c.min()),
           "zero_load_experts": int((c == 0).sum()), "mean": float(c.mean()),
           "experts_at_least_312_rows": int((c >= 312).sum())}
    print(out)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_alpha.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
