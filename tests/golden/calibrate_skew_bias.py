"""Finds the scale lambda of the skewed workload's Zipf-rank logit bias.

The skewed workload (T=16384, d=2048, E=256, top-8 softmax, shared expert)
asks for a per-expert logit bias drawn from a Zipf(s=1.1) popularity rank,
scaled so that the hottest expert gets about 10x the mean token count.
This script bisects lambda in [0, 8] on the workload's own seeded tokens and
router, using only the CPU oracle's routing, and prints the value stored as
``moe_workloads.SKEW_BIAS_SCALE`` together with the achieved ratio.

    python tests/golden/calibrate_skew_bias.py
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "..", ".."))

import moe_workloads as mw  # noqa: E402
from oracle import moe_oracle as mo  # noqa: E402


def ratio_for(inp, cfg, lam):
    bias = mw.skew_bias(cfg, lam)
    r = mo.route(inp.as_f32("x"), inp.as_f32("w_router"), cfg.k,
                 cfg.score, cfg.normalize, logit_bias=bias)
    mean = cfg.T * cfg.k / cfg.E
    return r.counts.max() / mean, r.counts.min()


def main(steps=20):
    cfg = mw.get("skew_shared")
    inp = mw.make_layer_inputs(cfg, with_experts=False)
    lo, hi = 0.0, 8.0
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        rt, _ = ratio_for(inp, cfg, mid)
        if rt < 10.0:
            lo = mid
        else:
            hi = mid
    best = min((lo, hi), key=lambda v: abs(ratio_for(inp, cfg, v)[0] - 10.0))
    rt, cmin = ratio_for(inp, cfg, best)
    print(f"lambda={best!r} hottest/mean={rt:.4f} coldest={cmin}")
    return best, rt


if __name__ == "__main__":
    main()
