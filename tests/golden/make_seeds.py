"""Pick the route seed of every workload (and the Zipf strength of the skewed one).

Writes tests/golden/seeds.json.  Uses only the CPU oracle (router, top-k,
permutation) and the seeded input generator.

Rule: starting from the workload's base seed, the first seed for which every
token's k-th and (k+1)-th largest router logits differ by more than 1e-3
(fp64), so that the top-k set cannot depend on fp32 rounding.  For the
batched-verify workload (Zipf(s=1.1) expert popularity) the bias strength
beta is chosen by bisection so that the busiest expert receives 35..45 of the
T tokens (target 40) while some experts receive none.

Run:  python tests/golden/make_seeds.py
"""
from __future__ import annotations

import json
import os
import sys
from dataclasses import replace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle  # noqa: E402
from synth import synth  # noqa: E402

GAP = 1e-3
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "seeds.json")


def routing(cfg, beta=None):
    x, wr = synth.routing_inputs(cfg, beta)
    logits = oracle.router(x, wr)
    idx, gates, gap = oracle.topk(logits, cfg.k)
    offsets, _, _ = oracle.permute(idx, cfg.E)
    counts = np.diff(offsets)
    return gap, counts


def calibrate_beta(cfg, target=40, lo=0.0, hi=4.0, iters=24):
    """Smallest-error beta with max per-expert count near `target`."""
    best = None
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        _, counts = routing(cfg, mid)
        m = int(counts.max())
        if best is None or abs(m - target) < abs(best[1] - target):
            best = (mid, m)
        if m == target:
            break
        if m < target:
            lo = mid
        else:
            hi = mid
    return best[0]


def main():
    rec = {}
    for name in synth.config_names():
        base = synth._BASE[name]
        s = base.seed
        while True:
            cfg = replace(base, route_seed=s)
            beta = 0.0
            if cfg.zipf_s is not None:
                beta = calibrate_beta(cfg)
                cfg = replace(cfg, zipf_beta=beta)
            gap, counts = routing(cfg, beta if cfg.zipf_s is not None else None)
            ok = gap > GAP
            if cfg.zipf_s is not None:
                ok = ok and 35 <= counts.max() <= 45 and (counts == 0).any()
            print(f"{name}: seed {s} gap {gap:.3e} max count {counts.max()} active {(counts > 0).sum()}"
                  + (f" beta {beta:.5f}" if cfg.zipf_s is not None else "") + (" OK" if ok else ""), flush=True)
            if ok:
                rec[name] = {"base_seed": base.seed, "route_seed": s, "min_gap": gap,
                             "active_experts": int((counts > 0).sum()), "max_count": int(counts.max())}
                if cfg.zipf_s is not None:
                    rec[name]["zipf_beta"] = beta
                    rec[name]["zero_count_experts"] = int((counts == 0).sum())
                break
            s += 1
    rec["_rule"] = ("route_seed: first seed >= base_seed with every token's k-th minus (k+1)-th fp64 router "
                    "logit > 1e-3 (oracle router); zipf_beta: bisection so the busiest expert gets 35..45 tokens")
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
