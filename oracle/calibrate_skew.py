"""Find the Zipf bias strength of the hot-expert workload.

Bisection over alpha so that, at seed 0, the top 10% of experts receive 60%
of the routed assignments.  Routing is computed by the oracle only (logits,
softmax/top-k, permutation counts); the result is frozen as
expert_ffn_layer_amd.synth.SKEW_ALPHA so that input generation never runs
routing arithmetic.  Usage:  python -m oracle.calibrate_skew
"""
import dataclasses
import sys

import numpy as np

import oracle
from expert_ffn_layer_amd import synth


def stats(o, cfg, seed=0):
    lay = synth.make_layer(cfg, seed=seed, router_only=True)
    r = o.route(o.logits(lay.x, lay.wg, lay.bias), cfg.k, cfg.renorm)
    counts = o.permute(r["ids"], cfg.E)["counts"]
    top = np.sort(counts)[::-1][: int(0.1 * cfg.E)].sum() / cfg.A
    return float(top), int((counts <= 3).sum()), int(counts.max())


def main(target=0.60):
    o = oracle.Oracle()
    base = synth.CONFIGS["skew"]
    lo, hi = 0.0, 2.0
    for _ in range(20):
        mid = 0.5 * (lo + hi)
        share, _, _ = stats(o, dataclasses.replace(base, zipf_alpha=mid))
        lo, hi = (mid, hi) if share < target else (lo, mid)
    alpha = round(0.5 * (lo + hi), 3)
    share, light, mx = stats(o, dataclasses.replace(base, zipf_alpha=alpha))
    print(f"alpha={alpha} top10%-share={share:.4f} experts<=3 tokens={light} max rows={mx}")
    return alpha


if __name__ == "__main__":
    sys.exit(0 if main() is not None else 1)
