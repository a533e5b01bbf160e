"""Fit the strength alpha of the static router bias that shapes expert load
toward Zipf(s): bias[e] = -alpha * s * ln(rank_e) over a seeded ranking.

For a given alpha the script routes a sample of seeded tokens with the CPU
oracle's router and top-k, counts assignments per expert, and fits the slope
of log(count) against log(rank) over ranks 9..E (ranks 1..k cannot follow
Zipf: one expert takes at most one assignment per token).  Bisection on alpha
makes that slope equal -s.  Writes moegen/zipf_alpha.json, which moegen reads.

    python moegen/fit_zipf_alpha.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import moegen  # noqa: E402
import oracle  # noqa: E402


def slope_for(alpha, w, T, layer=0):
    L = moegen.make_layer(moegen.Workload(**{**w.__dict__, "zipf_alpha": alpha, "I": 256,
                                             "fmt_down": moegen.FMT_NVFP4}), layer=layer)
    # only the router matters here; experts are not evaluated
    x = moegen.make_tokens(w, T, step=999)
    _, idx, _ = oracle.route(x, L)
    counts = np.bincount(idx.reshape(-1), minlength=w.E).astype(np.float64)
    _, rank = moegen.zipf_bias(moegen.key(w.seed, moegen.TAG_BIAS, layer, 0), w.E, w.zipf_s, alpha)
    sel = rank >= 9
    xs = np.log(rank[sel].astype(np.float64))
    ys = np.log(np.maximum(counts[sel], 0.5))
    return float(np.polyfit(xs, ys, 1)[0]), counts


def fit(name, T=4096, lo=0.05, hi=1.5, iters=14):
    w = moegen.WORKLOADS[name]
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        s, _ = slope_for(mid, w, T)
        if s > -w.zipf_s:   # not steep enough: more bias
            lo = mid
        else:
            hi = mid
    a = round(0.5 * (lo + hi), 4)
    s, counts = slope_for(a, w, T)
    return a, s, counts


if __name__ == "__main__":
    out = {}
    for name in ("prefill", "tiered"):
        a, s, counts = fit(name)
        srt = np.sort(counts)[::-1]
        out[name] = a
        print(f"{name}: alpha={a} slope={s:.3f} top-8 share={srt[:8].sum() / counts.sum():.3f} "
              f"min={int(counts.min())} max={int(counts.max())}")
    with open(os.path.join(ROOT, "moegen", "zipf_alpha.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
