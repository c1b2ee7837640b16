"""Proposal noise sd of the stride/concurrency sweep, by bisection on the oracle.

The sweep runs at two acceptance rates, 0.5 and 0.9 (the tokens-per-forward regimes of
「I-DLM – introspektive Diffusion Language Models」 "Speedup Factor Explorer").  The
proposal rows are anchor + N(0, sigma), anchors N(0, 3), vocabulary 151936, bf16.  For
each target this bisects sigma until the mean of oracle.verify.expected_acceptance over
the draft rows of the sweep point (N=4, B=64) with the sweep's seed is within 0.002 of
the target (the noise draw is the same for every sigma, so the mean falls as sigma
grows).  Writes sweep_sigma.json next to this file.  Calls only oracle/ and the seeded
input generator.

    python tests/golden/sweep_sigma.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from strided_verify_propose_amd import synth  # noqa: E402

TOL = 0.002


sweep_index = synth.sweep_index


def mean_acceptance(sigma, N, B, p):
    cfg = synth.sweep_config(N, B, sigma, sweep_index(N, B, p))
    v = synth.verify_inputs(cfg)
    acc = [oracle.verify.expected_acceptance(v.logits[b, i], v.draft_logits[b, i])
           for b in range(B) for i in range(N - 1)]
    return float(np.mean(acc)), len(acc)


def calibrate(p, N=4, B=64):
    lo, hi = 0.01, 6.0                      # acceptance(lo) > p > acceptance(hi)
    for it in range(40):
        mid = 0.5 * (lo + hi)
        m, n = mean_acceptance(mid, N, B, p)
        print(f"  p={p}: sigma {mid:.5f} -> mean acceptance {m:.5f} over {n} rows", flush=True)
        if abs(m - p) <= TOL:
            return mid, m, n
        if m > p:
            lo = mid
        else:
            hi = mid
    raise RuntimeError("bisection did not converge")


def main():
    out = {"source": "tests/golden/sweep_sigma.py (bisection on oracle.verify.expected_acceptance)",
           "vocab": 151936, "anchor_sd": 3.0, "tolerance": TOL, "points": {}}
    for p in (0.5, 0.9):
        sigma, m, n = calibrate(p)
        out["points"][str(p)] = {"sigma": round(sigma, 6), "mean_acceptance": round(m, 6),
                                 "rows": n, "seed": 1200 + sweep_index(4, 64, p)}
    with open(os.path.join(HERE, "sweep_sigma.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
