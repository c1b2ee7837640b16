"""The sweep's calibrated proposal noise (synth.SWEEP_SIGMA) is the one the committed
bisection on the oracle found (tests/golden/sweep_sigma.json), and it gives the target
acceptance on the oracle; the acceptance rate itself is pinned by closed cases and a
Monte-Carlo run of the accept test."""
import json
import os

import numpy as np

import oracle
from strided_verify_propose_amd import synth


def test_synth_sigma_is_the_bisected_one(golden_dir):
    with open(os.path.join(golden_dir, "sweep_sigma.json")) as f:
        g = json.load(f)
    for p, rec in g["points"].items():
        assert synth.SWEEP_SIGMA[float(p)] == rec["sigma"]
        assert abs(rec["mean_acceptance"] - float(p)) <= g["tolerance"]
        assert rec["seed"] == 1200 + synth.sweep_index(4, 64, float(p))


def test_sigma_gives_the_target_on_a_few_rows():
    # 2 requests x 3 draft rows of the p = 0.9 point: per-row acceptance near 0.9
    v = synth.verify_inputs(synth.sweep_point(4, 1, 0.9))
    acc = [oracle.verify.expected_acceptance(v.logits[0, i], v.draft_logits[0, i]) for i in range(3)]
    assert all(abs(a - 0.9) < 0.02 for a in acc), acc


def test_expected_acceptance_closed_cases():
    rng = np.random.default_rng(3)
    row = rng.standard_normal(50)
    assert abs(oracle.verify.expected_acceptance(row, row) - 1.0) < 1e-12
    a = np.full(6, -1e3)
    b = np.full(6, -1e3)
    a[0] = 0.0
    b[5] = 0.0
    assert oracle.verify.expected_acceptance(a, b) < 1e-300     # disjoint supports


def test_expected_acceptance_matches_monte_carlo():
    """d ~ q~, accept iff u < min(1, p(d)/q~(d)): the accepted fraction of 2e5 draws."""
    rng = np.random.default_rng(4)
    anc, dft = rng.standard_normal(8) * 1.5, rng.standard_normal(8) * 1.5
    p = np.exp(anc - anc.max()); p /= p.sum()
    q = np.exp(dft - dft.max()); q /= q.sum()
    n = 200_000
    d = rng.choice(8, size=n, p=q)
    u = rng.random(n)
    frac = float(np.mean(u < np.minimum(1.0, p[d] / q[d])))
    e = oracle.verify.expected_acceptance(anc, dft)
    assert abs(frac - e) < 4 * np.sqrt(e * (1 - e) / n)
