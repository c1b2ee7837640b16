"""Pins for oracle.chain: the printed TPF/efficiency values, limits, and simulation."""
import json
import os

import numpy as np
import pytest

from oracle import chain


@pytest.fixture(scope="module")
def printed(golden_dir):
    with open(os.path.join(golden_dir, "printed_values.json")) as f:
        return json.load(f)


def test_printed_tpf_and_efficiency(printed):
    t = printed["tpf_n4_p09"]
    assert round(chain.tpf_closed_form(t["N"], t["p"]), t["decimals"]) == t["value"]
    e = printed["efficiency_n4_p09"]
    assert 2 * e["N"] - 1 == e["queries"] == printed["queries_per_forward_n4"]["value"]
    assert round(chain.efficiency(e["N"], e["p"]), e["decimals"]) == e["value"]


def test_sdar_efficiency_definition(printed):
    s = printed["sdar_efficiency"]
    # the definition TPF^2 / queries reproduces the printed value at a TPF that rounds to 1.1
    assert round(1.105 ** 2 / s["queries"], 2) == s["value"] and round(1.105, 1) == s["tpf"]


@pytest.mark.parametrize("N", [2, 3, 4, 6])
def test_limits(N):
    assert chain.tpf_closed_form(N, 1.0) == pytest.approx(N)        # everything accepted
    assert chain.tpf_closed_form(N, 0.0) == pytest.approx(1.0)      # plain AR pace
    ps = np.linspace(0, 1, 21)
    vals = [chain.tpf_closed_form(N, p) for p in ps]
    assert np.all(np.diff(vals) > 0)


def test_closed_form_values():
    # hand-evaluated: N=2: 2/(2-p); N=3: (2+p)/(2-p^2)
    assert chain.tpf_closed_form(2, 0.5) == pytest.approx(4 / 3)
    assert chain.tpf_closed_form(3, 0.9) == pytest.approx(2.9 / (2 - 0.81))
    assert chain.tpf_closed_form(4, 0.9) == pytest.approx(3.71 / 1.271)


@pytest.mark.parametrize("N,p", [(2, 0.5), (2, 0.9), (3, 0.5), (3, 0.9), (4, 0.5), (4, 0.9)])
def test_chain_simulation_matches_closed_form(N, p):
    sim = chain.simulate_chain(N, p, steps=1000, chains=1000, seed=N * 10 + int(p * 10))
    assert abs(sim - chain.tpf_closed_form(N, p)) < 0.01


@pytest.mark.parametrize("N,p", [(3, 0.5), (4, 0.9)])
def test_renewal_estimator(N, p):
    rng = np.random.default_rng(1)
    acc = rng.random((400000, N - 1)) < p
    n = np.where(acc.all(1), N - 1, np.argmin(acc, 1))
    tpf, p_hat = chain.renewal_estimate(n, N)
    assert abs(p_hat - p) < 0.003
    assert abs(tpf - chain.tpf_closed_form(N, p_hat)) < 0.005
