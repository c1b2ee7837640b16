"""Pins for oracle.verify: exact laws, closed forms, brute force, library routines."""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax
from scipy.stats import binomtest, chisquare

import oracle
from oracle.verify import verify
from strided_verify_propose_amd import synth


def u24(rng, shape):
    return (rng.integers(0, 1 << 24, size=shape) / float(1 << 24)).astype(np.float32)


def draw(rng, probs, n):
    return rng.choice(len(probs), size=n, p=probs / probs.sum()).astype(np.int32)


def law_case(kind, V=8, seed=0):
    """(p logits, q~ logits or None, fixed argmax draft or None) for a V-token vocab."""
    rng = np.random.default_rng(seed)
    lp = rng.standard_normal(V) * 1.2
    lq = lp + rng.standard_normal(V) * 0.9
    if kind == "q_equals_p":
        lq = lp.copy()
    elif kind == "q_zero_where_p_positive":
        lq[[1, 4]] = -1000.0
    elif kind == "p_zero_where_q_positive":
        lp[[2, 5]] = -1000.0
        lq[[2, 5]] = 2.0
    elif kind == "onehot":
        return lp.astype(np.float32), None
    return lp.astype(np.float32), lq.astype(np.float32)


def run_first_token(lp, lq, n, seed, N=2):
    """Batch of n independent requests sharing p and q~; returns emitted first tokens."""
    rng = np.random.default_rng(seed)
    V = lp.size
    R = 2 * N - 1
    logits = np.tile(rng.standard_normal((1, R, V)).astype(np.float32), (n, 1, 1))
    logits[:, :N - 1] = lp
    if lq is None:
        d = np.full((n, N - 1), int(np.argmax(lp + 0.3 * np.arange(V))), np.int32)   # a fixed draft
        draft_logits = None
    else:
        q = softmax(lq.astype(np.float64))
        d = np.stack([draw(rng, q, n) for _ in range(N - 1)], 1)
        draft_logits = np.tile(lq, (n, N - 1, 1))
    u = u24(rng, (n, R))
    res = verify(logits, draft_logits, d, u, N)
    first = np.where(res["accept"][:, 0] == 1, d[:, 0], res["next_token"])
    return first, res, d


@pytest.mark.parametrize("kind", ["random", "q_equals_p", "q_zero_where_p_positive",
                                  "p_zero_where_q_positive", "onehot"])
def test_emitted_token_follows_anchor_distribution(kind):
    """min(1, p/q) acceptance plus residual resampling emits exactly p (chi-square, V=8)."""
    seeds = {"random": 1, "q_equals_p": 2, "q_zero_where_p_positive": 3,
             "p_zero_where_q_positive": 4, "onehot": 5}
    lp, lq = law_case(kind, seed=seeds[kind])
    n = 60000
    first, _, _ = run_first_token(lp, lq, n, seed=42)
    p = softmax(lp.astype(np.float64))
    counts = np.bincount(first, minlength=lp.size)
    zero = p < 1e-300
    assert counts[zero].sum() == 0
    assert chisquare(counts[~zero], p[~zero] * n).pvalue > 1e-3


def test_second_position_law_given_first_accepted():
    """Given draft 0 accepted, the token emitted at position 1 follows p_1."""
    rng = np.random.default_rng(5)
    V, N, n = 8, 3, 60000
    lp0, lq0 = rng.standard_normal(V), rng.standard_normal(V)
    lp1, lq1 = rng.standard_normal(V) * 1.5, rng.standard_normal(V)
    logits = np.tile(rng.standard_normal((1, 5, V)), (n, 1, 1)).astype(np.float32)
    logits[:, 0], logits[:, 1] = lp0, lp1
    dl = np.tile(np.stack([lq0, lq1]).astype(np.float32), (n, 1, 1))
    d = np.stack([draw(rng, softmax(lq0), n), draw(rng, softmax(lq1), n)], 1)
    res = verify(logits, dl, d, u24(rng, (n, 5)), N)
    sel = res["accept"][:, 0] == 1
    tok = np.where(res["accept"][sel, 1] == 1, d[sel, 1], res["next_token"][sel])
    p1 = softmax(logits[0, 1].astype(np.float64))
    assert chisquare(np.bincount(tok, minlength=V), p1 * sel.sum()).pvalue > 1e-3


def test_q_identical_to_p_accepts_everything():
    v = synth.verify_inputs(synth.StepConfig("t", "bf16", B=6, N=4, Hq=1, Hkv=1, D=64, V=5000,
                                             ctx=("fixed", 0), anchor_sd=3, noise_sd=0.3, seed=9))
    logits = v.logits.copy()
    logits[:, :3] = v.draft_logits                   # anchor rows equal the draft rows
    res = verify(logits, v.draft_logits, v.draft_ids, v.uniforms, 4)
    assert np.all(res["n_accept"] == 3) and np.all(res["accept"] == 1)
    np.testing.assert_allclose(res["p_draft"], res["q_draft"], rtol=0, atol=0)


def test_onehot_draft_closed_form():
    """Argmax drafts: P(accept) = p(d); the residual is p restricted to ids != d."""
    rng = np.random.default_rng(6)
    V, n = 8, 50000
    lp = (rng.standard_normal(V) * 1.2).astype(np.float32)
    p = softmax(lp.astype(np.float64))
    d_fix = 3
    logits = np.tile(rng.standard_normal((1, 3, V)).astype(np.float32), (n, 1, 1))
    logits[:, 0] = lp
    d = np.full((n, 1), d_fix, np.int32)
    res = verify(logits, None, d, u24(rng, (n, 3)), 2)
    acc = int(res["accept"][:, 0].sum())
    assert binomtest(acc, n, p[d_fix]).pvalue > 1e-3
    np.testing.assert_allclose(res["p_draft"][:, 0], p[d_fix], rtol=1e-12)
    assert np.all(res["q_draft"] == 1.0)
    rej = res["accept"][:, 0] == 0
    counts = np.bincount(res["next_token"][rej], minlength=V)
    assert counts[d_fix] == 0
    ref = np.delete(p, d_fix) / (1 - p[d_fix]) * rej.sum()
    assert chisquare(np.delete(counts, d_fix), ref).pvalue > 1e-3


def brute_inverse_cdf(weights, u):
    tot = math.fsum(weights)
    acc = 0.0
    for k, w in enumerate(weights):
        acc += w
        if acc > u * tot:
            return k
    return max(k for k, w in enumerate(weights) if w > 0)


def test_samples_and_bonus_match_brute_force():
    cfg = synth.StepConfig("t", "f32", B=40, N=3, Hq=1, Hkv=1, D=64, V=300,
                           ctx=("fixed", 0), anchor_sd=2, noise_sd=0.1, seed=21)
    v = synth.verify_inputs(cfg)
    res = verify(v.logits, v.draft_logits, v.draft_ids, v.uniforms, 3)
    full = 0
    for b in range(cfg.B):
        for j in range(3):
            row = v.logits[b, 2 + j].astype(np.float64)
            w = [math.exp(x - row.max()) for x in row]
            assert res["sampled_ids"][b, j] == brute_inverse_cdf(w, float(v.uniforms[b, 2 + j]))
        if res["n_accept"][b] == 2:
            full += 1
            assert res["next_token"][b] == res["sampled_ids"][b, 0]
    assert 0 < full < cfg.B


def test_residual_matches_hand_computation():
    """Rejected draft: next token = inverse CDF of max(0, p - q~) at (u - a)/(1 - a)."""
    rng = np.random.default_rng(8)
    V = 12
    for trial in range(200):
        lp, lq = rng.standard_normal(V).astype(np.float32), rng.standard_normal(V).astype(np.float32)
        logits = rng.standard_normal((1, 3, V)).astype(np.float32)
        logits[0, 0] = lp
        d = np.array([[rng.integers(V)]], np.int32)
        u = u24(rng, (1, 3))
        res = verify(logits, lq[None, None, :], d, u, 2)
        p = softmax(lp.astype(np.float64))
        q = softmax(lq.astype(np.float64))
        a = min(1.0, p[d[0, 0]] / q[d[0, 0]])
        if float(u[0, 0]) < a:
            assert res["accept"][0, 0] == 1 and res["n_accept"][0] == 1
            continue
        assert res["n_accept"][0] == 0
        w = [max(0.0, pi - qi) for pi, qi in zip(p, q)]
        up = (float(u[0, 0]) - a) / (1 - a)
        assert res["next_token"][0] == brute_inverse_cdf(w, up)


def test_lse_matches_scipy():
    cfg = synth.StepConfig("t", "bf16", B=3, N=3, Hq=1, Hkv=1, D=64, V=20000,
                           ctx=("fixed", 0), anchor_sd=3, noise_sd=0.3, seed=2)
    v = synth.verify_inputs(cfg)
    res = verify(v.logits, v.draft_logits, v.draft_ids, v.uniforms, 3, temperature=0.7)
    rows = np.concatenate([oracle.stored.to_f64(v.logits), oracle.stored.to_f64(v.draft_logits)], 1)
    np.testing.assert_allclose(res["row_lse"], logsumexp(rows / 0.7, axis=-1), rtol=1e-13)


def test_argmax_lowest_id_on_ties():
    V = 1000
    logits = np.zeros((2, 3, V), np.uint16)
    top = synth.bf16_rne(np.float32(5.0))[0]
    logits[0, 1, [17, 400, 999]] = top
    logits[0, 2, [998, 999]] = top
    logits[1, 1, 0] = top
    logits[1, 2, [3, 2, 1]] = synth.bf16_rne(np.array([4.0, 5.0, 5.0], np.float32))
    res = verify(logits, None, np.zeros((2, 1), np.int32), np.full((2, 3), 0.5, np.float32), 2)
    assert res["argmax_ids"].tolist() == [[17, 998], [0, 1]]


def test_temperature_scales_logits():
    cfg = synth.StepConfig("t", "f32", B=8, N=3, Hq=1, Hkv=1, D=64, V=500,
                           ctx=("fixed", 0), anchor_sd=2, noise_sd=0.4, seed=4)
    v = synth.verify_inputs(cfg)
    a = verify(v.logits, v.draft_logits, v.draft_ids, v.uniforms, 3, temperature=2.0)
    b = verify(v.logits / np.float32(2), v.draft_logits / np.float32(2), v.draft_ids, v.uniforms, 3)
    for key in ("n_accept", "next_token", "sampled_ids", "accept"):
        assert np.array_equal(a[key], b[key])
    np.testing.assert_allclose(a["p_draft"], b["p_draft"], rtol=1e-12)


def test_near_threshold_draws_are_flagged():
    V = 16
    rng = np.random.default_rng(3)
    lp, lq = rng.standard_normal(V).astype(np.float32), rng.standard_normal(V).astype(np.float32)
    logits = np.tile(rng.standard_normal((1, 3, V)).astype(np.float32), (3, 1, 1))
    logits[:, 0] = lp
    d = np.array([[int(np.argmax(lq - lp))]] * 3, np.int32)      # a draft with p < q
    probe = verify(logits[:1], lq[None, None], d[:1], np.full((1, 3), 0.5, np.float32), 2)
    a = probe["accept_prob"][0, 0]
    assert a < 1
    u = np.full((3, 3), 0.5, np.float32)
    u[0, 0] = np.float32(a) + np.float32(2e-7)       # just above the threshold -> rejected, flagged
    u[1, 0] = np.float32(a) - np.float32(2e-7)       # just below -> accepted, flagged
    u[2, 0] = np.float32(min(a + 0.05, 0.99))        # far -> unflagged
    res = verify(logits, np.tile(lq, (3, 1, 1)), d, u, 2)
    assert res["accept_flag"][:, 0].tolist() == [True, True, False]
    assert res["accept"][:, 0].tolist() == [0, 1, 0]
    # a sample drawn exactly on a CDF boundary is flagged too
    row = logits[0, 1].astype(np.float64)
    c = np.cumsum(np.exp(row - row.max()))
    u2 = np.full((1, 3), 0.25, np.float32)
    u2[0, 1] = np.float32(c[4] / c[-1])
    res2 = verify(logits[:1], lq[None, None], d[:1], u2, 2)
    assert res2["sample_flag"][0, 0]
