"""Pins for the closed decoding loop in the oracle: cold requests in verification and
the commit step (the hot/cold chain of tokens per forward)."""
import numpy as np
from scipy.special import softmax
from scipy.stats import chisquare

import oracle
from oracle.verify import commit, verify


def u24(rng, shape):
    return (rng.integers(0, 1 << 24, size=shape) / float(1 << 24)).astype(np.float32)


def test_cold_request_draws_row0_exactly():
    """A cold request emits one token distributed as p_0 (chi-square over 20000
    requests) and accepts nothing; hot requests in the same batch are unaffected."""
    rng = np.random.default_rng(11)
    N, V, n = 3, 8, 20000
    R = 2 * N - 1
    base = rng.standard_normal((1, R, V)).astype(np.float32) * 1.3
    logits = np.tile(base, (n, 1, 1))
    dl = np.tile(rng.standard_normal((1, N - 1, V)).astype(np.float32), (n, 1, 1))
    d = rng.integers(0, V, size=(n, N - 1)).astype(np.int32)
    d[::2] = -1                                   # even requests cold
    u = u24(rng, (n, R))
    res = verify(logits, dl, d, u, N)
    cold = np.arange(n) % 2 == 0
    assert (res["n_accept"][cold] == 0).all() and (res["accept"][cold] == 0).all()
    assert (res["p_draft"][cold] == 0).all()
    p0 = softmax(base[0, 0].astype(np.float64))
    counts = np.bincount(res["next_token"][cold], minlength=V)
    assert chisquare(counts, p0 * counts.sum()).pvalue > 1e-4
    # the same requests made hot (any valid draft) keep their proposals and samples
    d_hot = np.where(d < 0, 0, d)
    res_hot = verify(logits, dl, d_hot, u, N)
    assert np.array_equal(res["sampled_ids"], res_hot["sampled_ids"])
    assert np.array_equal(res["argmax_ids"], res_hot["argmax_ids"])
    assert np.array_equal(res["next_token"][~cold], res_hot["next_token"][~cold])


def test_cold_next_token_brute_force():
    """Pure-Python inverse CDF of softmax(row 0) at u_0."""
    rng = np.random.default_rng(12)
    N, V, B = 4, 50, 30
    logits = rng.standard_normal((B, 2 * N - 1, V)).astype(np.float32) * 2
    d = np.full((B, N - 1), -1, np.int32)
    u = u24(rng, (B, 2 * N - 1))
    res = verify(logits, None, d, u, N)
    for b in range(B):
        z = [float(x) for x in logits[b, 0]]
        m = max(z)
        w = [np.exp(x - m) for x in z]
        tot, acc, k = sum(w), 0.0, None
        for i, wi in enumerate(w):
            acc += wi
            if acc > float(u[b, 0]) * tot:
                k = i
                break
        assert res["next_token"][b] == k


def test_commit_hand_cases():
    """Hot with every draft accepted, hot with a rejection, cold."""
    N = 4
    n_accept = np.array([3, 1, 0])
    next_token = np.array([70, 71, 72])
    sampled = np.array([[70, 11, 12, 13], [80, 21, 22, 23], [90, 31, 32, 33]])
    drafts = np.array([[1, 2, 3], [4, 5, 6], [-1, -1, -1]])
    ctx = np.array([100, 200, 300])
    ctx2, nxt, toks, cnt = commit(n_accept, next_token, sampled, drafts, ctx, N)
    assert ctx2.tolist() == [104, 202, 301]
    assert nxt.tolist() == [[11, 12, 13], [-1, -1, -1], [31, 32, 33]]
    assert toks.tolist() == [[1, 2, 3, 70], [4, 71, -1, -1], [72, -1, -1, -1]]
    assert cnt.tolist() == [4, 2, 1]


def test_loop_tokens_per_forward_match_closed_form():
    """Verification and commit in a closed loop on synthetic rows -- each anchor row is
    the previous step's [MASK] row plus noise -- emit tokens at the rate of the hot/cold
    chain: the measured tokens per forward equal the closed form at the measured
    acceptance rate, within 4 standard errors over independent requests."""
    rng = np.random.default_rng(13)
    N, V, B, steps = 3, 64, 400, 40
    R = 2 * N - 1
    drafts = np.full((B, N - 1), -1, np.int32)
    dl = np.zeros((B, N - 1, V), np.float32)
    ctx = np.zeros(B, np.int32)
    emitted = np.zeros(B)
    acc = np.zeros(B)
    evald = np.zeros(B)
    for _ in range(steps):
        logits = (rng.standard_normal((B, R, V)) * 2).astype(np.float32)
        hot = drafts[:, 0] >= 0
        logits[hot, :N - 1] = dl[hot] + (rng.standard_normal((int(hot.sum()), N - 1, V)) * 0.5).astype(np.float32)
        u = u24(rng, (B, R))
        res = verify(logits, dl, drafts, u, N)
        n = res["n_accept"]
        acc += np.where(hot, n, 0)
        evald += np.where(hot, n + (n < N - 1), 0)
        ctx, drafts, _, cnt = commit(n, res["next_token"], res["sampled_ids"], drafts, ctx, N)
        emitted += cnt
        dl = logits[:, N:].copy()
    p_hat = acc.sum() / evald.sum()
    per_req = emitted / steps
    tpf = per_req.mean()
    se = per_req.std(ddof=1) / np.sqrt(B)
    closed = oracle.tpf_closed_form(N, p_hat)
    assert abs(tpf - closed) < 4 * se + 0.02, (tpf, closed, se)   # + the start-up (cold) step
    assert (ctx == emitted).all()
