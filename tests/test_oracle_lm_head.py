"""Pins of the LM-head oracle (CPU): logits = nearest bf16 of hidden . w_lm^T.

The oracle's product is checked against things other than itself: a one-hot special
case where each logit is a single stored weight, exact integer arithmetic on the
dyadic grid the parity inputs use, with ties-to-even rounding done on integers, and
exact rational arithmetic on tiny Gaussian inputs."""
from fractions import Fraction

import numpy as np

import oracle.lm_head as olm
from oracle.stored import to_f64
from oracle.verify import verify
from strided_verify_propose_amd import synth
from tests.test_oracle_proj import nearest_bf16_exact


def _bits(x32):
    return synth.bf16_rne(np.asarray(x32, np.float32))


def test_one_hot_rows_pick_one_weight_each():
    """hidden row m = c_m e_{k_m} (c_m a power of two): logit[m, v] = c_m w[v, k_m] exactly.
    V != Dm, so a transposed operand or a wrong index cannot pass."""
    rng = np.random.default_rng(3)
    M, Dm, V = 6, 40, 97
    w = _bits(rng.standard_normal((V, Dm)))
    ks = rng.integers(0, Dm, M)
    cs = 2.0 ** rng.integers(-3, 4, M)
    h = np.zeros((M, Dm), np.float32)
    h[np.arange(M), ks] = cs
    got = olm.lm_head_logits(_bits(h), w)
    want = to_f64(w)[:, ks].T * cs[:, None]
    assert got.shape == (M, V)
    assert np.array_equal(got, want)


def _rne_int(n, keep=8):
    """Nearest integer with `keep` significant bits, ties to even, on Python integers."""
    a = abs(int(n))
    if a < (1 << keep):
        return int(n)
    shift = a.bit_length() - keep
    q, rem = divmod(a, 1 << shift)
    half = 1 << (shift - 1)
    if rem > half or (rem == half and q % 2 == 1):
        q += 1
    return (q << shift) * (1 if n >= 0 else -1)


def test_grid_inputs_give_the_exact_product_rounded_to_bf16():
    cfg = synth.LmHeadConfig("pin", B=2, N=3, Dm=4096, V=300, h_sd=1, w_sd=1, draft_sd=3,
                             grid=True, seed=11)
    x = synth.lm_head_inputs(cfg)
    kh = np.rint(to_f64(x.hidden) * 4).astype(np.int64)          # hidden = kh / 4
    kw = np.rint(to_f64(x.w_lm) * 32).astype(np.int64)           # w = kw / 32
    assert np.array_equal(kh / 4.0, to_f64(x.hidden)) and np.array_equal(kw / 32.0, to_f64(x.w_lm))
    exact = kh @ kw.T                                             # logits * 128, integers
    want = np.vectorize(_rne_int)(exact) / 128.0
    got = olm.lm_head_logits(x.hidden, x.w_lm)
    assert np.array_equal(got, want)
    assert np.mean(want != exact / 128.0) > 0.05                  # rounding is exercised


def test_tiny_gaussian_product_matches_exact_rationals():
    rng = np.random.default_rng(5)
    M, Dm, V = 3, 7, 11
    h = _bits(rng.standard_normal((M, Dm)))
    w = _bits(rng.standard_normal((V, Dm)) * 0.1)
    H, W = to_f64(h), to_f64(w)
    got = olm.lm_head_logits(h, w)
    for m in range(M):
        for v in range(V):
            s = sum(Fraction(float(H[m, k])) * Fraction(float(W[v, k])) for k in range(Dm))
            assert got[m, v] == nearest_bf16_exact(s)


def test_rows_are_request_major():
    """hidden row b R + r feeds logits[b, r]: with one-hot rows, row (b, r)'s argmax is
    the vocabulary entry planted for it."""
    N, B, Dm = 3, 2, 16
    R, V = 2 * N - 1, 64
    w = np.zeros((V, Dm), np.float32)
    h = np.zeros((B * R, Dm), np.float32)
    target = np.arange(B * R) * 3 + 1
    for m in range(B * R):
        h[m, m % Dm] = 1.0
        w[target[m], m % Dm] += 8.0 + m
    rng = np.random.default_rng(0)
    logits, res = olm.lm_head_verify(_bits(h), _bits(w), None, np.zeros((B, N - 1), np.int32),
                                 rng.random((B, R), dtype=np.float32), N)
    assert logits.shape == (B, R, V)
    for b in range(B):
        for r in range(R):
            assert int(np.argmax(logits[b, r])) == target[b * R + r]
    assert np.array_equal(res["argmax_ids"], np.array([[target[b * R + N - 1 + j] for j in range(N)]
                                                       for b in range(B)]))


def test_fused_oracle_is_verification_of_the_stored_logits():
    cfg = synth.LmHeadConfig("pin", B=2, N=4, Dm=64, V=257, h_sd=1, w_sd=1, draft_sd=2,
                             grid=True, seed=12)
    x = synth.lm_head_inputs(cfg)
    logits, res = olm.lm_head_verify(x.hidden, x.w_lm, x.draft_logits, x.draft_ids, x.uniforms, cfg.N)
    ref = verify(_bits(logits.astype(np.float32)), x.draft_logits, x.draft_ids, x.uniforms, cfg.N)
    for k in ("n_accept", "accept", "next_token", "argmax_ids", "sampled_ids"):
        assert np.array_equal(res[k], ref[k]), k
