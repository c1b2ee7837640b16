"""Pins for oracle.proj (gated LoRA) and oracle.stored (bf16 rounding)."""
import math
from fractions import Fraction

import numpy as np

import oracle
from oracle.stored import round_bf16, to_f64
from strided_verify_propose_amd import synth


def nearest_bf16_exact(x):
    """Nearest bf16 to a Python float by exact rational arithmetic (ties to even)."""
    if x == 0:
        return 0.0
    f = Fraction(x)
    e = math.floor(math.log2(abs(x)))
    while Fraction(2) ** e > abs(f):
        e -= 1
    while Fraction(2) ** (e + 1) <= abs(f):
        e += 1
    ulp = Fraction(2) ** (e - 7)                 # 8 significant bits
    k = f / ulp
    lo = math.floor(k)
    r = k - lo
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return float(lo * ulp)


def test_round_bf16_is_nearest_ties_to_even():
    rng = np.random.default_rng(0)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-3, 4, 3000))
    # exact halfway points between neighbouring bf16 values
    base = to_f64(rng.integers(0x3C00, 0x4400, 500).astype(np.uint16))
    xs += list(base * (1 + 2.0 ** -9))
    got = round_bf16(np.array(xs))
    ref = np.array([nearest_bf16_exact(float(x)) for x in xs])
    assert np.array_equal(got, ref)


def brute_proj(X, W, A, Bm, gate):
    """Loops with math.fsum; the low-rank product rounded with the exact-rational rule."""
    M, K = X.shape
    Nout, r = W.shape[0], A.shape[0]
    Y = np.zeros((M, Nout))
    for m in range(M):
        t = [nearest_bf16_exact(math.fsum(X[m, k] * A[i, k] for k in range(K))) for i in range(r)]
        for n in range(Nout):
            y = math.fsum(X[m, k] * W[n, k] for k in range(K))
            if gate[m]:
                y = y + math.fsum(t[i] * Bm[n, i] for i in range(r))
            Y[m, n] = y
    return Y


def small_case(seed, M=6, K=24, Nout=10, r=4):
    rng = np.random.default_rng(seed)
    x = synth.bf16_rne(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_rne((rng.standard_normal((Nout, K)) * 0.3).astype(np.float32))
    a = synth.bf16_rne((rng.standard_normal((r, K)) * 0.3).astype(np.float32))
    b = synth.bf16_rne((rng.standard_normal((Nout, r)) * 0.3).astype(np.float32))
    gate = np.resize(np.array([0, 1, 1], np.uint8), M)
    return x, w, a, b, gate


def test_gated_proj_matches_brute_force():
    x, w, a, b, gate = small_case(1)
    Y = oracle.gated_lora_proj(x, w, a, b, gate)
    ref = brute_proj(to_f64(x), to_f64(w), to_f64(a), to_f64(b), gate)
    np.testing.assert_allclose(Y, ref, rtol=1e-12, atol=1e-12)


def test_ungated_rows_identical_to_base_only():
    x, w, a, b, gate = small_case(2, M=9)
    Y = oracle.gated_lora_proj(x, w, a, b, gate)
    Yb = oracle.gated_lora_proj(x, w)
    assert np.array_equal(Y[gate == 0], Yb[gate == 0])
    assert np.all(np.abs(Y[gate == 1] - Yb[gate == 1]).max(axis=1) > 0)


def test_base_only_is_a_plain_matmul_of_the_stored_values():
    x, w, _, _, _ = small_case(3, M=5, K=40, Nout=7)
    ref = np.array([[math.fsum(float(xi) * float(wi) for xi, wi in zip(to_f64(x)[m], to_f64(w)[n]))
                     for n in range(7)] for m in range(5)])
    np.testing.assert_allclose(oracle.gated_lora_proj(x, w), ref, rtol=1e-12, atol=1e-13)
