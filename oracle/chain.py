"""Oracle: tokens per forward (TPF) of ISD.  (Test infrastructure.)

What it follows:
  * 「I-DLM – introspektive Diffusion Language Models」 "Speedup Factor Explorer": in the memory-bound regime the speedup is about
    TPF, given (with its exponents lost in extraction) as (2+p+...+p^(N-2)) / (2-p^(N-1)),
    and R-ISD's lossless speedup is about TPF / alpha.
  * 「首次超越 AR 模型」 "為什麼 I-DLM 能在高並發下保持高效" and 「I-DLM – introspektive Diffusion Language Models」 "Durchsatz (Throughput)":
    compute efficiency is TPF^2 / query count, with 2N-1 queries per forward for ISD.

The closed form is what a two-state chain gives, which `simulate_chain` runs:
  hot  -- N-1 valid drafts.  Each is accepted with probability p until the first
          rejection; the step emits (accepted + 1) tokens (residual or bonus token).
          All accepted -> stay hot, else -> cold (the new proposals were made after
          a token that was just rejected).
  cold -- no valid drafts: the step emits 1 exact token and N-1 fresh drafts -> hot.
Stationary: pi_hot = 1/(2 - p^(N-1)); TPF = pi_hot (1 + p + ... + p^(N-1)) + pi_cold.
"""
import numpy as np


def tpf_closed_form(N, p):
    """(2 + p + ... + p^(N-2)) / (2 - p^(N-1)) for N >= 2; 1 for N = 1 (plain AR)."""
    if N == 1:
        return 1.0
    num = 2.0 + sum(p ** k for k in range(1, N - 1))
    return num / (2.0 - p ** (N - 1))


def efficiency(N, p, queries=None):
    """TPF^2 / queries per forward (2N-1 for ISD)."""
    q = 2 * N - 1 if queries is None else queries
    return tpf_closed_form(N, p) ** 2 / q


def simulate_chain(N, p, steps, chains=1000, seed=0):
    """Tokens per step of the hot/cold chain, run for `steps` steps on each of
    `chains` independent chains (vectorised over chains).  Returns the pooled mean."""
    rng = np.random.default_rng(seed)
    hot = np.zeros(chains, bool)          # every chain starts cold (no drafts yet)
    tokens = 0
    for _ in range(steps):
        acc = rng.random((chains, N - 1)) < p
        k = np.where(acc.all(axis=1), N - 1, np.argmin(acc, axis=1))   # accepted prefix
        emitted = np.where(hot, k + 1, 1)
        tokens += int(emitted.sum())
        hot = np.where(hot, k == N - 1, True)
    return tokens / (steps * chains)


def renewal_estimate(n_accept, N):
    """(TPF_hat, p_hat) from the accepted-prefix lengths of hot steps.

    Each hot step emits n+1 tokens and, when it rejected (n < N-1), is followed by one
    cold step emitting 1 token:  TPF_hat = (mean(n+1) + r) / (1 + r), r = P(n < N-1).
    p_hat = accepted drafts / evaluated drafts, evaluated = n + [n < N-1]."""
    n = np.asarray(n_accept, dtype=np.float64).ravel()
    rej = (n < N - 1).astype(np.float64)
    r = rej.mean()
    tpf = (np.mean(n + 1) + r) / (1 + r)
    evaluated = np.sum(n + rej)
    p_hat = np.sum(n) / evaluated if evaluated > 0 else 1.0
    return tpf, p_hat
