"""Kernel-driven tokens per forward.

Over the stride sweep (N in {2, 3, 4}, acceptance near 0.5 and 0.9, 64 requests, the
Qwen3-8B vocabulary), the renewal estimate of TPF taken on isd_verify's own n_accept
must match the closed form (2 + p + ... + p^(N-2)) / (2 - p^(N-1)) of the
「I-DLM – introspektive Diffusion Language Models」 page, section "Speedup Factor
Explorer", at the measured acceptance rate p_hat, within 4 bootstrap standard errors.
Inputs are drawn on the device from a seeded generator: anchors ~ N(0, 3), proposal
rows = anchor + N(0, sigma), drafts sampled from their proposal row (Gumbel-max), with
sigma the sweep's calibrated noise (bisected on the oracle's expected acceptance).  The
kernel's acceptance rate p_hat must also match that calibrated acceptance within 4
standard errors of a binomial rate (plus the calibration tolerance): the rate at which
the kernel accepts sampled drafts is the law sum_k min(p_k, q~_k)."""
import numpy as np
import pytest
import torch

import oracle
from strided_verify_propose_amd import isd, synth

pytestmark = pytest.mark.gpu

V, B, STEPS = 151936, 64, 16
SIGMA = synth.SWEEP_SIGMA  # proposal noise sd giving mean acceptance 0.5 / 0.9
CALIBRATION_TOL = 0.002


def device_step(N, sigma, gen):
    R = 2 * N - 1
    anchor = torch.randn((B, R, V), generator=gen, device="cuda") * 3.0
    prop = anchor + torch.randn((B, R, V), generator=gen, device="cuda") * sigma
    logits = torch.cat([anchor[:, :N - 1], prop[:, N - 1:]], dim=1).to(torch.bfloat16).contiguous()
    draft = prop[:, :N - 1].to(torch.bfloat16).contiguous()
    del anchor, prop
    u01 = torch.rand(draft.shape, generator=gen, device="cuda", dtype=torch.float64)
    ids = torch.argmax(draft.double() - torch.log(-torch.log(u01)), dim=-1).to(torch.int32).contiguous()
    u = (torch.randint(0, 1 << 24, (B, R), generator=gen, device="cuda") / float(1 << 24)).to(torch.float32)
    return logits, draft, ids, u


@pytest.mark.parametrize("N", [2, 3, 4])
@pytest.mark.parametrize("p", [0.5, 0.9])
def test_tpf_from_kernel_matches_closed_form(N, p):
    index = synth.sweep_index(N, B, p)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1200 + index)
    n = []
    for _ in range(STEPS):
        logits, draft, ids, u = device_step(N, SIGMA[p], gen)
        out = isd.verify(logits, draft, ids, u, with_diagnostics=False)
        n.append(out["n_accept"].cpu().numpy())
    n = np.concatenate(n).astype(np.int64)
    tpf_hat, p_hat = oracle.renewal_estimate(n, N)
    diff = tpf_hat - oracle.tpf_closed_form(N, p_hat)
    rng = np.random.default_rng(index)
    boot = []
    for _ in range(400):
        s = n[rng.integers(0, len(n), len(n))]
        t, ph = oracle.renewal_estimate(s, N)
        boot.append(t - oracle.tpf_closed_form(N, ph))
    se = float(np.std(boot))
    print(f"  N={N} p~{p}: p_hat {p_hat:.4f} TPF_hat {tpf_hat:.4f} closed form "
          f"{oracle.tpf_closed_form(N, p_hat):.4f} diff {diff:+.4f} (se {se:.4f}, n={len(n)})", flush=True)
    evaluated = int(np.sum(np.minimum(n + 1, N - 1)))
    se_p = np.sqrt(p * (1 - p) / evaluated)
    print(f"  p_hat {p_hat:.4f} vs calibrated {p} (se {se_p:.4f}, {evaluated} draft tests)", flush=True)
    assert abs(p_hat - p) <= 4 * se_p + CALIBRATION_TOL, "kernel acceptance rate off the calibrated law"
    assert abs(diff) <= 4 * se + 1e-12
