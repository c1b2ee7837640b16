"""GPU parity at the stride/concurrency sweep points: N in {2, 3, 4} (3, 5, 7 query rows)
x B in {1, 4, 16} requests, context 2048, Qwen3-8B heads and vocabulary, proposal noise
calibrated to mean acceptance 0.5 and 0.9 (「首次超越 AR 模型」 "為什麼 I-DLM 能在高並發下保持高效";
「I-DLM – introspektive Diffusion Language Models」 "Durchsatz (Throughput)").  Inputs are the
seeded host inputs of each point; attention and verification are compared with the
oracle on every request."""
import pytest

from strided_verify_propose_amd import synth
from tests import test_gpu_attention as t_att
from tests import test_gpu_verify as t_ver

pytestmark = pytest.mark.gpu

POINTS = [(N, B) for N in (2, 3, 4) for B in (1, 4, 16)]


@pytest.mark.parametrize("N,B", POINTS, ids=[f"n{N}_b{B}" for N, B in POINTS])
def test_sweep_attention(N, B):
    t_att.run(synth.sweep_point(N, B, 0.9))


@pytest.mark.parametrize("p", [0.5, 0.9])
@pytest.mark.parametrize("N,B", POINTS, ids=[f"n{N}_b{B}" for N, B in POINTS])
def test_sweep_verify(N, B, p):
    c = synth.sweep_point(N, B, p)
    out, ref, compared, excluded = t_ver.run(c)
    print(f"  sweep N={N} B={B} p~{p}: mean accepted drafts {ref['n_accept'].mean():.2f} of {N - 1}",
          flush=True)
