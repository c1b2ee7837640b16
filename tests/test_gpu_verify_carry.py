"""Verification with the draft rows' statistics carried from the previous step
(isd_verify_carry): every output equals isd_verify's on the same inputs, bit for bit, and
the statistics a call hands on do not depend on whether it received any."""
import pytest
import torch

from strided_verify_propose_amd import isd, synth
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


CASES = [
    ("bf16_qwen3_8b", "bf16", 64, 4, 151936, 1001, 1.0),
    ("bf16_v300_unaligned", "bf16", 12, 3, 300, 31, 1.0),     # rows not 16-byte aligned: per-chunk grid
    ("f32_v5001_unaligned", "f32", 8, 3, 5001, 32, 1.0),
    ("bf16_n8", "bf16", 6, 8, 20000, 33, 1.0),
    ("bf16_n2", "bf16", 16, 2, 9000, 34, 1.0),
    ("bf16_temperature", "bf16", 8, 4, 9000, 35, 0.7),
    ("bf16_v2pow20", "bf16", 2, 4, 1 << 20, 36, 1.0),          # sub-chunk sums past the walk's registers
]


@pytest.mark.parametrize("name,dtype,B,N,V,seed,T", CASES, ids=[c[0] for c in CASES])
def test_carried_statistics_change_nothing(name, dtype, B, N, V, seed, T):
    c = synth.StepConfig(name, dtype, B=B, N=N, Hq=1, Hkv=1, D=64, V=V, ctx=("fixed", 0),
                         anchor_sd=3.0, noise_sd=0.3, seed=seed)
    v = synth.verify_inputs(c)
    print(f"verify_carry case {name} dtype={dtype} B={B} N={N} V={V} T={T}", flush=True)
    logits, draft = to_dev(v.logits), to_dev(v.draft_logits)
    ids, u = to_dev(v.draft_ids), to_dev(v.uniforms)
    # the previous step: its rows N .. 2N-2 are this step's draft rows
    prev_logits = logits.clone()
    prev_logits[:, N:] = draft
    nbytes = isd.verify_carry_bytes(B, N, V)
    assert nbytes > 0
    carried, handed_on, handed_on_plain = (torch.zeros(nbytes, dtype=torch.uint8, device=logits.device)
                                           for _ in range(3))
    isd.verify(prev_logits, draft, ids, u, T, q_stats_next=carried)
    ref = isd.verify(logits, draft, ids, u, T)
    got = isd.verify(logits, draft, ids, u, T, q_stats_prev=carried, q_stats_next=handed_on)
    isd.verify(logits, draft, ids, u, T, q_stats_next=handed_on_plain)
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(bits(got[k]), bits(ref[k])), k
    assert torch.equal(handed_on, handed_on_plain)
    print(f"  n_accept mean {ref['n_accept'].float().mean().item():.2f}", flush=True)


def test_statistics_handed_on_do_not_depend_on_the_draft_mode():
    """With argmax drafts there are no draft rows, but a call still hands its rows N..2N-2
    on; they equal what a sampled-draft call on the same logits hands on."""
    B, N, V = 8, 4, 12000
    c = synth.StepConfig("carry_modes", "bf16", B=B, N=N, Hq=1, Hkv=1, D=64, V=V, ctx=("fixed", 0),
                         anchor_sd=3.0, noise_sd=0.3, seed=41)
    v = synth.verify_inputs(c)
    print(f"verify_carry modes B={B} N={N} V={V}", flush=True)
    logits, draft = to_dev(v.logits), to_dev(v.draft_logits)
    ids, u = to_dev(v.draft_ids), to_dev(v.uniforms)
    nbytes = isd.verify_carry_bytes(B, N, V)
    sampled, argmax = (torch.zeros(nbytes, dtype=torch.uint8, device=logits.device) for _ in range(2))
    isd.verify(logits, draft, ids, u, q_stats_next=sampled)
    ref = isd.verify(logits, None, ids, u)
    got = isd.verify(logits, None, ids, u, q_stats_next=argmax)
    torch.cuda.synchronize()
    assert torch.equal(sampled, argmax)
    for k in ref:
        assert torch.equal(bits(got[k]), bits(ref[k])), k
