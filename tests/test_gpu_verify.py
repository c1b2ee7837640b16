"""GPU parity of isd_verify against the oracle, plus the exact laws through the kernel."""
import numpy as np
import pytest
import torch
from scipy.special import softmax
from scipy.stats import chisquare

import oracle
from strided_verify_propose_amd import isd, synth
from tests.helpers import RTOL, assert_close, to_dev, to_np, verify_parity

pytestmark = pytest.mark.gpu


def cfg(name, dtype, B, N, V, seed, anchor_sd=3.0, noise_sd=0.3, argmax=False):
    return synth.StepConfig(name, dtype, B=B, N=N, Hq=1, Hkv=1, D=64, V=V, ctx=("fixed", 0),
                            anchor_sd=anchor_sd, noise_sd=noise_sd, seed=seed, argmax_drafts=argmax)


def run(c, temperature=1.0):
    v = synth.verify_inputs(c)
    print(f"verify case {c.name} dtype={c.dtype} B={c.B} N={c.N} V={c.V} argmax={c.argmax_drafts}", flush=True)
    ref = oracle.verify_step(v.logits, v.draft_logits, v.draft_ids, v.uniforms, c.N, temperature)
    out = isd.verify(to_dev(v.logits), None if v.draft_logits is None else to_dev(v.draft_logits),
                     to_dev(v.draft_ids), to_dev(v.uniforms), temperature)
    torch.cuda.synchronize()
    compared, excluded = verify_parity(out, ref, c.N)
    rt = RTOL[c.dtype]
    assert_close(to_np(out["p_draft"]), ref["p_draft"], rt, "p_draft")
    assert_close(to_np(out["q_draft"]), ref["q_draft"], rt, "q_draft")
    R = c.R
    nrows = R + (c.N - 1 if v.draft_logits is not None else 0)
    assert_close(to_np(out["row_lse"])[:, :nrows], ref["row_lse"][:, :nrows], rt, "row_lse")
    if v.draft_logits is None:
        assert np.all(to_np(out["row_lse"])[:, R:] == 0)
    print(f"  compared {compared} decisions/ids, excluded {excluded} near-threshold draws", flush=True)
    return out, ref, compared, excluded


CASES = [
    cfg("tiny_fp32", "f32", 1, 2, 1024, 1000, anchor_sd=2.0, noise_sd=0.5),
    cfg("tiny_fp32_argmax", "f32", 3, 2, 1024, 1010, anchor_sd=2.0, noise_sd=0.5, argmax=True),
    cfg("bf16_v5000", "bf16", 16, 4, 5000, 11),
    cfg("bf16_v300_unaligned", "bf16", 12, 3, 300, 12, anchor_sd=1.0, noise_sd=0.5),
    cfg("f32_v301_unaligned", "f32", 12, 3, 301, 13, anchor_sd=1.0, noise_sd=0.5),
    cfg("bf16_v8", "bf16", 64, 2, 8, 14, anchor_sd=1.0, noise_sd=1.0),
    cfg("bf16_v40000_chunks", "bf16", 10, 4, 40000, 15),
    cfg("bf16_n1", "bf16", 9, 1, 3000, 16),
    cfg("bf16_n8", "bf16", 6, 8, 20000, 17, noise_sd=0.1),
    cfg("bf16_argmax", "bf16", 16, 4, 33000, 18, argmax=True, noise_sd=0.05),
    cfg("f32_big_noise", "f32", 16, 4, 17000, 19, noise_sd=2.0),
    # the largest vocabulary: 64 chunks, 1024 sub-chunk sums per row (past the walk's
    # registers and its LDS stash, so those paths read them from memory)
    cfg("bf16_v2pow20", "bf16", 2, 4, 1 << 20, 22),
    cfg("bf16_v2pow20_argmax", "bf16", 2, 4, 1 << 20, 23, argmax=True, noise_sd=0.05),
]


@pytest.mark.parametrize("c", CASES, ids=[c.name for c in CASES])
def test_verify_parity(c):
    run(c)


def test_verify_max_requests():
    """65535 requests, the most one call takes (the grids' request dimension at its limit):
    N = 2, V = 300.  Requests are independent, so the oracle runs on a sample of them --
    both ends of the batch and 240 seeded picks -- and the sampled rows of the outputs
    must match it."""
    c = cfg("bf16_b65535", "bf16", 65535, 2, 300, 24, anchor_sd=1.0, noise_sd=0.5)
    v = synth.verify_inputs(c)
    print(f"verify case {c.name} B={c.B} N={c.N} V={c.V}", flush=True)
    out = isd.verify(to_dev(v.logits), to_dev(v.draft_logits), to_dev(v.draft_ids), to_dev(v.uniforms))
    torch.cuda.synchronize()
    bs = np.unique(np.concatenate([np.arange(8), np.arange(c.B - 8, c.B),
                                   np.random.default_rng(24).integers(0, c.B, 240)]))
    ref = oracle.verify_step(v.logits[bs], v.draft_logits[bs], v.draft_ids[bs], v.uniforms[bs], c.N, 1.0)
    idx = torch.as_tensor(bs, device=out["n_accept"].device)
    sub = {k: t[idx] for k, t in out.items()}
    compared, excluded = verify_parity(sub, ref, c.N)
    rt = RTOL[c.dtype]
    assert_close(to_np(sub["p_draft"]), ref["p_draft"], rt, "p_draft")
    assert_close(to_np(sub["q_draft"]), ref["q_draft"], rt, "q_draft")
    assert_close(to_np(sub["row_lse"]), ref["row_lse"], rt, "row_lse")
    print(f"  {len(bs)} requests: compared {compared} decisions/ids, excluded {excluded}", flush=True)
    assert compared >= len(bs)


def test_verify_temperature():
    run(cfg("bf16_temp", "bf16", 8, 4, 9000, 21), temperature=0.7)


def test_verify_qwen3_8b_full_size():
    """B=64, N=4, vocab 151936, anchor N(0,3), proposal = anchor + N(0,0.3)."""
    out, ref, compared, excluded = run(synth.QWEN3_8B)
    assert compared > 64 * 4
    acc = ref["n_accept"].mean()
    print(f"  mean accepted drafts {acc:.2f} of 3", flush=True)


def test_verify_q_equals_p_accepts_all():
    c = cfg("qp", "bf16", 32, 4, 20000, 31)
    v = synth.verify_inputs(c)
    logits = v.logits.copy()
    logits[:, :3] = v.draft_logits
    out = isd.verify(to_dev(logits), to_dev(v.draft_logits), to_dev(v.draft_ids), to_dev(v.uniforms))
    assert np.all(to_np(out["n_accept"]) == 3)
    assert np.all(to_np(out["accept"]) == 1)


def test_verify_deterministic():
    c = cfg("det", "bf16", 16, 4, 151936, 41)
    v = synth.verify_inputs(c)
    args = (to_dev(v.logits), to_dev(v.draft_logits), to_dev(v.draft_ids), to_dev(v.uniforms))
    a = isd.verify(*args)
    b = isd.verify(*args)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("argmax", [False, True])
def test_emitted_token_law_through_kernel(argmax):
    """Chi-square on an 8-token vocab: the first emitted token follows p."""
    rng = np.random.default_rng(7 + argmax)
    V, n = 8, 60000
    lp = (rng.standard_normal(V) * 1.2).astype(np.float32)
    lq = (lp + rng.standard_normal(V) * 0.9).astype(np.float32)
    logits = np.tile(rng.standard_normal((1, 3, V)).astype(np.float32), (n, 1, 1))
    logits[:, 0] = lp
    if argmax:
        d = np.full((n, 1), 5, np.int32)
        dl = None
    else:
        d = rng.choice(V, size=(n, 1), p=softmax(lq.astype(np.float64))).astype(np.int32)
        dl = to_dev(np.tile(lq, (n, 1, 1)))
    u = (rng.integers(0, 1 << 24, size=(n, 3)) / float(1 << 24)).astype(np.float32)
    out = isd.verify(to_dev(logits), dl, to_dev(d), to_dev(u))
    acc = to_np(out["accept"])[:, 0]
    first = np.where(acc == 1, d[:, 0], to_np(out["next_token"]))
    p = softmax(lp.astype(np.float64))
    stat = chisquare(np.bincount(first, minlength=V), p * n)
    print(f"  chi-square {stat.statistic:.2f} (7 dof), p-value {stat.pvalue:.3g}", flush=True)
    assert stat.statistic < 24.32       # 7 dof, alpha = 1e-3


@pytest.mark.parametrize("argmax", [False, True])
def test_verify_cold_requests(argmax):
    """Every third request is cold (draft_ids[b][0] = -1): no walk, the next token drawn
    from row 0 at u_0; the others are ordinary.  Parity with the oracle on the whole batch."""
    c = cfg("cold_argmax" if argmax else "cold", "bf16", 24, 4, 151936, 51, argmax=argmax)
    v = synth.verify_inputs(c)
    d = v.draft_ids.copy()
    d[::3] = -1
    print(f"verify cold mix argmax={argmax}: {int((d[:, 0] < 0).sum())} cold of {c.B}", flush=True)
    ref = oracle.verify_step(v.logits, v.draft_logits, d, v.uniforms, c.N)
    out = isd.verify(to_dev(v.logits), None if v.draft_logits is None else to_dev(v.draft_logits),
                     to_dev(d), to_dev(v.uniforms))
    torch.cuda.synchronize()
    compared, excluded = verify_parity(out, ref, c.N)
    assert np.all(to_np(out["n_accept"])[::3] == 0) and np.all(to_np(out["accept"])[::3] == 0)
    assert np.all(to_np(out["p_draft"])[::3] == 0)
    print(f"  compared {compared}, excluded {excluded}", flush=True)


def test_commit_matches_oracle():
    """isd_commit against the oracle's commit on a random mix of hot (all accepted or
    not) and cold requests, N in {1, 2, 4, 8}."""
    rng = np.random.default_rng(61)
    for N in (1, 2, 4, 8):
        B = 300
        n_acc = rng.integers(0, N, size=B).astype(np.int32)
        nxt = rng.integers(0, 1000, size=B).astype(np.int32)
        smp = rng.integers(0, 1000, size=(B, N)).astype(np.int32)
        drafts = rng.integers(0, 1000, size=(B, N - 1)).astype(np.int32)
        if N > 1:
            drafts[rng.random(B) < 0.3] = -1
        ctx = rng.integers(0, 5000, size=B).astype(np.int32)
        ctx_r, nxt_d, toks_r, cnt_r = oracle.commit_step(n_acc, nxt, smp, drafts, ctx, N)
        D = to_dev(drafts)
        C = to_dev(ctx)
        toks = torch.empty((B, N), dtype=torch.int32, device="cuda")
        cnt = torch.empty(B, dtype=torch.int32, device="cuda")
        isd.commit(to_dev(n_acc), to_dev(nxt), to_dev(smp), D, C, toks, cnt)
        torch.cuda.synchronize()
        assert np.array_equal(to_np(C), ctx_r), N
        assert np.array_equal(to_np(D), nxt_d), N
        assert np.array_equal(to_np(toks), toks_r), N
        assert np.array_equal(to_np(cnt), cnt_r), N
