"""GPU parity of the LM head (isd_lm_head) and of the LM head fused with verification
(isd_lm_head_verify) against the oracle.

Parity inputs use the exact grid (hidden = k/4, weights = k/32): every float32 summation
order then gives the exact product, so the stored bf16 logits must match the oracle's bit
for bit.  Gaussian inputs are checked to one bf16 step."""
import numpy as np
import pytest
import torch

import oracle
import oracle.lm_head as olm
from strided_verify_propose_amd import isd, synth
from tests.helpers import RTOL, assert_close, as_f64, to_dev, to_np, verify_parity

pytestmark = pytest.mark.gpu


def lcfg(name, B, N, Dm, V, seed, grid=True, draft_sd=2.0):
    return synth.LmHeadConfig(name, B=B, N=N, Dm=Dm, V=V, h_sd=1.0, w_sd=3.0 / np.sqrt(Dm),
                              draft_sd=draft_sd, grid=grid, seed=seed)


def oracle_logits(hidden, w_lm, rows=None, step=16384):
    """Oracle logits of the given rows, computed a vocabulary slice at a time (each logit
    depends on its own row and column only)."""
    h = hidden if rows is None else hidden[rows]
    return np.concatenate([olm.lm_head_logits(h, w_lm[v0:v0 + step])
                           for v0 in range(0, w_lm.shape[0], step)], axis=1)


LOGIT_CASES = [
    lcfg("m7_dm32_v8", 1, 4, 32, 8, 40),             # one k step, one column block
    lcfg("m14_dm256_v5000", 2, 4, 256, 5000, 41),    # ragged vocabulary tile
    lcfg("m448_dm4096_v2048", 64, 4, 4096, 2048, 42),
    lcfg("m700_dm96_v1032", 100, 4, 96, 1032, 43),   # two row tiles, the second ragged; 3 k steps
    lcfg("m9_dm160_v4104", 3, 2, 160, 4104, 44),
    lcfg("m1_dm64_v1000", 1, 1, 64, 1000, 46),      # a single row; two k steps, fewer than the ring
]


@pytest.mark.parametrize("c", LOGIT_CASES, ids=[c.name for c in LOGIT_CASES])
def test_lm_head_logits_bitwise_on_grid(c):
    x = synth.lm_head_inputs(c)
    print(f"lm_head case {c.name}: M={c.M} Dm={c.Dm} V={c.V}", flush=True)
    out = isd.lm_head(to_dev(x.hidden), to_dev(x.w_lm))
    torch.cuda.synchronize()
    got = as_f64(to_np(out))
    ref = oracle_logits(x.hidden, x.w_lm)
    assert np.array_equal(got, ref), f"{int(np.sum(got != ref))} of {ref.size} logits differ"


def test_lm_head_gaussian_within_one_bf16_step():
    c = lcfg("gauss", 8, 4, 1024, 6000, 45, grid=False)
    x = synth.lm_head_inputs(c)
    out = as_f64(to_np(isd.lm_head(to_dev(x.hidden), to_dev(x.w_lm))))
    H = synth.bf16_bits_to_f32(x.hidden).astype(np.float64)
    W = synth.bf16_bits_to_f32(x.w_lm).astype(np.float64)
    exact = H @ W.T
    ref = oracle_logits(x.hidden, x.w_lm)
    # one bf16 step of the exact value, plus the float32 dot-product bound K 2^-24 sum|h w|
    # (which matters only where the sum cancels to far below its terms)
    step = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
    accum = c.Dm * 2.0 ** -24 * (np.abs(H) @ np.abs(W).T)
    assert np.all(np.abs(out - exact) <= step + accum)
    frac_equal = float(np.mean(out == ref))
    print(f"  {frac_equal:.5f} of logits equal the oracle's bf16 rounding", flush=True)
    assert frac_equal > 0.99


def run_fused(c, argmax=False, cold=(), temperature=1.0):
    x = synth.lm_head_inputs(c, argmax_drafts=argmax)
    ids = x.draft_ids.copy()
    for b in cold:
        ids[b, :] = -1
    print(f"lm_head_verify case {c.name}: B={c.B} N={c.N} Dm={c.Dm} V={c.V} argmax={argmax} "
          f"cold={list(cold)}", flush=True)
    logits_ref, ref = olm.lm_head_verify(x.hidden, x.w_lm, x.draft_logits, ids, x.uniforms, c.N,
                                         temperature)
    out = isd.lm_head_verify(to_dev(x.hidden), to_dev(x.w_lm),
                             None if x.draft_logits is None else to_dev(x.draft_logits),
                             to_dev(ids), to_dev(x.uniforms), temperature)
    torch.cuda.synchronize()
    got = as_f64(to_np(out["logits"]))
    assert np.array_equal(got, logits_ref), "stored logits differ from the oracle's"
    compared, excluded = verify_parity(out, ref, c.N)
    rt = RTOL["bf16"]
    assert_close(to_np(out["p_draft"]), ref["p_draft"], rt, "p_draft")
    assert_close(to_np(out["q_draft"]), ref["q_draft"], rt, "q_draft")
    nrows = c.R + (c.N - 1 if x.draft_logits is not None else 0)
    assert_close(to_np(out["row_lse"])[:, :nrows], ref["row_lse"][:, :nrows], 1e-5, "row_lse")
    print(f"  compared {compared} decisions/ids, excluded {excluded}", flush=True)
    return x, out, ref


FUSED_CASES = [
    (lcfg("b2_n4_v5000", 2, 4, 256, 5000, 51), False, ()),
    (lcfg("b6_n2_v20000", 6, 2, 64, 20000, 52), False, ()),        # two chunks, ragged
    (lcfg("b5_n4_v9000_argmax", 5, 4, 128, 9000, 53), True, ()),
    (lcfg("b4_n3_v3000_cold", 4, 3, 96, 3000, 54), False, (0, 2)),
    (lcfg("b9_n1_v4000", 9, 1, 64, 4000, 55), False, ()),
    (lcfg("b3_n8_v33000", 3, 8, 64, 33000, 56), False, ()),
    (lcfg("b70_n4_v2048", 70, 4, 64, 2048, 57), False, ()),        # 490 rows: two row tiles
    (lcfg("b2_n4_v2pow20", 2, 4, 32, 1 << 20, 64), False, ()),     # the largest vocabulary
]


@pytest.mark.parametrize("c,argmax,cold", FUSED_CASES, ids=[c[0].name for c in FUSED_CASES])
def test_lm_head_verify_parity(c, argmax, cold):
    run_fused(c, argmax, cold)


def test_lm_head_verify_temperature():
    run_fused(lcfg("temp", 4, 4, 128, 7000, 58), temperature=0.6)


def test_lm_head_verify_agrees_with_unfused_verify():
    """Same logits through isd_lm_head + isd_verify: argmax ids identical, every other id
    identical here (they could differ only within float rounding of a boundary)."""
    c = lcfg("fused_vs_unfused", 16, 4, 512, 40000, 59, grid=False, draft_sd=3.0)
    x = synth.lm_head_inputs(c)
    h, w, d = to_dev(x.hidden), to_dev(x.w_lm), to_dev(x.draft_logits)
    ids, u = to_dev(x.draft_ids), to_dev(x.uniforms)
    fused = isd.lm_head_verify(h, w, d, ids, u)
    logits = isd.lm_head(h, w).view(c.B, c.R, c.V)
    plain = isd.verify(logits, d, ids, u)
    torch.cuda.synchronize()
    assert torch.equal(fused["logits"], logits)
    for k in ("n_accept", "accept", "next_token", "argmax_ids", "sampled_ids"):
        assert torch.equal(fused[k], plain[k]), k
    for k in ("p_draft", "q_draft", "row_lse"):
        assert_close(to_np(fused[k]), to_np(plain[k]).astype(np.float64), 1e-5, k)


def test_lm_head_verify_qwen3_8b_shape_sampled():
    """B=64, N=4, Dm=4096, V=151936 on the exact grid: the logits of sampled rows bit for
    bit, and two whole requests through the oracle's verification."""
    c = lcfg("qwen3_8b_grid", 64, 4, 4096, 151936, 60)
    x = synth.lm_head_inputs(c)
    out = isd.lm_head_verify(to_dev(x.hidden), to_dev(x.w_lm), to_dev(x.draft_logits),
                             to_dev(x.draft_ids), to_dev(x.uniforms))
    torch.cuda.synchronize()
    logits = to_np(out["logits"]).reshape(c.M, c.V)
    reqs = [5, 63]
    rows = [b * c.R + r for b in reqs for r in range(c.R)] + [0, 200, 447]
    ref_rows = oracle_logits(x.hidden, x.w_lm, rows)
    assert np.array_equal(as_f64(logits[rows]), ref_rows)
    k = len(reqs) * c.R
    ref = oracle.verify_step(ref_rows[:k].reshape(len(reqs), c.R, c.V), x.draft_logits[reqs],
                             x.draft_ids[reqs], x.uniforms[reqs], c.N)
    sub = {key: v[reqs] for key, v in out.items() if key != "logits"}
    compared, excluded = verify_parity(sub, ref, c.N)
    assert_close(to_np(out["row_lse"])[reqs], ref["row_lse"], 1e-5, "row_lse")
    print(f"  compared {compared}, excluded {excluded}", flush=True)


def test_lm_head_verify_deterministic():
    c = lcfg("det", 8, 4, 256, 12000, 61, grid=False)
    x = synth.lm_head_inputs(c)
    args = (to_dev(x.hidden), to_dev(x.w_lm), to_dev(x.draft_logits), to_dev(x.draft_ids),
            to_dev(x.uniforms))
    a = isd.lm_head_verify(*args)
    a = {k: v.clone() for k, v in a.items()}
    b = isd.lm_head_verify(*args)
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_lm_head_qwen3_32b_hidden_sampled_rows():
    """Hidden size 5120 (Qwen3-32B) on the exact grid: sampled rows bit for bit."""
    c = lcfg("qwen3_32b_grid", 64, 4, 5120, 151936, 62)
    x = synth.lm_head_inputs(c)
    out = to_np(isd.lm_head(to_dev(x.hidden), to_dev(x.w_lm)))
    rows = [0, 1, 223, 224, 300, 447]
    assert np.array_equal(as_f64(out[rows]), oracle_logits(x.hidden, x.w_lm, rows))


def test_lm_head_verify_back_to_back_calls_are_identical():
    c = lcfg("b2b", 16, 4, 1024, 40000, 63, grid=False)
    x = synth.lm_head_inputs(c)
    args = (to_dev(x.hidden), to_dev(x.w_lm), to_dev(x.draft_logits), to_dev(x.draft_ids),
            to_dev(x.uniforms))
    outs = [isd.lm_head_verify(*args) for _ in range(12)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for k in o:
            assert torch.equal(o[k], outs[0][k]), k
