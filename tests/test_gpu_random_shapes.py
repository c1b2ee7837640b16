"""Seeded random shapes against the oracle: attention (both dtypes, every supported query
rows per KV head, contexts with page-boundary residues) and verification (sampled, argmax
and cold requests mixed, vocabularies off the 16-byte grid, carried statistics), so that
combinations no hand-picked case names are still checked element by element."""
import numpy as np
import pytest
import torch

import oracle
from strided_verify_propose_amd import isd, synth
from tests.helpers import RTOL, assert_close, to_dev, to_np, verify_parity

pytestmark = pytest.mark.gpu


def attention_cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        dtype = "f32" if len(cases) % 4 == 3 else "bf16"
        N = int(rng.integers(1, 9))
        R = 2 * N - 1
        Hkv = int(rng.choice([1, 2, 3, 4, 8]))
        G = int(rng.integers(1, 9))
        if dtype == "bf16" and R * G > 64:
            continue
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 25))
        # contexts: random, with page-boundary residues and empty contexts mixed in
        L = rng.integers(0, 1200, size=B)
        special = np.array([0, 1, 15, 16, 17, 255, 256, 257])
        pick = rng.random(B) < 0.3
        L[pick] = rng.choice(special, size=int(pick.sum()))
        cases.append((len(cases), dtype, B, N, Hkv * G, Hkv, D, [int(x) for x in L]))
    return cases


@pytest.mark.parametrize("case", attention_cases(64), ids=lambda c: f"a{c[0]}_{c[1]}_B{c[2]}_N{c[3]}_G{c[4] // c[5]}_D{c[6]}")
def test_attention_random_shape(case):
    i, dtype, B, N, Hq, Hkv, D, L = case
    cfg = synth.StepConfig(f"rand_attn_{i}", dtype, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=2, ctx=("fixed", 0),
                           anchor_sd=1, noise_sd=1, seed=3000 + i)
    inp = synth.attention_inputs(cfg, ctx_lens=L)
    print(f"random attention {i}: {dtype} B={B} N={N} Hq={Hq} Hkv={Hkv} D={D} ctx={L[:6]}", flush=True)
    d = dict(q=to_dev(inp.q), k_new=to_dev(inp.k_new), v_new=to_dev(inp.v_new),
             k_cache=to_dev(synth.k_tile_layout(inp.k_pages)), v_cache=to_dev(synth.v_tile_layout(inp.v_pages)),
             page_table=to_dev(inp.page_table), ctx_lens=to_dev(inp.ctx_lens))
    out = isd.attention_step(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["page_table"],
                             d["ctx_lens"], int(inp.ctx_lens.max()))
    torch.cuda.synchronize()
    kp, vp = oracle.attention.append_block(inp.k_pages, inp.v_pages, inp.k_new, inp.v_new, inp.page_table,
                                           inp.ctx_lens)
    assert np.array_equal(to_np(d["k_cache"]), synth.k_tile_layout(kp)), "K cache after append"
    assert np.array_equal(to_np(d["v_cache"]), synth.v_tile_layout(vp)), "V cache after append"
    ref, _, _ = oracle.attention_step(inp.q, inp.k_new, inp.v_new, inp.k_pages, inp.v_pages, inp.page_table,
                                      inp.ctx_lens, inp.scale)
    worst = assert_close(to_np(out), ref, RTOL[dtype], "attention output")
    print(f"  worst relative error {worst:.3e}", flush=True)


def verify_cases(n, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = "f32" if i % 4 == 3 else "bf16"
        N = int(rng.integers(1, 9))
        V = int(rng.choice([2, 7, 300, 1023, 4096, 5001, 16385, 40000, 70001]))
        B = int(rng.integers(1, 17))
        argmax = bool(rng.random() < 0.3)
        cold = rng.random(B) < 0.25
        T = float(rng.choice([1.0, 1.0, 0.7, 1.5]))
        sd = float(rng.choice([0.05, 0.3, 1.0]))
        cases.append((i, dtype, B, N, V, argmax, cold.tolist(), T, sd))
    return cases


@pytest.mark.parametrize("case", verify_cases(60), ids=lambda c: f"v{c[0]}_{c[1]}_B{c[2]}_N{c[3]}_V{c[4]}")
def test_verify_random_shape(case):
    i, dtype, B, N, V, argmax, cold, T, sd = case
    cfg = synth.StepConfig(f"rand_ver_{i}", dtype, B=B, N=N, Hq=1, Hkv=1, D=64, V=V, ctx=("fixed", 0),
                           anchor_sd=2.0, noise_sd=sd, seed=4000 + i, argmax_drafts=argmax)
    v = synth.verify_inputs(cfg)
    ids = v.draft_ids.copy()
    if N > 1:
        ids[np.asarray(cold)] = -1
    print(f"random verify {i}: {dtype} B={B} N={N} V={V} argmax={argmax} cold={int(np.sum(cold)) if N > 1 else 0} "
          f"T={T} noise={sd}", flush=True)
    ref = oracle.verify_step(v.logits, v.draft_logits, ids, v.uniforms, N, T)
    logits = to_dev(v.logits)
    draft = None if v.draft_logits is None else to_dev(v.draft_logits)
    out = isd.verify(logits, draft, to_dev(ids), to_dev(v.uniforms), T)
    torch.cuda.synchronize()
    compared, excluded = verify_parity(out, ref, N)
    rt = RTOL[dtype]
    assert_close(to_np(out["p_draft"]), ref["p_draft"], rt, "p_draft")
    assert_close(to_np(out["q_draft"]), ref["q_draft"], rt, "q_draft")
    rows = 2 * N - 1 + (N - 1 if draft is not None else 0)
    assert_close(to_np(out["row_lse"])[:, :rows], ref["row_lse"][:, :rows], rt, "row_lse")
    if draft is not None:
        # the same step with its draft rows' statistics carried from a previous step
        prev = logits.clone()
        prev[:, N:] = draft
        nb = isd.verify_carry_bytes(B, N, V)
        carried = torch.zeros(nb, dtype=torch.uint8, device=logits.device)
        isd.verify(prev, draft, to_dev(ids), to_dev(v.uniforms), T, q_stats_next=carried)
        got = isd.verify(logits, draft, to_dev(ids), to_dev(v.uniforms), T, q_stats_prev=carried)
        torch.cuda.synchronize()
        for k in out:
            a, b = got[k], out[k]
            if a.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), f"carried statistics change {k}"
    print(f"  compared {compared}, excluded {excluded}", flush=True)


def proj_cases(n, seed=20261205):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(rng.choice([1, 7, 63, 64, 65, 130, 448, 700]))
        K = int(64 * rng.integers(1, 33))            # 64 .. 2048
        Nout = int(128 * rng.integers(1, 9))         # 128 .. 1024
        r = int(rng.choice([128, 256]))
        pattern = tuple(int(x) for x in (rng.random(int(rng.integers(1, 9))) < 0.5))
        cases.append((i, M, K, Nout, r, pattern))
    return cases


@pytest.mark.parametrize("case", proj_cases(32), ids=lambda c: f"p{c[0]}_M{c[1]}_K{c[2]}_N{c[3]}_r{c[4]}")
def test_projection_random_shape(case):
    """Gated projection against the oracle; ungated rows equal the base-only call; packed
    weights (from either orientation) give the row-major result bit for bit."""
    i, M, K, Nout, r, pattern = case
    cfg = synth.ProjConfig(f"rand_proj_{i}", B=1, N=1, K=K, Nout=Nout, r=r, x_sd=1.0, w_sd=0.02,
                           seed=5000 + i, gate_pattern=pattern)
    p = synth.proj_inputs(cfg, M=M)
    print(f"random projection {i}: M={M} K={K} Nout={Nout} r={r} gate pattern {pattern}", flush=True)
    x, w, a, b, gate = (to_dev(t) for t in (p.x, p.w, p.a, p.b, p.gate))
    y = isd.gated_lora_proj(x, w, a, b, gate)
    yb = isd.gated_lora_proj(x, w)
    yp = isd.gated_lora_proj_packed(x, isd.pack_proj_weights(w, a, b), gate)
    ykn = isd.gated_lora_proj_packed(
        x, isd.pack_proj_weights_kn(w.t().contiguous(), a.t().contiguous(), b.t().contiguous()), gate)
    torch.cuda.synchronize()
    assert torch.equal(yp, y) and torch.equal(ykn, y), "packed results differ from row-major"
    g = p.gate.astype(bool)
    Y = to_np(y)
    assert np.array_equal(Y[~g], to_np(yb)[~g]), "ungated rows differ from the base-only call"
    worst = assert_close(Y, oracle.gated_lora_proj(p.x, p.w, p.a, p.b, p.gate), RTOL["bf16"], "gated projection")
    print(f"  worst relative error {worst:.3e}", flush=True)
