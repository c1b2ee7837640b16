"""The closed decoding loop on the device: every step checked against the oracle, and
tokens per forward of a long loop against the closed form of the hot/cold chain."""
import numpy as np
import pytest
import torch

import oracle
from strided_verify_propose_amd import synth
from strided_verify_propose_amd.loop import ClosedLoop, LoopConfig
from tests.helpers import RTOL, assert_close, to_np, verify_parity

pytestmark = pytest.mark.gpu


def test_loop_steps_match_oracle():
    """Five steps of a small loop (hot and cold requests, contexts growing, block K/V
    appended over earlier steps' slots): attention, the cache after the append,
    verification and the commit of every step equal the oracle run on that step's inputs."""
    cfg = LoopConfig(B=6, N=4, Hq=8, Hkv=2, D=64, V=5000, ctx0=(20, 90), steps=8, proj=None,
                     sigma=0.2, seed=77)
    lp = ClosedLoop(cfg)
    for s in range(5):
        lp.model()
        torch.cuda.synchronize()
        x = {k: to_np(getattr(lp, k)) for k in ("q", "k_new", "v_new", "k_cache", "v_cache", "page_table",
                                                   "ctx_lens", "logits", "draft_rows", "draft_ids", "uniforms")}
        cold = int((x["draft_ids"][:, 0] < 0).sum())
        print(f"loop step {s}: ctx {x['ctx_lens'].tolist()}, {cold} cold", flush=True)
        lp.hot_path()
        torch.cuda.synchronize()
        kl = synth.k_logical_layout(x["k_cache"].reshape(x["k_cache"].shape[0], cfg.Hkv, -1), cfg.D)
        vl = synth.v_logical_layout(x["v_cache"].reshape(x["v_cache"].shape[0], cfg.Hkv, -1), cfg.D)
        ref_o, ref_k, ref_v = oracle.attention_step(x["q"], x["k_new"], x["v_new"], kl, vl, x["page_table"],
                                                    x["ctx_lens"])
        assert_close(to_np(lp.att_out), ref_o, RTOL["bf16"], f"attention step {s}")
        k_after = synth.k_logical_layout(to_np(lp.k_cache).reshape(x["k_cache"].shape[0], cfg.Hkv, -1), cfg.D)
        v_after = synth.v_logical_layout(to_np(lp.v_cache).reshape(x["v_cache"].shape[0], cfg.Hkv, -1), cfg.D)
        assert np.array_equal(k_after, ref_k) and np.array_equal(v_after, ref_v), f"cache after step {s}"
        ref = oracle.verify_step(x["logits"], x["draft_rows"], x["draft_ids"], x["uniforms"], cfg.N)
        verify_parity(lp.out, ref, cfg.N)
        # the commit from the kernel's own verification outputs (identical to the oracle's
        # except for near-threshold draws, which verify_parity excludes)
        g = {k: to_np(v) for k, v in lp.out.items()}
        ctx, nxt, toks, cnt = oracle.commit_step(g["n_accept"], g["next_token"], g["sampled_ids"],
                                                 x["draft_ids"], x["ctx_lens"], cfg.N)
        assert np.array_equal(to_np(lp.ctx_lens), ctx) and np.array_equal(to_np(lp.draft_ids), nxt)
        assert np.array_equal(to_np(lp.tokens), toks) and np.array_equal(to_np(lp.counts), cnt)
        lp.keep_draft_rows()


@pytest.mark.parametrize("N", [2, 4])
def test_loop_tokens_per_forward(N):
    """A 120-step loop of 64 requests captured as one HIP graph and replayed: tokens per
    forward measured from the kept tokens equal the closed form
    (2 + p + ... + p^(N-2)) / (2 - p^(N-1)) at the measured acceptance rate, within
    4 standard errors over requests plus the start-up (cold first step) bias."""
    steps = 120
    cfg = LoopConfig(B=64, N=N, Hq=8, Hkv=2, D=64, V=32768, ctx0=(64, 256), steps=steps, proj=None,
                     sigma=0.3, seed=88 + N)
    lp = ClosedLoop(cfg)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        lp.step()                       # warm-up step on the capture stream (counted)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    if hasattr(g, "register_generator_state"):
        g.register_generator_state(lp.gen)
    with torch.cuda.graph(g):
        lp.step()
    for _ in range(steps - 1):
        g.replay()
    torch.cuda.synchronize()
    st = lp.stats(steps)
    ctx0 = ClosedLoop(cfg).ctx_lens        # same seed: the initial context lengths
    grown = to_np(lp.ctx_lens).astype(np.int64) - to_np(ctx0).astype(np.int64)
    print(f"  N={N}: TPF {st['tpf_meas']:.4f} (se {st['tpf_se']:.4f}), p_hat {st['p_hat']:.4f}, "
          f"closed form {st['tpf_closed_form_at_p_hat']:.4f}", flush=True)
    assert np.array_equal(grown, to_np(lp.kept)), "contexts grew by the kept tokens"
    assert 0.7 < st["p_hat"] < 0.99
    assert abs(st["tpf_meas"] - st["tpf_closed_form_at_p_hat"]) < 4 * st["tpf_se"] + 1.0 / steps
