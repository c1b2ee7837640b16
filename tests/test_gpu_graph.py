"""A whole ISD step (projection, attention, verification) captured in a HIP graph and
replayed several times, with eager work and synchronisation between the replays: every
replay must reproduce the eager step bit for bit."""
import numpy as np
import pytest
import torch

from strided_verify_propose_amd import isd, synth
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager():
    scfg = synth.StepConfig("graph_step", "bf16", B=8, N=4, Hq=32, Hkv=8, D=128, V=151936,
                            ctx=("uniform", 100, 900), anchor_sd=3.0, noise_sd=0.3, seed=2024)
    pcfg = synth.ProjConfig("graph_proj", B=8, N=4, K=4096, Nout=4096, r=128, x_sd=1.0, w_sd=0.02,
                            seed=2025)
    att = synth.attention_inputs(scfg)
    ver = synth.verify_inputs(scfg)
    other = synth.verify_inputs(scfg, seed=2026)
    pin = synth.proj_inputs(pcfg)
    print(f"graph step B={scfg.B} ctx={att.ctx_lens.tolist()} proj M={pcfg.M}", flush=True)
    A = dict(q=to_dev(att.q), k_new=to_dev(att.k_new), v_new=to_dev(att.v_new),
             k_cache=to_dev(synth.k_tile_layout(att.k_pages)),
             v_cache=to_dev(synth.v_tile_layout(att.v_pages)),
             page_table=to_dev(att.page_table), ctx_lens=to_dev(att.ctx_lens))
    V = dict(logits=to_dev(ver.logits), draft_logits=to_dev(ver.draft_logits),
             draft_ids=to_dev(ver.draft_ids), uniforms=to_dev(ver.uniforms))
    O = dict(logits=to_dev(other.logits), draft_logits=to_dev(other.draft_logits),
             draft_ids=to_dev(other.draft_ids), uniforms=to_dev(other.uniforms))
    P = dict(x=to_dev(pin.x), w=to_dev(pin.w), a=to_dev(pin.a), b=to_dev(pin.b), gate=to_dev(pin.gate))
    maxctx = int(att.ctx_lens.max())
    y = torch.empty((pcfg.M, pcfg.Nout), dtype=torch.bfloat16, device="cuda")
    att_out = torch.empty_like(A["q"])
    vout = {}

    def step():
        isd.gated_lora_proj(P["x"], P["w"], P["a"], P["b"], P["gate"], out=y)
        isd.attention_step(A["q"], A["k_new"], A["v_new"], A["k_cache"], A["v_cache"],
                           A["page_table"], A["ctx_lens"], maxctx, out=att_out)
        vout.update(isd.verify(V["logits"], V["draft_logits"], V["draft_ids"], V["uniforms"],
                               out=vout or None))

    step()
    torch.cuda.synchronize()
    ref = dict(y=y.clone(), att=att_out.clone(), k=A["k_cache"].clone(), v=A["v_cache"].clone(),
               **{k: t.clone() for k, t in vout.items()})

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(4):
        # scribble over the outputs, run unrelated eager work, then replay
        y.fill_(0)
        att_out.fill_(0)
        for t in vout.values():
            t.fill_(0)
        junk = isd.verify(O["logits"], O["draft_logits"], O["draft_ids"], O["uniforms"])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"  replay {rep}: eager junk n_accept sum {int(junk['n_accept'].sum())}", flush=True)
        if not torch.equal(y, ref["y"]):
            d = (y != ref["y"]).cpu().numpy()
            raise AssertionError(f"projection differs on replay {rep}: {int(d.sum())} elements in rows "
                                 f"{np.flatnonzero(d.any(1)).tolist()[:16]}, columns "
                                 f"{np.flatnonzero(d.any(0)).tolist()[:16]}")
        assert torch.equal(att_out, ref["att"]), f"attention differs on replay {rep}"
        assert torch.equal(A["k_cache"], ref["k"]) and torch.equal(A["v_cache"], ref["v"]), "cache"
        for k, t in vout.items():
            assert torch.equal(t, ref[k]), f"verify output {k} differs on replay {rep}"
    assert np.isfinite(ref["att"].float().cpu().numpy()).all()
