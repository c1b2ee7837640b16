"""R-ISD through a whole decoder layer (「首次超越 AR 模型」 "無損 R-ISD"; 「I-DLM –
introspektive Diffusion Language Models」 "Lossless R-ISD"):
  * the layer built from the library's calls matches oracle.decoder_layer -- output and
    the K/V the block appends -- on seeded inputs, gated and base-only, at a small shape
    and at Qwen3-8B's shape (sampled requests);
  * the clean rows' outputs and their K/V equal the base-only layer's bit for bit, and
    the gated rows differ."""
import numpy as np
import pytest
import torch

import oracle
from strided_verify_propose_amd import synth
from strided_verify_propose_amd.layer import LayerConfig, RIsdLayer
from tests.helpers import RTOL, assert_close, to_np

pytestmark = pytest.mark.gpu


def build(icfg):
    inp = synth.layer_inputs(icfg)
    cfg = LayerConfig(B=icfg.B, N=icfg.N, hidden=icfg.hidden, Hq=icfg.Hq, Hkv=icfg.Hkv, D=icfg.D,
                      inter=icfg.inter, r=icfg.r)
    return inp, RIsdLayer(cfg, inputs=inp)


def compare_with_oracle(inp, lay, gated, requests):
    c, at = inp.cfg, inp.attn
    k0, v0 = lay.k_cache.clone(), lay.v_cache.clone()
    out = to_np(lay.forward(gated=gated))
    kc = synth.k_logical_layout(to_np(lay.k_cache), c.D)
    vc = synth.v_logical_layout(to_np(lay.v_cache), c.D)
    lay.k_cache.copy_(k0)
    lay.v_cache.copy_(v0)
    R = c.R
    rows = np.concatenate([np.arange(b * R, (b + 1) * R) for b in requests])
    ref, kp, vp = oracle.decoder_layer(inp.x[rows], inp.weights, at.k_pages, at.v_pages,
                                       at.page_table[requests], at.ctx_lens[requests], c.Hq, c.Hkv, c.D,
                                       gate=inp.gate[rows] if gated else None)
    assert_close(out[rows], ref, RTOL["bf16"], f"layer output (gated={gated})")
    # the appended K/V of the compared requests, slot by slot; the rest of the cache unchanged
    touched = np.zeros(at.k_pages.shape[:1] + at.k_pages.shape[2:3], bool)   # [pages, 16]
    for b in requests:
        for t in range(R):
            j = int(at.ctx_lens[b]) + t
            p, s = at.page_table[b, j // 16], j % 16
            touched[p, s] = True
            assert_close(kc[p, :, s], oracle.stored.to_f64(kp[p, :, s]), RTOL["bf16"], f"K slot {b},{t}")
            assert_close(vc[p, :, s], oracle.stored.to_f64(vp[p, :, s]), RTOL["bf16"], f"V slot {b},{t}")
    for b in range(c.B):            # slots of requests not compared hold their block rows too
        for t in range(R):
            j = int(at.ctx_lens[b]) + t
            touched[at.page_table[b, j // 16], j % 16] = True
    keep = ~touched
    assert np.array_equal(kc.transpose(0, 2, 1, 3)[keep], at.k_pages.transpose(0, 2, 1, 3)[keep])
    assert np.array_equal(vc.transpose(0, 2, 1, 3)[keep], at.v_pages.transpose(0, 2, 1, 3)[keep])


@pytest.mark.parametrize("gated", [True, False])
def test_small_layer_matches_oracle(gated):
    icfg = synth.LayerInputsConfig("layer_small", B=3, N=4, hidden=256, Hq=4, Hkv=2, D=64, inter=512,
                                   r=128, ctx=("uniform", 0, 300), seed=1610)
    inp, lay = build(icfg)
    print(f"layer small gated={gated} ctx={inp.attn.ctx_lens.tolist()}", flush=True)
    compare_with_oracle(inp, lay, gated, list(range(icfg.B)))


def test_qwen3_8b_layer_matches_oracle_on_sampled_requests():
    icfg = synth.LayerInputsConfig("layer_qwen3_8b", B=4, N=4, hidden=4096, Hq=32, Hkv=8, D=128,
                                   inter=12288, r=128, ctx=("uniform", 512, 4096), seed=1620)
    inp, lay = build(icfg)
    print(f"layer qwen3-8b ctx={inp.attn.ctx_lens.tolist()}", flush=True)
    compare_with_oracle(inp, lay, True, [0, 3])


def test_clean_rows_bit_identical_through_the_layer():
    cfg = LayerConfig(B=8, N=4, ctx0=(100, 700))
    lay = RIsdLayer(cfg)
    print(f"layer B={cfg.B} N={cfg.N} ctx={lay.ctx_lens.tolist()}", flush=True)
    k0, v0 = lay.k_cache.clone(), lay.v_cache.clone()
    base = lay.forward(gated=False)
    kb, vb = lay.k_cache.clone(), lay.v_cache.clone()
    lay.k_cache.copy_(k0)
    lay.v_cache.copy_(v0)
    gated = lay.forward(gated=True)
    torch.cuda.synchronize()
    R, N = lay.R, cfg.N
    rows = torch.arange(lay.M, device=base.device) % R
    clean = rows < N - 1
    assert torch.equal(gated[clean], base[clean]), "clean rows differ from the base-only layer"
    assert not torch.equal(gated[~clean], base[~clean]), "gated rows should carry the delta"
    assert torch.isfinite(gated.float()).all()
    # the cache: the clean rows' K/V slots hold the base-only values
    for b in range(cfg.B):
        L = int(lay.ctx_lens[b])
        for j in range(N - 1):
            pos = L + j
            page = int(lay.page_table[b, pos // 16])
            s = pos % 16
            assert torch.equal(lay.k_cache[page, :, :, s, :], kb[page, :, :, s, :]), (b, j)
            assert torch.equal(lay.v_cache[page, :, :, s // 4, :, s % 4], vb[page, :, :, s // 4, :, s % 4]), (b, j)
