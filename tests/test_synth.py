"""The seeded input module: dtype rounding, page tables, tile layouts, draws."""
import numpy as np
import pytest
import torch

from strided_verify_propose_amd import synth


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, -3.5, 1e-30, 3e38], np.float32)])
    # ties: values exactly halfway between two bf16 numbers
    base = synth.bf16_bits_to_f32(rng.integers(0x3F00, 0x4100, 1000).astype(np.uint16))
    halfway = (base.view(np.uint32) + 0x8000).view(np.float32)
    x = np.concatenate([x, halfway])
    ours = synth.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_tile_layouts_roundtrip_and_formula():
    rng = np.random.default_rng(1)
    P, H, D = 3, 2, 128
    k = rng.standard_normal((P, H, 16, D)).astype(np.float32)
    kt = synth.k_tile_layout(k)
    vt = synth.v_tile_layout(k)
    assert np.array_equal(synth.k_logical_layout(kt, D), k)
    assert np.array_equal(synth.v_logical_layout(vt, D), k)
    flat_k, flat_v = kt.ravel(), vt.ravel()
    for (p, h, t, d) in [(0, 0, 0, 0), (2, 1, 15, 127), (1, 0, 7, 9), (1, 1, 4, 77)]:
        base = (p * H + h) * 16 * D
        assert flat_k[base + (d // 8) * 128 + t * 8 + d % 8] == k[p, h, t, d]
        assert flat_v[base + (d // 16) * 256 + (t // 4) * 64 + (d % 16) * 4 + t % 4] == k[p, h, t, d]


def test_attention_inputs_pages_cover_context_and_block():
    cfg = synth.StepConfig("t", "bf16", B=5, N=3, Hq=4, Hkv=2, D=64, V=64,
                           ctx=("uniform", 0, 70), anchor_sd=1, noise_sd=1, seed=7)
    inp = synth.attention_inputs(cfg)
    R = cfg.R
    used = []
    for b in range(cfg.B):
        n = (int(inp.ctx_lens[b]) + R + 15) // 16
        used.extend(inp.page_table[b, :n].tolist())
    assert sorted(used) == list(range(inp.num_pages))          # a permutation, no sharing
    # slots at and past ctx_len start at zero
    for b in range(cfg.B):
        L = int(inp.ctx_lens[b])
        for j in range(L, L + R):
            assert not inp.k_pages[inp.page_table[b, j // 16], :, j % 16].any()


def test_seeded_inputs_are_reproducible():
    a = synth.verify_inputs(synth.TINY)
    b = synth.verify_inputs(synth.TINY)
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.draft_ids, b.draft_ids)
    assert np.array_equal(a.uniforms, b.uniforms)
    k = a.uniforms.astype(np.float64) * (1 << 24)
    assert np.array_equal(k, np.round(k)) and a.uniforms.max() < 1.0


def test_gumbel_draws_follow_softmax():
    from scipy.special import softmax
    from scipy.stats import chisquare
    rng = np.random.default_rng(3)
    row = rng.standard_normal(6).astype(np.float32) * 1.5
    g = np.random.default_rng(4)
    draws = synth.gumbel_argmax(np.broadcast_to(row, (200000, 6)), g)
    counts = np.bincount(draws, minlength=6)
    p = softmax(row.astype(np.float64))
    assert chisquare(counts, p * counts.sum()).pvalue > 1e-3


@pytest.mark.parametrize("cfg", [synth.TINY])
def test_verify_inputs_shapes(cfg):
    v = synth.verify_inputs(cfg)
    assert v.logits.shape == (cfg.B, cfg.R, cfg.V)
    assert v.draft_logits.shape == (cfg.B, cfg.N - 1, cfg.V)
    assert v.draft_ids.shape == (cfg.B, cfg.N - 1) and v.uniforms.shape == (cfg.B, cfg.R)


def test_proj_inputs_gate_pattern():
    p = synth.proj_inputs(synth.PROJ, M=14)
    assert p.gate.tolist() == [0, 0, 0, 1, 1, 1, 1] * 2
    assert p.w.shape == (4096, 4096) and p.a.shape == (128, 4096) and p.b.shape == (4096, 128)
