"""GPU parity of isd_attention_step against the oracle (outputs and the appended cache)."""
import numpy as np
import pytest
import torch

import oracle
from strided_verify_propose_amd import isd, synth
from tests.helpers import RTOL, assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def step_cfg(name, dtype, B, N, Hq, Hkv, D, seed):
    return synth.StepConfig(name, dtype, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=2, ctx=("fixed", 0),
                            anchor_sd=1, noise_sd=1, seed=seed)


def device_inputs(inp):
    k_tiles = synth.k_tile_layout(inp.k_pages)
    v_tiles = synth.v_tile_layout(inp.v_pages)
    return dict(q=to_dev(inp.q), k_new=to_dev(inp.k_new), v_new=to_dev(inp.v_new),
                k_cache=to_dev(k_tiles), v_cache=to_dev(v_tiles),
                page_table=to_dev(inp.page_table), ctx_lens=to_dev(inp.ctx_lens))


def run(cfg, ctx_lens=None, sample=None, repeats=1):
    inp = synth.attention_inputs(cfg, ctx_lens=ctx_lens)
    print(f"attention case {cfg.name} dtype={cfg.dtype} B={cfg.B} N={cfg.N} Hq={cfg.Hq} "
          f"Hkv={cfg.Hkv} D={cfg.D} ctx={inp.ctx_lens.tolist()[:8]}", flush=True)
    d = device_inputs(inp)
    maxctx = int(inp.ctx_lens.max())
    outs = []
    for _ in range(repeats):
        outs.append(isd.attention_step(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"],
                                       d["page_table"], d["ctx_lens"], maxctx))
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "repeated call differs"
    out = to_np(outs[0])
    # expected cache: the oracle's append, then the tile layout
    kp, vp = oracle.attention.append_block(inp.k_pages, inp.v_pages, inp.k_new, inp.v_new,
                                           inp.page_table, inp.ctx_lens)
    assert np.array_equal(to_np(d["k_cache"]), synth.k_tile_layout(kp)), "K cache after append"
    assert np.array_equal(to_np(d["v_cache"]), synth.v_tile_layout(vp)), "V cache after append"
    bs = np.arange(cfg.B) if sample is None else np.asarray(sample)
    ref, _, _ = oracle.attention_step(inp.q[bs], inp.k_new[bs], inp.v_new[bs], inp.k_pages,
                                      inp.v_pages, inp.page_table[bs], inp.ctx_lens[bs], inp.scale)
    worst = assert_close(out[bs], ref, RTOL[cfg.dtype], "attention output")
    print(f"  worst relative error {worst:.3e}", flush=True)


def test_tiny_fp32():
    run(synth.TINY)


def test_tiny_fp32_ragged_contexts():
    run(step_cfg("f32_ragged", "f32", 4, 3, 8, 2, 64, 101), ctx_lens=[0, 1, 17, 300])


RAGGED = [0, 1, 15, 16, 17, 31, 511, 512, 513, 1100, 2047]


@pytest.mark.parametrize("name,N,Hq,Hkv,D", [
    ("g4_d128_n4", 4, 32, 8, 128),
    ("g8_d128_n4_four_blocks", 4, 64, 8, 128),
    ("g1_d128_n4", 4, 8, 8, 128),
    ("g2_d64_n3", 3, 8, 4, 64),
    ("g4_d64_n1", 1, 16, 4, 64),
    ("g4_d128_n8_60rows", 8, 8, 2, 128),
    ("g6_d128_n4_three_blocks", 4, 48, 8, 128),  # two wave groups, the second with one block
    ("g4_d128_n2_one_block", 2, 32, 8, 128),     # 12 query rows: one block over eight waves
])
def test_bf16_ragged_contexts(name, N, Hq, Hkv, D):
    run(step_cfg(name, "bf16", len(RAGGED), N, Hq, Hkv, D, 200 + N), ctx_lens=RAGGED, repeats=2)


def test_qwen3_8b_full_size():
    """B=64, 32 query / 8 KV heads, D=128, N=4, contexts ~ U[512, 4096]; oracle on 6 requests."""
    run(synth.QWEN3_8B, sample=[0, 1, 17, 33, 50, 63])


def test_qwen3_32b_full_size():
    """B=64, 64 query / 8 KV heads, N=4, contexts ~ U[2048, 8192]; oracle on 3 requests."""
    run(synth.QWEN3_32B, sample=[0, 31, 63])


def test_long_context_many_pieces():
    """One 32000-token request next to a 5-token one: each long item is cut into ~64
    pieces, so the combine stages its pieces in several chunks."""
    run(step_cfg("long_ctx", "bf16", 2, 4, 32, 8, 128, 300), ctx_lens=[32000, 5], repeats=2)


def test_most_requests_per_call():
    """2048 requests (the bf16 path's limit), short ragged contexts: many items per
    workgroup, the cost prefix at its full length; the oracle checks a sample."""
    ctx = list(np.random.default_rng(5).integers(0, 41, 2048))
    run(step_cfg("max_b", "bf16", 2048, 2, 8, 2, 64, 301), ctx_lens=ctx,
        sample=[0, 1, 700, 1023, 1024, 2047])
