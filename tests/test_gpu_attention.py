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


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_pack_kv_pages_is_the_tile_layout_and_round_trips(dtype, D):
    """isd_pack_kv_pages gives exactly the documented tile layout of logical pages, and
    isd_unpack_kv_pages gives them back, bit for bit."""
    cfg = step_cfg("pack_pages", dtype, 3, 4, 8, 2, D, 131)
    inp = synth.attention_inputs(cfg, ctx_lens=[5, 40, 300])
    print(f"pack_kv_pages {dtype} D={D} pages={inp.num_pages}", flush=True)
    kc, vc = isd.pack_kv_pages(to_dev(inp.k_pages), to_dev(inp.v_pages))
    torch.cuda.synchronize()
    assert np.array_equal(to_np(kc), synth.k_tile_layout(inp.k_pages))
    assert np.array_equal(to_np(vc), synth.v_tile_layout(inp.v_pages))
    kp, vp = isd.unpack_kv_pages(kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(kp), inp.k_pages)
    assert np.array_equal(to_np(vp), inp.v_pages)


def test_plain_c_step_from_logical_pages(tmp_path):
    """A C program using only include/isd.h and the HIP runtime packs logical pages,
    runs the step and unpacks the cache; the output matches the oracle and the cache
    after the step is the oracle's append, bit for bit."""
    import os
    import shutil
    import subprocess
    from tests.test_abi_c import ROOT
    from strided_verify_propose_amd.build import LIB
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "step_from_pages"
    libdir = os.path.dirname(LIB)
    subprocess.run([gcc, "-std=c99", "-O1", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "c", "step_from_pages.c"), "-o", str(exe),
                    "-L", libdir, "-lisd", f"-Wl,-rpath,{libdir}", "-L", "/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-lm"], check=True)
    cfg = step_cfg("c_pages", "bf16", 4, 4, 32, 8, 128, 141)
    inp = synth.attention_inputs(cfg, ctx_lens=[0, 17, 513, 1100])
    print(f"c caller step B={cfg.B} ctx={inp.ctx_lens.tolist()} pages={inp.num_pages}", flush=True)
    hdr = np.array([cfg.B, cfg.N, cfg.Hq, cfg.Hkv, cfg.D, inp.num_pages, inp.page_table.shape[1],
                    int(inp.ctx_lens.max())], np.int32)
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        for a in (hdr, inp.q, inp.k_new, inp.v_new, inp.k_pages, inp.v_pages,
                  inp.page_table.astype(np.int32), inp.ctx_lens.astype(np.int32)):
            f.write(np.ascontiguousarray(a).tobytes())
    dst = tmp_path / "out.bin"
    res = subprocess.run([str(exe), str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    raw = np.fromfile(dst, np.uint16)
    nq, npg = inp.q.size, inp.k_pages.size
    out = raw[:nq].reshape(inp.q.shape)
    kp = raw[nq:nq + npg].reshape(inp.k_pages.shape)
    vp = raw[nq + npg:].reshape(inp.v_pages.shape)
    ref, rkp, rvp = oracle.attention_step(inp.q, inp.k_new, inp.v_new, inp.k_pages, inp.v_pages,
                                          inp.page_table, inp.ctx_lens, inp.scale)
    assert np.array_equal(kp, rkp) and np.array_equal(vp, rvp), "cache after the step"
    assert_close(out, ref, RTOL["bf16"], "attention output from the C caller")


def test_stale_slots_past_the_context_change_nothing():
    """Rollback is not advancing ctx_lens: the slots of rejected drafts stay in the cache.
    With those slots (and every other slot past each context, up to the end of its pages)
    filled with garbage -- huge values and NaN bit patterns -- the step's output is
    bitwise the output on a clean cache, and the block's append overwrites its slots."""
    cfg = step_cfg("stale_slots", "bf16", 4, 4, 32, 8, 128, 151)
    inp = synth.attention_inputs(cfg, ctx_lens=[3, 16, 37, 700])
    print(f"stale slots ctx={inp.ctx_lens.tolist()}", flush=True)
    dirty_k, dirty_v = inp.k_pages.copy(), inp.v_pages.copy()
    rng = np.random.default_rng(7)
    for b in range(cfg.B):
        for j in range(int(inp.ctx_lens[b]), (int(inp.ctx_lens[b]) + cfg.R + 15) // 16 * 16):
            p = inp.page_table[b, j // 16]
            junk = rng.choice(np.array([0x7FC0, 0xFFC0, 0x7F7F, 0x4B00], np.uint16), size=(cfg.Hkv, cfg.D))
            dirty_k[p, :, j % 16] = junk
            dirty_v[p, :, j % 16] = junk[:, ::-1]
    outs = []
    for kp, vp in ((inp.k_pages, inp.v_pages), (dirty_k, dirty_v)):
        d = device_inputs(inp)
        d["k_cache"], d["v_cache"] = to_dev(synth.k_tile_layout(kp)), to_dev(synth.v_tile_layout(vp))
        o = isd.attention_step(d["q"], d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["page_table"],
                               d["ctx_lens"], int(inp.ctx_lens.max()))
        torch.cuda.synchronize()
        outs.append((to_np(o), synth.k_logical_layout(to_np(d["k_cache"]), cfg.D),
                     synth.v_logical_layout(to_np(d["v_cache"]), cfg.D)))
    assert np.array_equal(outs[0][0], outs[1][0]), "stale slots changed the output"
    for b in range(cfg.B):
        for t in range(cfg.R):
            j = int(inp.ctx_lens[b]) + t
            p = inp.page_table[b, j // 16]
            assert np.array_equal(outs[1][1][p, :, j % 16], inp.k_new[b, t])
            assert np.array_equal(outs[1][2][p, :, j % 16], inp.v_new[b, t])
