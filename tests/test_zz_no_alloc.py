"""isd_verify_noalloc against isd_verify: the entry point that allocates nothing (its
scratch is the library's fixed device array) gives the same outputs, bit for bit, as the
workspace entry point on the same inputs -- on two calls in a row, the second with a
smaller input -- and rejects shapes beyond the array before touching the GPU."""
import numpy as np
import pytest
import torch

from strided_verify_propose_amd import isd, synth
from tests.helpers import to_dev, to_np

KEYS = ("n_accept", "accept", "next_token", "argmax_ids", "sampled_ids", "p_draft", "q_draft", "row_lse")


def _inputs(cfg):
    v = synth.verify_inputs(cfg)
    return (to_dev(v.logits), None if v.draft_logits is None else to_dev(v.draft_logits),
            to_dev(v.draft_ids), to_dev(v.uniforms))


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_on_two_calls():
    big = synth.QWEN3_8B                                   # B=64, N=4, V=151936
    small = synth.StepConfig("noalloc_small", "bf16", B=5, N=3, Hq=1, Hkv=1, D=64, V=40000,
                             ctx=("fixed", 0), anchor_sd=3.0, noise_sd=0.3, seed=1701)
    for cfg in (big, small):
        print(f"noalloc case {cfg.name} B={cfg.B} N={cfg.N} V={cfg.V}", flush=True)
        args = _inputs(cfg)
        got = isd.verify_noalloc(*args)
        ref = isd.verify(*args)
        torch.cuda.synchronize()
        for k in KEYS:
            a, b = to_np(got[k]), to_np(ref[k])
            assert a.shape == b.shape, k
            assert np.array_equal(a, b), f"{cfg.name}: {k} differs from isd_verify"


def test_noalloc_rejects_shapes_beyond_the_array():
    L = isd.lib()
    need = L.isd_verify_workspace_bytes(65535, 8, 1 << 20)
    assert need > (8 << 20)
    fake = __import__("ctypes").c_void_p(0x1000)
    st = L.isd_verify_noalloc(1, fake, fake, fake, fake, 65535, 8, 1 << 20, 1.0, fake, fake, fake, fake,
                              fake, None, None, None, None)
    assert st == 2
    assert b"scratch" in L.isd_last_error()
