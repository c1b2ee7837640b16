"""R-ISD through a whole decoder layer of Qwen3-8B's shape: the clean rows' outputs and
the K/V they append equal the base-only layer's bit for bit; the gated rows differ."""
import pytest
import torch

from strided_verify_propose_amd.layer import LayerConfig, RIsdLayer

pytestmark = pytest.mark.gpu


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
