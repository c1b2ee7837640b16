"""GPU parity of isd_gated_lora_proj: oracle tolerance, bit-identity of ungated rows."""
import numpy as np
import pytest
import torch

import oracle
from strided_verify_propose_amd import isd, synth
from tests.helpers import assert_close, to_dev, to_np

pytestmark = pytest.mark.gpu


def run(M, K, Nout, r, seed, pattern=(0, 0, 0, 1, 1, 1, 1)):
    cfg = synth.ProjConfig("p", B=1, N=1, K=K, Nout=Nout, r=r, x_sd=1.0, w_sd=0.02, seed=seed,
                           gate_pattern=pattern)
    p = synth.proj_inputs(cfg, M=M)
    print(f"projection case M={M} K={K} Nout={Nout} r={r}", flush=True)
    x, w, a, b, gate = (to_dev(t) for t in (p.x, p.w, p.a, p.b, p.gate))
    y = isd.gated_lora_proj(x, w, a, b, gate)
    y2 = isd.gated_lora_proj(x, w, a, b, gate)
    yb = isd.gated_lora_proj(x, w)
    # the packed-weight path computes the same MFMA sequence: bit-identical results
    pk = isd.pack_proj_weights(w, a, b)
    yp = isd.gated_lora_proj_packed(x, pk, gate)
    ybp = isd.gated_lora_proj_packed(x, pk)
    ybp0 = isd.gated_lora_proj_packed(x, isd.pack_proj_weights(w))
    # packing from the y = x W storage gives the same buffer, byte for byte
    pk_kn = isd.pack_proj_weights_kn(w.t().contiguous(), a.t().contiguous(), b.t().contiguous())
    pk0, pk0_kn = isd.pack_proj_weights(w), isd.pack_proj_weights_kn(w.t().contiguous())
    torch.cuda.synchronize()
    assert torch.equal(pk_kn.data.view(torch.int16), pk.data.view(torch.int16)), "packed from [K, Nout] differs"
    assert torch.equal(pk0_kn.data.view(torch.int16), pk0.data.view(torch.int16)), "base-only packing differs"
    assert torch.equal(y, y2), "not deterministic"
    assert torch.equal(yp, y), "packed path differs from the row-major path"
    assert torch.equal(ybp, yb) and torch.equal(ybp0, yb), "packed base-only path differs"
    g = p.gate.astype(bool)
    Y, Yb = to_np(y), to_np(yb)
    assert np.array_equal(Y[~g], Yb[~g]), "ungated rows differ from the base-only call"
    ref = oracle.gated_lora_proj(p.x, p.w, p.a, p.b, p.gate)
    worst = assert_close(Y, ref, 2e-2, "gated projection")
    assert_close(Yb, oracle.gated_lora_proj(p.x, p.w), 2e-2, "base projection")
    print(f"  worst relative error {worst:.3e}", flush=True)


def test_rlora_full_size():
    """448 = 64 requests x 7 rows, K = Nout = 4096, rank 128, gate 0001111 per request."""
    run(448, 4096, 4096, 128, 1004)


@pytest.mark.parametrize("M,K,Nout,r", [(1, 64, 128, 128), (130, 512, 256, 128),
                                        (7, 4096, 128, 256), (300, 1024, 640, 128),
                                        (448, 4096, 1024, 128), (7, 4096, 4096, 128),
                                        (112, 12288, 4096, 128), (65536, 64, 128, 128),
                                        (1300, 4096, 4096, 128), (448, 12288, 3072, 128),
                                        (448, 6144, 6144, 256)])
def test_ragged_shapes(M, K, Nout, r):
    """Includes shapes with few tiles, whose K is split over 2, 4 or 8 workgroups, the
    largest M (65536 rows, 1024 row tiles), and the large-tile path: 224 x 256 tiles over 2
    K ranges with a ragged last row tile (1300 rows), over 8 ranges (K = 12288), and over 4
    with rank 256 (two column tiles of A^T rows)."""
    run(M, K, Nout, r, 7 + M)


def test_all_gated_and_none_gated():
    run(64, 256, 128, 128, 3, pattern=(1,))
    run(64, 256, 128, 128, 4, pattern=(0,))


def test_packed_layout():
    """The packed buffer follows the documented layout: S = [w; a] in fragments, fragment
    (nb, kb) holding S[16 nb + l % 16][32 kb + 8 (l / 16) + e] at ((nb (K/32) + kb) 64 + l) 8 + e,
    then b as it is."""
    rng = np.random.default_rng(5)
    K, Nout, r = 128, 256, 128
    w = rng.integers(0, 1 << 16, size=(Nout, K), dtype=np.uint16)
    a = rng.integers(0, 1 << 16, size=(r, K), dtype=np.uint16)
    b = rng.integers(0, 1 << 16, size=(Nout, r), dtype=np.uint16)
    pk = isd.pack_proj_weights(to_dev(w), to_dev(a), to_dev(b))
    got = to_np(pk.data)

    def frag_order(S):
        n, k = S.shape
        return S.reshape(n // 16, 16, k // 32, 4, 8).transpose(0, 2, 3, 1, 4).ravel()

    want = np.concatenate([frag_order(np.concatenate([w, a])), b.ravel()])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [56, 448, 1344])
def test_back_to_back_calls_are_identical(M):
    """Many calls in a row without synchronising, on 64 x 128 tiles with K split (56 rows)
    and without (448 rows), and on the large-tile path (1344 rows), on both weight layouts:
    every result bitwise
    equal to the first.  Covers the order of the first LDS refill against the waves' first
    fragment reads."""
    cfg = synth.ProjConfig("b2b", B=8, N=4, K=4096, Nout=4096, r=128, x_sd=1.0, w_sd=0.02, seed=2030)
    p = synth.proj_inputs(cfg, M=M)
    x, w, a, b, g = (to_dev(t) for t in (p.x, p.w, p.a, p.b, p.gate))
    packed = isd.pack_proj_weights(w, a, b)
    print(f"back-to-back projection M={M}", flush=True)
    for call in (lambda o: isd.gated_lora_proj(x, w, a, b, g, out=o),
                 lambda o: isd.gated_lora_proj_packed(x, packed, g, out=o)):
        outs = [torch.empty((M, cfg.Nout), dtype=torch.bfloat16, device="cuda") for _ in range(40)]
        for o in outs:
            call(o)
        torch.cuda.synchronize()
        for i, o in enumerate(outs[1:], 1):
            assert torch.equal(o, outs[0]), f"call {i} differs from call 0"
