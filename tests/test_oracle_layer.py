"""Pins for oracle.layer, the R-ISD decoder layer (seven gated linears around the
block's attention): brute force on tiny shapes, and the R-ISD invariants."""
import math

import numpy as np
import pytest

import oracle
from oracle.stored import round_bf16, to_bf16_bits, to_f64
from strided_verify_propose_amd import synth
from tests.test_oracle_proj import brute_proj, nearest_bf16_exact


def tiny(seed, B=2, N=3, ctx=("uniform", 0, 20), hidden=8, Hq=2, Hkv=1, D=4, inter=12, r=2):
    cfg = synth.LayerInputsConfig("tiny_layer", B=B, N=N, hidden=hidden, Hq=Hq, Hkv=Hkv, D=D,
                                  inter=inter, r=r, ctx=ctx, seed=seed)
    return synth.layer_inputs(cfg)


def run_oracle(inp, gated=True, gate=None):
    c, at = inp.cfg, inp.attn
    g = (inp.gate if gate is None else gate) if gated else None
    return oracle.decoder_layer(inp.x, inp.weights, at.k_pages, at.v_pages, at.page_table,
                                at.ctx_lens, c.Hq, c.Hkv, c.D, gate=g)


def brute_layer(inp, gated=True):
    """Pure-Python loops: math.fsum sums, math.exp, exact-rational bf16 rounding."""
    c, at = inp.cfg, inp.attn
    B, R, Hq, Hkv, D = c.B, c.R, c.Hq, c.Hkv, c.D
    G = Hq // Hkv
    M = c.M
    X = to_f64(inp.x)
    gate = inp.gate if gated else np.zeros(M, np.uint8)
    rnd = lambda v: nearest_bf16_exact(float(v))

    def lin(Y, name):
        w, a, b = (to_f64(t) for t in inp.weights[name])
        P = brute_proj(Y, w, a, b, gate)
        return np.array([[rnd(v) for v in row] for row in P])

    q, k, v = lin(X, "q"), lin(X, "k"), lin(X, "v")
    kp, vp = to_f64(at.k_pages), to_f64(at.v_pages)
    att = np.zeros((M, Hq * D))
    for b in range(B):
        L = int(at.ctx_lens[b])
        for r in range(R):
            for h in range(Hq):
                g = h // G
                keys = [kp[at.page_table[b, j // 16], g, j % 16] for j in range(L)]
                vals = [vp[at.page_table[b, j // 16], g, j % 16] for j in range(L)]
                keys += [k[b * R + t, g * D:(g + 1) * D] for t in range(r + 1)]
                vals += [v[b * R + t, g * D:(g + 1) * D] for t in range(r + 1)]
                qv = q[b * R + r, h * D:(h + 1) * D]
                s = [math.fsum(float(qv[d]) * float(kk[d]) for d in range(D)) / math.sqrt(D) for kk in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for d in range(D):
                    att[b * R + r, h * D + d] = rnd(math.fsum(e[j] * float(vals[j][d]) for j in range(len(e))) / tot)
    o = lin(att, "o")
    hh = np.array([[rnd(X[m, i] + o[m, i]) for i in range(c.hidden)] for m in range(M)])
    gt, up = lin(hh, "gate"), lin(hh, "up")
    act = np.array([[rnd(rnd(z / (1.0 + math.exp(-z))) * u) for z, u in zip(gr, ur)]
                    for gr, ur in zip(gt, up)])
    dn = lin(act, "down")
    out = np.array([[rnd(hh[m, i] + dn[m, i]) for i in range(c.hidden)] for m in range(M)])
    return out, k, v


@pytest.mark.parametrize("seed,gated", [(11, True), (12, True), (13, False)])
def test_layer_matches_brute_force(seed, gated):
    inp = tiny(seed)
    out, kp, vp = run_oracle(inp, gated)
    ref, k, v = brute_layer(inp, gated)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # the block's K/V sit in their slots after the call, as the projections produced them
    c, at = inp.cfg, inp.attn
    for b in range(c.B):
        for t in range(c.R):
            j = int(at.ctx_lens[b]) + t
            page = at.page_table[b, j // 16]
            for g in range(c.Hkv):
                assert np.array_equal(to_f64(kp[page, g, j % 16]), k[b * c.R + t, g * c.D:(g + 1) * c.D])
                assert np.array_equal(to_f64(vp[page, g, j % 16]), v[b * c.R + t, g * c.D:(g + 1) * c.D])


def test_gate_all_zero_is_the_base_only_layer():
    inp = tiny(21)
    zero = np.zeros(inp.cfg.M, np.uint8)
    a = run_oracle(inp, gated=True, gate=zero)
    b = run_oracle(inp, gated=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("seed,N", [(31, 2), (32, 4)])
def test_clean_rows_and_their_kv_equal_the_base_only_layer(seed, N):
    inp = tiny(seed, N=N, ctx=("uniform", 3, 40))
    c, at = inp.cfg, inp.attn
    out_g, kp_g, vp_g = run_oracle(inp, gated=True)
    out_b, kp_b, vp_b = run_oracle(inp, gated=False)
    clean = inp.gate == 0
    assert np.array_equal(out_g[clean], out_b[clean])
    assert not np.array_equal(out_g[~clean], out_b[~clean])
    for b in range(c.B):
        for t in range(c.N - 1):
            j = int(at.ctx_lens[b]) + t
            page = at.page_table[b, j // 16]
            assert np.array_equal(kp_g[page, :, j % 16], kp_b[page, :, j % 16])
            assert np.array_equal(vp_g[page, :, j % 16], vp_b[page, :, j % 16])


def test_silu_closed_values():
    assert oracle.layer.silu(0.0) == 0.0
    np.testing.assert_allclose(oracle.layer.silu(np.array([1.0, -2.0, 30.0])),
                               [1 / (1 + math.exp(-1)), -2 / (1 + math.exp(2)), 30 / (1 + math.exp(-30))], rtol=1e-15)


def test_bf16_bits_round_trip():
    rng = np.random.default_rng(5)
    vals = round_bf16(rng.standard_normal(1000) * 7)
    assert np.array_equal(to_f64(to_bf16_bits(vals)), vals)
    with pytest.raises(ValueError):
        to_bf16_bits(np.array([1.0 + 2.0 ** -10]))
