"""Pins for oracle.attention: brute force, library special cases, invariants."""
import math

import numpy as np
import pytest
import torch

import oracle
from strided_verify_propose_amd import synth


def build_case(seed, B, N, Hq, Hkv, D, Ls, dtype="f32"):
    """Per-request logical token sequences, then paged through a random page table.
    Returns (pages inputs for the oracle, the plain sequences for brute force)."""
    rng = np.random.default_rng(seed)
    R = 2 * N - 1
    enc = (lambda a: a.astype(np.float32)) if dtype == "f32" else synth.bf16_rne
    dec = (lambda a: a.astype(np.float64)) if dtype == "f32" else \
        (lambda a: synth.bf16_bits_to_f32(a).astype(np.float64))
    seqs_k = [enc(rng.standard_normal((L, Hkv, D)).astype(np.float32)) for L in Ls]
    seqs_v = [enc(rng.standard_normal((L, Hkv, D)).astype(np.float32)) for L in Ls]
    q = enc(rng.standard_normal((B, R, Hq, D)).astype(np.float32))
    kn = enc(rng.standard_normal((B, R, Hkv, D)).astype(np.float32))
    vn = enc(rng.standard_normal((B, R, Hkv, D)).astype(np.float32))
    npg = [(L + R + 15) // 16 for L in Ls]
    perm = rng.permutation(sum(npg))
    table = np.zeros((B, max(npg)), np.int32)
    kp = np.zeros((sum(npg), Hkv, 16, D), q.dtype)
    vp = np.zeros_like(kp)
    off = 0
    for b, L in enumerate(Ls):
        table[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
        for j in range(L):
            kp[table[b, j // 16], :, j % 16] = seqs_k[b][j]
            vp[table[b, j // 16], :, j % 16] = seqs_v[b][j]
        # stale garbage in the block's slots must be overwritten by the append
        for j in range(L, L + R):
            kp[table[b, j // 16], :, j % 16] = enc(np.full((Hkv, D), 9.0, np.float32))
    ctx = np.asarray(Ls, np.int32)
    seq = dict(k=[dec(s) for s in seqs_k], v=[dec(s) for s in seqs_v],
               q=dec(q), kn=dec(kn), vn=dec(vn))
    return (q, kn, vn, kp, vp, table, ctx), seq


def brute_force(seq, B, N, Hq, Hkv, D, Ls):
    """Pure-Python loops with math.exp over the unpaged sequences."""
    R = 2 * N - 1
    G = Hq // Hkv
    out = np.zeros((B, R, Hq, D))
    for b in range(B):
        L = Ls[b]
        for h in range(Hq):
            g = h // G
            for r in range(R):
                keys = [seq["k"][b][j, g] for j in range(L)] + [seq["kn"][b, t, g] for t in range(r + 1)]
                vals = [seq["v"][b][j, g] for j in range(L)] + [seq["vn"][b, t, g] for t in range(r + 1)]
                qv = seq["q"][b, r, h]
                s = [sum(float(qv[d]) * float(kk[d]) for d in range(D)) / math.sqrt(D) for kk in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                tot = math.fsum(e)
                for d in range(D):
                    out[b, r, h, d] = math.fsum(e[j] * float(vals[j][d]) for j in range(len(e))) / tot
    return out


@pytest.mark.parametrize("seed,B,N,Hq,Hkv,D,Ls,dtype", [
    (1, 1, 2, 4, 1, 8, [21], "f32"),
    (2, 2, 4, 4, 2, 16, [0, 40], "f32"),
    (3, 2, 3, 2, 2, 8, [16, 31], "bf16"),
    (4, 1, 1, 4, 4, 16, [33], "bf16"),
    (5, 2, 4, 8, 2, 8, [5, 17], "f32"),
])
def test_attention_matches_brute_force(seed, B, N, Hq, Hkv, D, Ls, dtype):
    args, seq = build_case(seed, B, N, Hq, Hkv, D, Ls, dtype)
    out, _, _ = oracle.attention_step(*args)
    ref = brute_force(seq, B, N, Hq, Hkv, D, Ls)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_tiny_config_matches_brute_force():
    cfg = synth.TINY
    inp = synth.attention_inputs(cfg)
    out, kp, vp = oracle.attention_step(inp.q, inp.k_new, inp.v_new, inp.k_pages, inp.v_pages,
                                        inp.page_table, inp.ctx_lens)
    L = int(inp.ctx_lens[0])
    seq = dict(k=[oracle.stored.to_f64(np.stack([inp.k_pages[inp.page_table[0, j // 16], :, j % 16]
                                                  for j in range(L)]))],
               v=[oracle.stored.to_f64(np.stack([inp.v_pages[inp.page_table[0, j // 16], :, j % 16]
                                                  for j in range(L)]))],
               q=inp.q.astype(np.float64), kn=inp.k_new.astype(np.float64),
               vn=inp.v_new.astype(np.float64))
    # one query head is enough to pin the shape (full brute force is slow in pure Python)
    ref = brute_force(seq, 1, cfg.N, 1, 1, cfg.D, [L])
    np.testing.assert_allclose(out[:, :, :1], ref, rtol=1e-12, atol=1e-12)


def _sdpa(q, k, v, mask):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=torch.from_numpy(mask)).numpy()


def test_stride_one_is_paged_decode_attention():
    """N=1 (one query row): ordinary decode attention over L+1 keys, via torch SDPA."""
    B, N, Hq, Hkv, D, Ls = 3, 1, 8, 2, 32, [7, 50, 16]
    args, seq = build_case(11, B, N, Hq, Hkv, D, Ls)
    out, _, _ = oracle.attention_step(*args)
    G = Hq // Hkv
    for b in range(B):
        K = np.concatenate([seq["k"][b], seq["kn"][b]], 0)       # [L+1, Hkv, D]
        V = np.concatenate([seq["v"][b], seq["vn"][b]], 0)
        q = seq["q"][b, 0][:, None, :]                              # [Hq, 1, D]
        k = np.repeat(K.transpose(1, 0, 2), G, axis=0)              # [Hq, L+1, D]
        v = np.repeat(V.transpose(1, 0, 2), G, axis=0)
        ref = _sdpa(q, k, v, np.zeros((1, K.shape[0])))
        np.testing.assert_allclose(out[b, 0], ref[:, 0], rtol=1e-10, atol=1e-12)


def test_empty_context_is_causal_self_attention():
    """L=0: plain causal self-attention over the 2N-1 block rows, via torch SDPA."""
    B, N, Hq, Hkv, D = 2, 4, 4, 1, 16
    args, seq = build_case(12, B, N, Hq, Hkv, D, [0, 0])
    out, _, _ = oracle.attention_step(*args)
    R = 2 * N - 1
    causal = np.where(np.tril(np.ones((R, R))) > 0, 0.0, -np.inf)
    for b in range(B):
        for h in range(Hq):
            q = seq["q"][b, :, h]
            k = seq["kn"][b, :, h // (Hq // Hkv)]
            v = seq["vn"][b, :, h // (Hq // Hkv)]
            np.testing.assert_allclose(out[b, :, h], _sdpa(q, k, v, causal), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_append_writes_block_bitwise(dtype):
    B, N, Ls = 2, 3, [13, 30]
    args, _ = build_case(13, B, N, 4, 2, 16, Ls, dtype)
    q, kn, vn, kp, vp, table, ctx = args
    _, kp2, vp2 = oracle.attention_step(*args)
    for b in range(B):
        for r in range(2 * N - 1):
            j = Ls[b] + r
            assert np.array_equal(kp2[table[b, j // 16], :, j % 16], kn[b, r])
            assert np.array_equal(vp2[table[b, j // 16], :, j % 16], vn[b, r])
    # every other slot is untouched
    mask = np.ones(kp.shape[:3], bool)
    for b in range(B):
        for r in range(2 * N - 1):
            j = Ls[b] + r
            mask[table[b, j // 16], :, j % 16] = False
    assert np.array_equal(kp2[mask], kp[mask]) and np.array_equal(vp2[mask], vp[mask])


def test_row_sees_itself_but_not_later_rows():
    """Row r depends on block row r (diagonal included) and not on rows > r."""
    B, N, Hq, Hkv, D, Ls = 1, 4, 2, 1, 8, [10]
    args, _ = build_case(14, B, N, Hq, Hkv, D, Ls)
    base, _, _ = oracle.attention_step(*args)
    R = 2 * N - 1
    for t in range(R):
        q, kn, vn, kp, vp, table, ctx = args
        vn2 = vn.copy()
        vn2[0, t] += np.float32(1.0)
        out, _, _ = oracle.attention_step(q, kn, vn2, kp, vp, table, ctx)
        changed = np.abs(out - base).max(axis=(2, 3))[0]
        assert np.all(changed[:t] == 0) and np.all(changed[t:] > 0)
