"""Oracle: attention of one ISD step over a paged KV cache.  (Test infrastructure.)

What it follows:
  * The block of one step holds 2N-1 query positions per request (「首次超越 AR 模型」 section
    "為什麼 I-DLM 能在高並發下保持高效": seven queries per forward at N=4).
  * Attention is strictly causal, which is what lets the model run on an AR serving
    stack (「首次超越 AR 模型」 "實際部署：SGLang 整合"; 「I-DLM – introspektive Diffusion Language Models」 "I-DLM-Methodik", AR-kompatibles Serving).
    Read as: row r of the block sees every cached token and block rows 0..r, itself
    included -- no bidirectional attention inside the block.
  * K/V live in a paged cache and the attention kernel reads them only through the
    pages (「首次超越 AR 模型」 "實際部署：SGLang 整合", paged KV cache and paged-only attention kernel;
    「I-DLM – introspektive Diffusion Language Models」 "Serving (SGLang)").  So the block's K/V are first written to their slots,
    then every key is gathered through the page table.
  * GQA: query head h reads KV head floor(h / (Hq/Hkv)); scale 1/sqrt(D); Q and K
    arrive after any positional transform.  (Head counts come from the Qwen3 shapes.)

Definition computed (float64):  for request b, query head h, block row r,
    keys j = 0 .. L_b + r,  s_j = scale * <q[b,r,h], k_j>,
    out[b,r,h] = sum_j softmax(s)_j v_j.
"""
import math

import numpy as np

from .stored import to_f64

PAGE = 16


def append_block(k_pages, v_pages, k_new, v_new, page_table, ctx_lens):
    """Copy block row r of request b into slot ctx_lens[b] + r (bit copy, stored dtype)."""
    kp = np.array(k_pages, copy=True)
    vp = np.array(v_pages, copy=True)
    B, R = k_new.shape[:2]
    for b in range(B):
        for r in range(R):
            j = int(ctx_lens[b]) + r
            page = int(page_table[b, j // PAGE])
            kp[page, :, j % PAGE, :] = k_new[b, r]
            vp[page, :, j % PAGE, :] = v_new[b, r]
    return kp, vp


def gather_keys(pages, page_table_row, n):
    """Tokens 0..n-1 of one request through its page table: [n, Hkv, D] float64."""
    j = np.arange(n)
    return to_f64(pages[page_table_row[j // PAGE], :, j % PAGE, :])


def causal_extent(L_b, r):
    """Number of keys block row r sees: the L_b cached tokens and block rows 0..r."""
    return L_b + r + 1


def attention_step(q, k_new, v_new, k_pages, v_pages, page_table, ctx_lens, scale=None):
    """Returns (out [B,R,Hq,D] float64, k_pages_after, v_pages_after).

    q [B,R,Hq,D]; k_new, v_new [B,R,Hkv,D]; k_pages, v_pages [num_pages,Hkv,16,D]
    (logical layout: page, kv head, slot, dim); page_table [B,max_pages] int;
    ctx_lens [B] = tokens cached before the block."""
    Q = to_f64(q)
    B, R, Hq, D = Q.shape
    Hkv = k_new.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kp, vp = append_block(k_pages, v_pages, k_new, v_new, page_table, ctx_lens)
    out = np.zeros((B, R, Hq, D))
    for b in range(B):
        Lb = int(ctx_lens[b])
        K = gather_keys(kp, page_table[b], Lb + R)
        V = gather_keys(vp, page_table[b], Lb + R)
        for h in range(Hq):
            g = h // G
            for r in range(R):
                n = causal_extent(Lb, r)
                s = scale * (K[:n, g, :] @ Q[b, r, h, :])
                e = np.exp(s - s.max())
                out[b, r, h] = (e / e.sum()) @ V[:n, g, :]
    return out, kp, vp
