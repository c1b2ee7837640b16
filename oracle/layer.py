"""Oracle: one R-ISD decoder layer of the strided block.  (Test infrastructure.)

What it follows:
  * R-ISD puts a gated LoRA adapter on the linears: the rank-r delta acts only on gated
    ([MASK]) rows, and verify rows use the base weights alone, so their outputs are the
    base AR model's (「首次超越 AR 模型」 "無損 R-ISD"; 「I-DLM – introspektive Diffusion
    Language Models」 "Lossless R-ISD", and "Speedup Factor Explorer" for the overhead
    alpha of those deltas).  The layer applies that to every linear of a Qwen3-shaped
    decoder layer: q, k, v, o, gate, up, down.
  * Attention inside the layer is the strictly causal GQA attention of the block over the
    paged cache, appending the block's K/V first (oracle.attention).
  * Activations are stored in bf16, the pages' serving dtype (「首次超越 AR 模型」 "快速開始"):
    every stored intermediate is the nearest bf16 of its exact value.  RMSNorm and the
    rotary embedding act on one row at a time and change neither R-ISD property; they
    are identity here (a reading; the pages give no layer internals).

Composition, in order (each line's result rounded to bf16, as stored):
    q = proj_q(x)   k = proj_k(x)   v = proj_v(x)
    att = attention(q, k, v) over the cache, after appending k, v
    h   = x + proj_o(att)
    act = silu(proj_gate(h)) * proj_up(h)        silu(z) = z / (1 + e^-z), rounded, then the product
    out = h + proj_down(act)
where proj_n(y) = y W_n + g * bf16(y A_n) B_n (oracle.proj), with the same per-row gate g
on all seven linears.
"""
import math

import numpy as np

from .attention import attention_step
from .proj import gated_lora_proj
from .stored import round_bf16, to_bf16_bits, to_f64

LINEARS = ("q", "k", "v", "o", "gate", "up", "down")


def silu(z):
    """z * sigmoid(z), float64."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def residual(x, y):
    """A residual add of stored rows: the nearest bf16 of x + y."""
    return round_bf16(np.asarray(x, np.float64) + np.asarray(y, np.float64))


def linear(y, weights, name, gate):
    """One gated linear, output stored in bf16.  weights[name] = (w, a, b) stored bf16,
    w [Nout, K] = W^T, a [r, K] = A^T, b [Nout, r] = B^T (a, b unused when gate is None)."""
    w, a, b = weights[name]
    return round_bf16(gated_lora_proj(y, w, a, b, gate) if gate is not None else gated_lora_proj(y, w))


def decoder_layer(x, weights, k_pages, v_pages, page_table, ctx_lens, Hq, Hkv, D, gate=None,
                  scale=None):
    """Returns (out [M, hidden] float64 holding bf16 values, k_pages', v_pages').

    x [M, hidden] stored bf16, M = B (2N-1) rows, request-major; weights: dict of the
    seven linears (see linear); k_pages, v_pages [num_pages, Hkv, 16, D] stored bf16
    (logical layout); page_table [B, max_pages]; ctx_lens [B]; gate [M] in {0, 1} or None
    (base only)."""
    X = to_f64(x)
    M = X.shape[0]
    B = len(ctx_lens)
    R = M // B
    q = linear(X, weights, "q", gate)
    k = linear(X, weights, "k", gate)
    v = linear(X, weights, "v", gate)
    att, kp, vp = attention_step(q.reshape(B, R, Hq, D),
                                 to_bf16_bits(k).reshape(B, R, Hkv, D),
                                 to_bf16_bits(v).reshape(B, R, Hkv, D),
                                 k_pages, v_pages, page_table, ctx_lens,
                                 1.0 / math.sqrt(D) if scale is None else scale)
    att = round_bf16(att.reshape(M, Hq * D))
    h = residual(X, linear(att, weights, "o", gate))
    act = round_bf16(round_bf16(silu(linear(h, weights, "gate", gate))) * linear(h, weights, "up", gate))
    out = residual(h, linear(act, weights, "down", gate))
    return out, kp, vp
