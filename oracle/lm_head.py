"""Oracle: the LM head in front of verification.  (Test infrastructure.)

What it follows:
  * One ISD forward turns the hidden states of the block's 2N-1 rows into vocabulary
    logits; the clean rows give the anchor p that verifies earlier proposals and the
    [MASK] rows give the proposal q (「首次超越 AR 模型」 "I-DLM 如何解決這些問題";
    「I-DLM – introspektive Diffusion Language Models」 "Inference & ISD").  The logits
    are the product of the hidden states with the output embedding, the usual LM head
    of the Qwen3 models the pages build on (「首次超越 AR 模型」 "模型生態與安裝").
  * The pages give no precision for the logits; they are read as stored in bf16 (the
    pages' serving dtype, 「首次超越 AR 模型」 "快速開始"), i.e. the nearest bf16 value of
    the exact product, and verification then runs on those stored values.

Storage: hidden [M, Dm] (M = B (2N-1) rows, request-major), w_lm [V, Dm] (the output
embedding in the linear-layer convention: one row of Dm weights per vocabulary entry).
"""
import numpy as np

from .stored import round_bf16, to_f64
from .verify import verify


def lm_head_logits(hidden, w_lm):
    """Stored logits [M, V] (float64 on the bf16 grid): nearest bf16 of hidden . w_lm^T."""
    return round_bf16(to_f64(hidden) @ to_f64(w_lm).T)


def lm_head_verify(hidden, w_lm, draft_logits, draft_ids, uniforms, N, temperature=1.0, eps=1e-6):
    """(logits [B, 2N-1, V], verification result) for the block rows' hidden states."""
    R = 2 * N - 1
    logits = lm_head_logits(hidden, w_lm)
    B = logits.shape[0] // R
    logits = logits.reshape(B, R, -1)
    return logits, verify(logits, draft_logits, draft_ids, uniforms, N, temperature, eps)
