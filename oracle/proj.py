"""Oracle: R-ISD gated residual adaptation of one linear layer.  (Test infrastructure.)

What it follows:
  * R-ISD adds a gated LoRA adapter that is active only at [MASK] positions; verify
    positions use the base weights alone, so their outputs are those of the base AR
    model bit for bit (「首次超越 AR 模型」 "無損 R-ISD"; 「内省扩散语言模型」 "1. 引言", gated residual
    adaptation; 「I-DLM – introspektive Diffusion Language Models」 "Speedup Factor Explorer" and "Lossless R-ISD").  Rank 128.
  * No LoRA scaling factor is given: the delta is added with scale 1, and the low-rank
    product X A is taken in the operand type of the second contraction (bf16).

Storage (the usual linear-layer convention): w is W^T [Nout, K], a is A^T [r, K],
b is B^T [Nout, r], so that  Y = X W + g * (bf16(X A)) B  with g in {0, 1} per row.

Rows with g = 0 come out of the very same base product as a gate-free call, so they
are identical to it by construction.
"""
import numpy as np

from .stored import round_bf16, to_f64


def gated_lora_proj(x, w, a=None, b=None, gate=None):
    """Y [M, Nout] float64."""
    X = to_f64(x)
    Y = X @ to_f64(w).T                                  # base product, every row
    if gate is None:
        return Y
    rows = np.flatnonzero(np.asarray(gate) != 0)
    if rows.size:
        T = round_bf16(X[rows] @ to_f64(a).T)            # [M_g, r]
        Y[rows] = Y[rows] + T @ to_f64(b).T
    return Y
