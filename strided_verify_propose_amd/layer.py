"""An R-ISD decoder layer of Qwen3-8B's shape, built from the library's calls, to show the
two properties the pages claim for R-ISD at the scale of a layer (「首次超越 AR 模型」
"無損 R-ISD"; 「I-DLM – introspektive Diffusion Language Models」 "Lossless R-ISD"):
  * every linear applies its rank-r delta only on gated ([MASK]) rows, so the clean rows'
    outputs -- and the K/V they append to the cache -- equal the base model's bit for bit;
  * the cost of the deltas (the overhead alpha over the base-only layer).
Layer: q, k, v projections (hidden 4096 -> 32 x 128, 8 x 128, 8 x 128), strictly causal
attention over the paged cache (appending the block's K/V), o projection and residual,
gate and up projections (-> 12288), silu(gate) * up, down projection and residual.
RMSNorm and the rotary embedding act on one row at a time and leave both properties
as they are; they are left out (identity).  Weights are random (no trained weights are
available), the LoRA factors on all seven linears, rank 128.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import isd

PAGE = 16


@dataclass
class LayerConfig:
    B: int = 64
    N: int = 4
    hidden: int = 4096
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    inter: int = 12288
    r: int = 128
    ctx0: tuple = (512, 4096)
    seed: int = 1600


class RIsdLayer:
    LINEARS = ("q", "k", "v", "o", "gate", "up", "down")

    def __init__(self, cfg: LayerConfig, device="cuda", inputs=None):
        """Random weights, cache and block rows drawn on the device (a torch generator
        seeded with cfg.seed), or, with `inputs` (synth.LayerInputs of the same shapes),
        exactly those seeded host arrays."""
        self.cfg = c = cfg
        dev = self.dev = torch.device(device)
        bf = torch.bfloat16
        H, I, r = c.hidden, c.inter, c.r
        B, R = c.B, 2 * c.N - 1
        self.R, self.M = R, B * R
        shapes = dict(q=(H, c.Hq * c.D), k=(H, c.Hkv * c.D), v=(H, c.Hkv * c.D), o=(c.Hq * c.D, H),
                      gate=(H, I), up=(H, I), down=(I, H))
        self.packed = {}
        if inputs is not None:
            from . import synth
            ic = inputs.cfg
            if (ic.B, ic.N, ic.hidden, ic.Hq, ic.Hkv, ic.D, ic.inter, ic.r) != \
                    (c.B, c.N, H, c.Hq, c.Hkv, c.D, I, r):
                raise ValueError("layer inputs were drawn for other shapes")
            bits = lambda a: torch.from_numpy(a.view("int16")).view(bf).to(dev)
            for name in self.LINEARS:
                w, a, b = inputs.weights[name]
                self.packed[name] = isd.pack_proj_weights(bits(w), bits(a), bits(b))
            at = inputs.attn
            self.ctx_lens = torch.from_numpy(at.ctx_lens).to(dev)
            self.max_ctx = int(at.ctx_lens.max())
            self.page_table = torch.from_numpy(at.page_table).to(dev)
            self.k_cache = bits(synth.k_tile_layout(at.k_pages))
            self.v_cache = bits(synth.v_tile_layout(at.v_pages))
            self.x = bits(inputs.x)
            self.gate = torch.from_numpy(inputs.gate).to(dev)
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(c.seed)
            for name in self.LINEARS:
                K, Nout = shapes[name]
                w = (torch.randn((Nout, K), generator=g, device=dev) / K ** 0.5).to(bf)
                a = (torch.randn((r, K), generator=g, device=dev) / K ** 0.5).to(bf)
                b = (torch.randn((Nout, r), generator=g, device=dev) * 0.02).to(bf)
                self.packed[name] = isd.pack_proj_weights(w, a, b)
            lo, hi = c.ctx0
            self.ctx_lens = torch.randint(lo, hi + 1, (B,), generator=g, device=dev, dtype=torch.int32)
            self.max_ctx = hi
            pages = (hi + R + PAGE - 1) // PAGE
            perm = torch.randperm(B * pages, generator=g, device=dev).to(torch.int32)
            self.page_table = perm.view(B, pages).contiguous()
            P = B * pages
            self.k_cache = torch.randn((P, c.Hkv, c.D // 8, PAGE, 8), generator=g, device=dev).to(bf)
            self.v_cache = torch.randn((P, c.Hkv, c.D // 16, 4, PAGE, 4), generator=g, device=dev).to(bf)
            self.x = torch.randn((self.M, H), generator=g, device=dev).to(bf)
            # clean rows (the N-1 verify rows) base-only; the bonus row and the [MASK] rows gated
            self.gate = torch.tensor(([0] * (c.N - 1) + [1] * c.N) * B, dtype=torch.uint8, device=dev)
        self.att_out = torch.empty((B, R, c.Hq, c.D), dtype=bf, device=dev)

    def forward(self, gated: bool = True):
        """One layer over the block's rows; returns the layer output [M, hidden].  With
        gated=False every linear is the base-only call."""
        c, B, R = self.cfg, self.cfg.B, self.R
        gate = self.gate if gated else None
        proj = lambda x, name: isd.gated_lora_proj_packed(x, self.packed[name], gate)
        q = proj(self.x, "q").view(B, R, c.Hq, c.D)
        k = proj(self.x, "k").view(B, R, c.Hkv, c.D)
        v = proj(self.x, "v").view(B, R, c.Hkv, c.D)
        isd.attention_step(q, k, v, self.k_cache, self.v_cache, self.page_table, self.ctx_lens,
                           self.max_ctx, out=self.att_out)
        h = self.x + proj(self.att_out.view(self.M, c.Hq * c.D), "o")
        a = torch.nn.functional.silu(proj(h, "gate")) * proj(h, "up")
        return h + proj(a, "down")
