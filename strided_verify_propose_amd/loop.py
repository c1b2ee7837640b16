"""Closed-loop ISD decoding on the device: every step's outputs become the next step's
inputs without leaving the GPU, and a whole step can be captured as a HIP graph.

State per request: the context length (KV rollback is simply not advancing it past the
kept tokens), the next step's draft ids (-1: cold) and, for sampled drafts, the rows they
were drawn from (the previous step's [MASK] rows).  One step:
  1. the synthetic model writes this step's rows (no trained weights are available):
     a hot request's verify row i is its draft row i plus N(0, sigma) noise, so that
     acceptance is in the regime the noise sets; every other row is fresh N(0, anchor_sd);
     the block's q, k, v rows are fresh N(0, 1)
  2. the hot path: the R-ISD projection of the block's rows, attention (appending the
     block's K/V), verification (cold requests: one exact token from row 0)
  3. isd_commit: context lengths grow by the tokens kept, the next drafts are the
     samples of the [MASK] rows when the request stays hot
  4. the [MASK] rows are kept as the next step's draft rows, and so are the softmax
     statistics verification computed for them (isd_verify_carry): the next step's
     verification reads them instead of reducing its draft rows again
Only step 1 and the bookkeeping of 4 are torch operations; 2 and 3 are the library's
kernels.  The synthetic model costs device time of its own, reported apart from the hot
path.  (The tokens are never embedded: the model ignores them, as its rows are synthetic.)
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import isd

PAGE = 16


@dataclass
class LoopConfig:
    B: int = 64
    N: int = 4
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    V: int = 151936
    ctx0: tuple = (512, 4096)     # initial context lengths ~ U{lo..hi}
    steps: int = 200              # capacity: the cache holds ctx0 + steps * N tokens
    anchor_sd: float = 3.0
    sigma: float = 0.3            # draft row -> verify row noise (acceptance near 0.9)
    proj: tuple = (4096, 4096, 128)   # K, Nout, r of the R-ISD projection (None: skip)
    carry_q_stats: bool = True    # hand the [MASK] rows' statistics on to the next step
    seed: int = 1500


class ClosedLoop:
    def __init__(self, cfg: LoopConfig, device="cuda"):
        self.cfg = c = cfg
        dev = self.dev = torch.device(device)
        g = self.gen = torch.Generator(device=dev)
        g.manual_seed(c.seed)
        B, N, R = c.B, c.N, 2 * c.N - 1
        self.R = R
        bf = torch.bfloat16
        lo, hi = c.ctx0
        self.ctx_lens = torch.randint(lo, hi + 1, (B,), generator=g, device=dev, dtype=torch.int32)
        self.max_ctx = hi + c.steps * N
        self.pages = (self.max_ctx + R + PAGE - 1) // PAGE
        perm = torch.randperm(B * self.pages, generator=g, device=dev).to(torch.int32)
        self.page_table = perm.view(B, self.pages).contiguous()
        P = B * self.pages
        self.k_cache = torch.randn((P, c.Hkv, c.D // 8, PAGE, 8), generator=g, device=dev).to(bf)
        self.v_cache = torch.randn((P, c.Hkv, c.D // 16, 4, PAGE, 4), generator=g, device=dev).to(bf)
        self.q = torch.empty((B, R, c.Hq, c.D), dtype=bf, device=dev)
        self.k_new = torch.empty((B, R, c.Hkv, c.D), dtype=bf, device=dev)
        self.v_new = torch.empty_like(self.k_new)
        self.att_out = torch.empty_like(self.q)
        self.logits = torch.empty((B, R, c.V), dtype=bf, device=dev)
        self.draft_rows = torch.zeros((B, max(N - 1, 1), c.V), dtype=bf, device=dev)
        self.draft_ids = torch.full((B, N - 1), -1, dtype=torch.int32, device=dev)  # all cold
        self.uniforms = torch.empty((B, R), dtype=torch.float32, device=dev)
        i32 = dict(dtype=torch.int32, device=dev)
        self.out = dict(n_accept=torch.empty(B, **i32), accept=torch.empty((B, N - 1), dtype=torch.uint8, device=dev),
                        next_token=torch.empty(B, **i32), argmax_ids=torch.empty((B, N), **i32),
                        sampled_ids=torch.empty((B, N), **i32))
        self.tokens = torch.empty((B, N), **i32)
        self.counts = torch.empty(B, **i32)
        # running totals over steps, per request
        self.kept = torch.zeros(B, dtype=torch.int64, device=dev)
        self.accepted = torch.zeros(B, dtype=torch.int64, device=dev)
        self.evaluated = torch.zeros(B, dtype=torch.int64, device=dev)
        self.hot_steps = torch.zeros(B, dtype=torch.int64, device=dev)
        self.steps_done = 0
        self.packed = None
        if c.proj is not None:
            K, Nout, r = c.proj
            w = (torch.randn((Nout, K), generator=g, device=dev) * 0.02).to(bf)
            a = (torch.randn((r, K), generator=g, device=dev) * 0.02).to(bf)
            b = (torch.randn((Nout, r), generator=g, device=dev) * 0.02).to(bf)
            self.packed = isd.pack_proj_weights(w, a, b)
            self.x = torch.randn((B * R, K), generator=g, device=dev).to(bf)
            self.y = torch.empty((B * R, Nout), dtype=bf, device=dev)
            self.gate = torch.tensor(([0] * (N - 1) + [1] * N) * B, dtype=torch.uint8, device=dev)
        self.hot = torch.zeros(B, dtype=torch.bool, device=dev)
        # statistics of this step's rows N..2N-2 for the next step, and the previous step's
        # for this step's draft rows (zeros before the first step, whose requests are all cold)
        self.q_next = self.q_prev = None
        if N > 1 and c.carry_q_stats:
            nb = isd.verify_carry_bytes(B, N, c.V)
            self.q_next = torch.zeros(nb, dtype=torch.uint8, device=dev)
            self.q_prev = torch.zeros(nb, dtype=torch.uint8, device=dev)

    # ---------------------------------------------------------------- one step
    def model(self):
        """Synthetic rows for this step (torch, on the device)."""
        c, g, N = self.cfg, self.gen, self.cfg.N
        for t in (self.q, self.k_new, self.v_new):
            t.copy_(torch.randn(t.shape, generator=g, device=self.dev))
        self.logits.copy_(torch.randn(self.logits.shape, generator=g, device=self.dev) * c.anchor_sd)
        if N > 1:
            self.hot.copy_(self.draft_ids[:, 0] >= 0)
            noisy = self.draft_rows.float() + torch.randn(self.draft_rows.shape, generator=g, device=self.dev) * c.sigma
            self.logits[:, :N - 1].copy_(torch.where(self.hot[:, None, None], noisy, self.logits[:, :N - 1].float()))
        self.uniforms.copy_(torch.randint(0, 1 << 24, self.uniforms.shape, generator=g, device=self.dev)
                            .to(torch.float32) / float(1 << 24))

    def hot_path(self, ev=None):
        """The library's kernels for one step; `ev`: five events around the calls
        (projection, attention, verification, commit)."""
        N = self.cfg.N
        if ev is not None:
            ev[0].record()
        if self.packed is not None:
            isd.gated_lora_proj_packed(self.x, self.packed, self.gate, out=self.y)
        if ev is not None:
            ev[1].record()
        isd.attention_step(self.q, self.k_new, self.v_new, self.k_cache, self.v_cache, self.page_table,
                           self.ctx_lens, self.max_ctx, out=self.att_out)
        if ev is not None:
            ev[2].record()
        isd.verify(self.logits, self.draft_rows if N > 1 else None, self.draft_ids, self.uniforms,
                   with_diagnostics=False, out=self.out, q_stats_prev=self.q_prev, q_stats_next=self.q_next)
        if ev is not None:
            ev[3].record()
        isd.commit(self.out["n_accept"], self.out["next_token"], self.out["sampled_ids"], self.draft_ids,
                   self.ctx_lens, self.tokens, self.counts)
        if ev is not None:
            ev[4].record()
        self.tally()

    def tally(self):
        """Running totals for the statistics (torch; this step's hot flags were taken
        before the commit replaced the drafts)."""
        N = self.cfg.N
        self.kept.add_(self.counts.to(torch.int64))
        if N > 1:
            n = self.out["n_accept"].to(torch.int64)
            hot = self.hot
            self.accepted.add_(torch.where(hot, n, 0))
            self.evaluated.add_(torch.where(hot, n + (n < N - 1).to(torch.int64), 0))
            self.hot_steps.add_(hot.to(torch.int64))

    def keep_draft_rows(self):
        N = self.cfg.N
        if N > 1:
            self.draft_rows.copy_(self.logits[:, N:])
        if self.q_next is not None:
            self.q_prev.copy_(self.q_next)

    def step(self, ev=None):
        self.model()
        self.hot_path(ev)
        self.keep_draft_rows()

    # ---------------------------------------------------------------- summary
    def stats(self, steps):
        """Tokens per forward measured from the kept tokens, the acceptance rate, and the
        closed form of the hot/cold chain at that rate."""
        N = self.cfg.N
        kept = self.kept.double().cpu()
        tpf = float(kept.sum()) / (self.cfg.B * steps)
        acc, ev = float(self.accepted.sum()), float(self.evaluated.sum())
        p_hat = acc / ev if ev > 0 else 1.0
        closed = 1.0 if N == 1 else (2 + sum(p_hat ** k for k in range(1, N - 1))) / (2 - p_hat ** (N - 1))
        per_req = kept / steps
        se = float(per_req.std()) / math.sqrt(self.cfg.B)
        return dict(tpf_meas=tpf, p_hat=p_hat, tpf_closed_form_at_p_hat=closed, tpf_se=se)
