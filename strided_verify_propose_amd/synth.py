"""Seeded synthetic inputs for one ISD decode step.

This module is the only code shared by the HIP path's callers (tests, bench) and the
oracle's tests.  It holds none of the method's arithmetic: it draws random arrays,
rounds them to their stored dtype, builds page tables, and permutes cache pages into
the tile layout the attention kernel reads.  Draft tokens are drawn with the
Gumbel-max trick (argmax of logits plus Gumbel noise), which samples softmax(logits)
exactly without normalising anything.

Workload shapes follow the pages' model family: Qwen3-8B / Qwen3-32B attention shapes
(「首次超越 AR 模型」 "模型生態與安裝", 「I-DLM – introspektive Diffusion Language Models」 "Model Zoo"), stride N=4 giving 2N-1 = 7 query rows
(「首次超越 AR 模型」 "為什麼 I-DLM 能在高並發下保持高效"), concurrency 64 (「首次超越 AR 模型」 "吞吐量與並發性能"),
bf16 (「首次超越 AR 模型」 "快速開始").  Distributions are synthetic stand-ins for real prompts.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

PAGE = 16

_STREAMS = ("ctx", "pageperm", "q", "kcache", "vcache", "knew", "vnew", "anchor",
            "noise", "drafts", "uniforms", "x", "w", "a", "b", "spare")


def streams(seed: int) -> dict:
    """One independent PCG64 generator per named input, spawned in a fixed order."""
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {n: np.random.Generator(np.random.PCG64(c)) for n, c in zip(_STREAMS, children)}


# ----------------------------------------------------------------------------- dtypes
def bf16_rne(x) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even. Inputs are finite."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return (((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF).astype(np.uint16)


def bf16_bits_to_f32(u16) -> np.ndarray:
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def store(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float32 array to the stored dtype: 'f32' -> float32, 'bf16' -> uint16 bits."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_rne(x32)
    raise ValueError(dtype)


def normal(g: np.random.Generator, shape, sd: float) -> np.ndarray:
    out = g.standard_normal(size=shape, dtype=np.float32)
    if sd != 1.0:
        out *= np.float32(sd)
    return out


# ----------------------------------------------------------------------------- configs
@dataclass
class StepConfig:
    """Attention + verification workload of one ISD step."""
    name: str
    dtype: str          # 'f32' or 'bf16'
    B: int              # concurrency (requests)
    N: int              # stride; 2N-1 query rows per request
    Hq: int
    Hkv: int
    D: int
    V: int
    ctx: tuple          # ('fixed', L) or ('uniform', lo, hi) inclusive
    anchor_sd: float
    noise_sd: float
    seed: int
    argmax_drafts: bool = False   # True: drafts are argmax ids and no draft logits are passed

    @property
    def R(self) -> int:
        return 2 * self.N - 1


@dataclass
class ProjConfig:
    """Gated-LoRA projection workload (R-ISD)."""
    name: str
    B: int
    N: int
    K: int
    Nout: int
    r: int
    x_sd: float
    w_sd: float
    seed: int
    gate_pattern: tuple = field(default=(0, 0, 0, 1, 1, 1, 1))

    @property
    def M(self) -> int:
        return self.B * (2 * self.N - 1)


TINY = StepConfig("tiny_fp32", "f32", B=1, N=2, Hq=4, Hkv=1, D=64, V=1024, ctx=("fixed", 128),
                  anchor_sd=2.0, noise_sd=0.5, seed=1000)
QWEN3_8B = StepConfig("qwen3_8b_b64_n4", "bf16", B=64, N=4, Hq=32, Hkv=8, D=128, V=151936,
                      ctx=("uniform", 512, 4096), anchor_sd=3.0, noise_sd=0.3, seed=1001)
QWEN3_32B = StepConfig("qwen3_32b_b64_n4", "bf16", B=64, N=4, Hq=64, Hkv=8, D=128, V=151936,
                       ctx=("uniform", 2048, 8192), anchor_sd=3.0, noise_sd=0.3, seed=1003)
PROJ = ProjConfig("rlora_448x4096x4096_r128", B=64, N=4, K=4096, Nout=4096, r=128,
                  x_sd=1.0, w_sd=0.02, seed=1004)


# Proposal noise sd of the sweep for mean acceptance 0.5 and 0.9 (anchors N(0, 3),
# vocabulary 151936), bisected on the oracle by tests/golden/sweep_sigma.py.
SWEEP_SIGMA = {0.5: 1.367109, 0.9: 0.255684}
SWEEP_B = (1, 4, 16, 64)


def sweep_index(N: int, B: int, p: float) -> int:
    """Sweep point index, lexicographic in (N, B, p): N in {2,3,4}, B in SWEEP_B, p in {0.5, 0.9}."""
    return ((N - 2) * len(SWEEP_B) + SWEEP_B.index(B)) * 2 + (0 if p == 0.5 else 1)


def sweep_point(N: int, B: int, p: float) -> StepConfig:
    """The sweep point (N, B, p) with its calibrated noise and seed 1200 + index."""
    return sweep_config(N, B, SWEEP_SIGMA[p], sweep_index(N, B, p))


def sweep_config(N: int, B: int, noise_sd: float, index: int) -> StepConfig:
    """Stride/concurrency sweep point on the Qwen3-8B shapes at fixed context 2048."""
    return StepConfig(f"sweep_n{N}_b{B}", "bf16", B=B, N=N, Hq=32, Hkv=8, D=128, V=151936,
                      ctx=("fixed", 2048), anchor_sd=3.0, noise_sd=noise_sd, seed=1200 + index)


# ----------------------------------------------------------------------------- attention
def context_lengths(cfg: StepConfig, g: np.random.Generator) -> np.ndarray:
    if cfg.ctx[0] == "fixed":
        return np.full(cfg.B, cfg.ctx[1], dtype=np.int32)
    lo, hi = cfg.ctx[1], cfg.ctx[2]
    return g.integers(lo, hi + 1, size=cfg.B).astype(np.int32)


def k_tile_layout(k_logical: np.ndarray) -> np.ndarray:
    """[P, H, 16, D] -> [P, H, D/8, 16, 8]: per page and head, blocks of 8 dims, tokens inside."""
    P, H, T, D = k_logical.shape
    return np.ascontiguousarray(k_logical.reshape(P, H, T, D // 8, 8).transpose(0, 1, 3, 2, 4))


def k_logical_layout(k_tiles: np.ndarray, D: int) -> np.ndarray:
    P, H = k_tiles.shape[:2]
    t = k_tiles.reshape(P, H, D // 8, PAGE, 8)
    return np.ascontiguousarray(t.transpose(0, 1, 3, 2, 4).reshape(P, H, PAGE, D))


def v_tile_layout(v_logical: np.ndarray) -> np.ndarray:
    """[P, H, 16, D] -> [P, H, D/16, 4, 16, 4]: (dim block n, token quad g, dim d16, token tt)
    with token = 4g + tt and dim = 16n + d16."""
    P, H, T, D = v_logical.shape
    v = v_logical.reshape(P, H, 4, 4, D // 16, 16)          # (P,H,g,tt,n,d16)
    return np.ascontiguousarray(v.transpose(0, 1, 4, 2, 5, 3))


def v_logical_layout(v_tiles: np.ndarray, D: int) -> np.ndarray:
    P, H = v_tiles.shape[:2]
    v = v_tiles.reshape(P, H, D // 16, 4, 16, 4)            # (P,H,n,g,d16,tt)
    return np.ascontiguousarray(v.transpose(0, 1, 3, 5, 2, 4).reshape(P, H, PAGE, D))


@dataclass
class AttentionInputs:
    cfg: StepConfig
    ctx_lens: np.ndarray        # [B] int32, tokens cached before the block
    page_table: np.ndarray      # [B, max_pages] int32
    num_pages: int
    q: np.ndarray               # [B, R, Hq, D] stored dtype
    k_new: np.ndarray           # [B, R, Hkv, D]
    v_new: np.ndarray
    k_pages: np.ndarray         # [num_pages, Hkv, 16, D] stored dtype, logical layout
    v_pages: np.ndarray
    scale: float

    @property
    def max_pages(self) -> int:
        return self.page_table.shape[1]


def attention_inputs(cfg: StepConfig, seed: int | None = None, ctx_lens=None) -> AttentionInputs:
    """Paged cache holding ctx_lens[b] tokens per request plus room for the 2N-1 block rows.

    Physical page ids are a seeded permutation assigned in request order; slots past
    ctx_lens[b] start at zero."""
    g = streams(cfg.seed if seed is None else seed)
    B, R, Hq, Hkv, D = cfg.B, cfg.R, cfg.Hq, cfg.Hkv, cfg.D
    L = context_lengths(cfg, g["ctx"]) if ctx_lens is None else np.asarray(ctx_lens, np.int32)
    n_pages = (L.astype(np.int64) + R + PAGE - 1) // PAGE
    total = int(n_pages.sum())
    perm = g["pageperm"].permutation(total).astype(np.int32)
    max_pages = int(n_pages.max())
    page_table = np.zeros((B, max_pages), np.int32)
    off = 0
    for b in range(B):
        page_table[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]
    dt = cfg.dtype
    k_pages = np.zeros((total, Hkv, PAGE, D), np.float32 if dt == "f32" else np.uint16)
    v_pages = np.zeros_like(k_pages)
    for b in range(B):
        Lb = int(L[b])
        if Lb == 0:
            continue
        kv = normal(g["kcache"], (Lb, Hkv, D), 1.0)
        vv = normal(g["vcache"], (Lb, Hkv, D), 1.0)
        pages = page_table[b, :(Lb + PAGE - 1) // PAGE]
        kpad = np.zeros((len(pages) * PAGE, Hkv, D), np.float32)
        vpad = np.zeros_like(kpad)
        kpad[:Lb] = kv
        vpad[:Lb] = vv
        k_pages[pages] = store(kpad, dt).reshape(len(pages), PAGE, Hkv, D).transpose(0, 2, 1, 3)
        v_pages[pages] = store(vpad, dt).reshape(len(pages), PAGE, Hkv, D).transpose(0, 2, 1, 3)
    q = store(normal(g["q"], (B, R, Hq, D), 1.0), dt)
    k_new = store(normal(g["knew"], (B, R, Hkv, D), 1.0), dt)
    v_new = store(normal(g["vnew"], (B, R, Hkv, D), 1.0), dt)
    return AttentionInputs(cfg, L, page_table, total, q, k_new, v_new, k_pages, v_pages,
                           1.0 / math.sqrt(D))


# ----------------------------------------------------------------------------- verification
@dataclass
class VerifyInputs:
    cfg: StepConfig
    logits: np.ndarray          # [B, 2N-1, V]: verify rows 0..N-2, proposal rows N-1..2N-2
    draft_logits: np.ndarray | None   # [B, N-1, V], the rows the drafts were drawn from
    draft_ids: np.ndarray       # [B, N-1] int32
    uniforms: np.ndarray        # [B, 2N-1] float32, k / 2^24


def gumbel_argmax(rows32: np.ndarray, g: np.random.Generator) -> np.ndarray:
    """One draw per row from softmax(row) by the Gumbel-max trick (float64)."""
    u = np.maximum(g.random(size=rows32.shape), 1e-300)   # (0, 1)
    gum = -np.log(-np.log(u))                              # standard Gumbel
    return np.argmax(rows32.astype(np.float64) + gum, axis=-1).astype(np.int32)


def uniforms24(g: np.random.Generator, shape) -> np.ndarray:
    """k / 2^24 with k uniform in [0, 2^24): exact in float32 and float64, never 1.0."""
    return (g.integers(0, 1 << 24, size=shape) / float(1 << 24)).astype(np.float32)


def verify_inputs(cfg: StepConfig, seed: int | None = None) -> VerifyInputs:
    """Anchor logits ~ N(0, anchor_sd); proposal logits = anchor + N(0, noise_sd).

    Verify row i holds the anchor of draft i; the draft row i (previous step's proposal)
    is that anchor plus noise, and draft i is drawn from it.  The current step's proposal
    rows are fresh anchors plus fresh noise.  With argmax_drafts the draft is the argmax
    of its proposal row and no draft logits are passed."""
    g = streams(cfg.seed if seed is None else seed)
    B, N, R, V = cfg.B, cfg.N, cfg.R, cfg.V
    anchor = normal(g["anchor"], (B, R, V), cfg.anchor_sd)
    noise = normal(g["noise"], (B, R, V), cfg.noise_sd)
    prop = anchor + noise
    logits32 = np.empty((B, R, V), np.float32)
    logits32[:, :N - 1] = anchor[:, :N - 1]
    logits32[:, N - 1:] = prop[:, N - 1:]
    logits = store(logits32, cfg.dtype)
    draft_stored = store(prop[:, :N - 1], cfg.dtype)
    draft_vals = draft_stored.astype(np.float32) if cfg.dtype == "f32" else bf16_bits_to_f32(draft_stored)
    if cfg.argmax_drafts:
        draft_ids = np.argmax(draft_vals, axis=-1).astype(np.int32)
        draft_logits = None
    else:
        draft_ids = gumbel_argmax(draft_vals, g["drafts"])
        draft_logits = draft_stored
    u = uniforms24(g["uniforms"], (B, R))
    return VerifyInputs(cfg, logits, draft_logits, draft_ids, u)


# ----------------------------------------------------------------------------- projection
@dataclass
class ProjInputs:
    cfg: ProjConfig
    x: np.ndarray      # [M, K] bf16 bits
    w: np.ndarray      # [Nout, K] bf16 bits (W^T: each output column's weights contiguous)
    a: np.ndarray      # [r, K]   (A^T)
    b: np.ndarray      # [Nout, r] (B^T)
    gate: np.ndarray   # [M] uint8


def proj_inputs(cfg: ProjConfig, seed: int | None = None, M: int | None = None) -> ProjInputs:
    g = streams(cfg.seed if seed is None else seed)
    M = cfg.M if M is None else M
    x = bf16_rne(normal(g["x"], (M, cfg.K), cfg.x_sd))
    w = bf16_rne(normal(g["w"], (cfg.Nout, cfg.K), cfg.w_sd))
    a = bf16_rne(normal(g["a"], (cfg.r, cfg.K), cfg.w_sd))
    b = bf16_rne(normal(g["b"], (cfg.Nout, cfg.r), cfg.w_sd))
    pat = np.asarray(cfg.gate_pattern, np.uint8)
    gate = np.resize(pat, M).astype(np.uint8)
    return ProjInputs(cfg, x, w, a, b, gate)


# ----------------------------------------------------------------------------- LM head
@dataclass
class LmHeadConfig:
    """LM head in front of verification: hidden [B (2N-1), Dm] times w_lm [V, Dm]^T.

    grid=True draws every hidden value as k/4 (k integer in [-4, 4]) and every weight as
    k/32 (k in [-2, 2]): all products and partial sums are multiples of 2^-7 below 2^15
    in magnitude for Dm <= 4096, so any float32 summation order gives the exact product
    and the stored bf16 logits are unique.  grid=False draws N(0, h_sd) and N(0, w_sd)."""
    name: str
    B: int
    N: int
    Dm: int
    V: int
    h_sd: float
    w_sd: float
    draft_sd: float
    grid: bool
    seed: int

    @property
    def R(self) -> int:
        return 2 * self.N - 1

    @property
    def M(self) -> int:
        return self.B * self.R


# Qwen3-8B's and Qwen3-32B's hidden sizes and vocabulary; weights scaled so the logits
# have sd ~3 like the verification workload's anchors.
LM_HEAD_8B = LmHeadConfig("lm_head_qwen3_8b_b64_n4", B=64, N=4, Dm=4096, V=151936,
                          h_sd=1.0, w_sd=3.0 / 64.0, draft_sd=3.0, grid=False, seed=1005)
LM_HEAD_32B = LmHeadConfig("lm_head_qwen3_32b_b64_n4", B=64, N=4, Dm=5120, V=151936,
                           h_sd=1.0, w_sd=3.0 / 5120 ** 0.5, draft_sd=3.0, grid=False, seed=1006)


@dataclass
class LmHeadInputs:
    cfg: LmHeadConfig
    hidden: np.ndarray          # [M, Dm] bf16 bits, request-major (row b R + r)
    w_lm: np.ndarray            # [V, Dm] bf16 bits
    draft_logits: np.ndarray | None   # [B, N-1, V] bf16 bits (previous step's proposal rows)
    draft_ids: np.ndarray       # [B, N-1] int32
    uniforms: np.ndarray        # [B, 2N-1] float32


def _grid(g: np.random.Generator, shape, kmax: int, scale: float) -> np.ndarray:
    return (g.integers(-kmax, kmax + 1, size=shape).astype(np.float32) * np.float32(scale))


def lm_head_inputs(cfg: LmHeadConfig, seed: int | None = None, argmax_drafts: bool = False) -> LmHeadInputs:
    """Hidden states, output embedding, and draft rows drawn independently of the
    product (N(0, draft_sd)); drafts are Gumbel draws from those rows, or their argmax."""
    g = streams(cfg.seed if seed is None else seed)
    B, N, R, V = cfg.B, cfg.N, cfg.R, cfg.V
    if cfg.grid:
        hidden = bf16_rne(_grid(g["x"], (cfg.M, cfg.Dm), 4, 0.25))
    else:
        hidden = bf16_rne(normal(g["x"], (cfg.M, cfg.Dm), cfg.h_sd))
    w_lm = np.empty((V, cfg.Dm), np.uint16)
    step = 8192                                          # bounded temporaries, in row order
    for v0 in range(0, V, step):
        shape = (min(step, V - v0), cfg.Dm)
        rows = _grid(g["w"], shape, 2, 1.0 / 32.0) if cfg.grid else normal(g["w"], shape, cfg.w_sd)
        w_lm[v0:v0 + step] = bf16_rne(rows)
    draft_stored = bf16_rne(normal(g["anchor"], (B, N - 1, V), cfg.draft_sd))
    draft_vals = bf16_bits_to_f32(draft_stored)
    if argmax_drafts:
        draft_ids = np.argmax(draft_vals, axis=-1).astype(np.int32)
        draft_logits = None
    else:
        draft_ids = gumbel_argmax(draft_vals, g["drafts"])
        draft_logits = draft_stored
    u = uniforms24(g["uniforms"], (B, R))
    return LmHeadInputs(cfg, hidden, w_lm, draft_logits, draft_ids, u)


# ----------------------------------------------------------------------------- decoder layer
@dataclass
class LayerInputsConfig:
    """An R-ISD decoder layer of a Qwen3-shaped model over one strided block: seven
    linears (q, k, v, o, gate, up, down) each with a rank-r delta, and the block's
    attention over a paged cache.  Qwen3-8B: hidden 4096, 32 query heads, 8 KV heads,
    head dim 128, intermediate 12288."""
    name: str
    B: int
    N: int
    hidden: int
    Hq: int
    Hkv: int
    D: int
    inter: int
    r: int
    ctx: tuple          # ('fixed', L) or ('uniform', lo, hi) inclusive
    seed: int

    @property
    def R(self) -> int:
        return 2 * self.N - 1

    @property
    def M(self) -> int:
        return self.B * self.R

    def shapes(self) -> dict:
        """(K, Nout) of each linear."""
        H, I = self.hidden, self.inter
        return dict(q=(H, self.Hq * self.D), k=(H, self.Hkv * self.D), v=(H, self.Hkv * self.D),
                    o=(self.Hq * self.D, H), gate=(H, I), up=(H, I), down=(I, H))


@dataclass
class LayerInputs:
    cfg: LayerInputsConfig
    x: np.ndarray               # [M, hidden] bf16 bits, request-major
    weights: dict               # name -> (w [Nout, K], a [r, K], b [Nout, r]) bf16 bits
    gate: np.ndarray            # [M] uint8: 0 on the N-1 verify rows, 1 on the others
    attn: AttentionInputs       # cache, page table, context lengths (its q/k/v unused)


def layer_inputs(cfg: LayerInputsConfig) -> LayerInputs:
    """x ~ N(0, 1); w, a ~ N(0, 1/K) (sd 1/sqrt(K)); b ~ N(0, 0.02); cached K/V ~ N(0, 1)
    in seeded pages (as attention_inputs).  The N-1 verify rows of each block are
    ungated, the bonus row and the [MASK] rows gated."""
    g = streams(cfg.seed)
    step = StepConfig(cfg.name, "bf16", B=cfg.B, N=cfg.N, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D, V=2,
                      ctx=cfg.ctx, anchor_sd=1.0, noise_sd=1.0, seed=cfg.seed + 1)
    attn = attention_inputs(step)
    x = bf16_rne(normal(g["x"], (cfg.M, cfg.hidden), 1.0))
    weights = {}
    for name, (K, Nout) in cfg.shapes().items():
        sd = 1.0 / math.sqrt(K)
        w = bf16_rne(normal(g["w"], (Nout, K), sd))
        a = bf16_rne(normal(g["a"], (cfg.r, K), sd))
        b = bf16_rne(normal(g["b"], (Nout, cfg.r), 0.02))
        weights[name] = (w, a, b)
    gate = np.resize(np.array([0] * (cfg.N - 1) + [1] * cfg.N, np.uint8), cfg.M)
    return LayerInputs(cfg, x, weights, gate, attn)
