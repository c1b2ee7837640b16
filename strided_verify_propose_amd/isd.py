"""Python binding of libisd.so (the C ABI in include/isd.h).

Argument marshalling only: tensors are checked for device, dtype, shape and layout,
their data pointers and the current HIP stream are passed through ctypes, and every
step of the computation runs in the library's kernels.  PyTorch provides device
memory and streams.  There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libisd.so")
_lib = None

ISD_F32, ISD_BF16 = 0, 1
PAGE_SIZE = 16
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
          3: "workspace too small", 4: "HIP error"}

EXPORTS = ("isd_abi_version", "isd_status_string", "isd_last_error",
           "isd_attention_workspace_bytes", "isd_attention_step",
           "isd_pack_kv_pages", "isd_unpack_kv_pages", "isd_kv_read_sweep",
           "isd_verify_workspace_bytes", "isd_verify", "isd_verify_noalloc",
           "isd_verify_carry_bytes", "isd_verify_carry",
           "isd_gated_lora_workspace_bytes", "isd_gated_lora_proj",
           "isd_proj_packed_bytes", "isd_pack_proj_weights", "isd_pack_proj_weights_kn",
           "isd_gated_lora_proj_packed",
           "isd_commit", "isd_lm_head", "isd_lm_head_verify_workspace_bytes",
           "isd_lm_head_verify")


class IsdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Open the library (after torch, so it binds to the HIP runtime torch loaded)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built: run `python -m strided_verify_propose_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.isd_abi_version.restype = i32
    L.isd_status_string.restype = ctypes.c_char_p
    L.isd_status_string.argtypes = [i32]
    L.isd_last_error.restype = ctypes.c_char_p
    L.isd_attention_workspace_bytes.restype = sz
    L.isd_attention_workspace_bytes.argtypes = [i32] * 6
    L.isd_attention_step.restype = i32
    L.isd_attention_step.argtypes = [i32] + [vp] * 8 + [i32] * 9 + [f32, vp, sz, vp]
    L.isd_pack_kv_pages.restype = i32
    L.isd_pack_kv_pages.argtypes = [i32] + [vp] * 4 + [i32] * 3 + [vp]
    L.isd_unpack_kv_pages.restype = i32
    L.isd_unpack_kv_pages.argtypes = [i32] + [vp] * 4 + [i32] * 3 + [vp]
    L.isd_kv_read_sweep.restype = i32
    L.isd_kv_read_sweep.argtypes = [vp] * 4 + [i32] * 6 + [vp, vp]
    L.isd_verify_workspace_bytes.restype = sz
    L.isd_verify_workspace_bytes.argtypes = [i32] * 3
    L.isd_verify.restype = i32
    L.isd_verify.argtypes = [i32] + [vp] * 4 + [i32] * 3 + [f32] + [vp] * 8 + [vp, sz, vp]
    L.isd_verify_noalloc.restype = i32
    L.isd_verify_noalloc.argtypes = [i32] + [vp] * 4 + [i32] * 3 + [f32] + [vp] * 8 + [vp]
    L.isd_verify_carry_bytes.restype = sz
    L.isd_verify_carry_bytes.argtypes = [i32] * 3
    L.isd_verify_carry.restype = i32
    L.isd_verify_carry.argtypes = [i32] + [vp] * 4 + [i32] * 3 + [f32] + [vp] * 10 + [vp, sz, vp]
    L.isd_gated_lora_workspace_bytes.restype = sz
    L.isd_gated_lora_workspace_bytes.argtypes = [i32] * 4
    L.isd_gated_lora_proj.restype = i32
    L.isd_gated_lora_proj.argtypes = [vp] * 6 + [i32] * 4 + [vp, sz, vp]
    L.isd_proj_packed_bytes.restype = sz
    L.isd_proj_packed_bytes.argtypes = [i32] * 3
    L.isd_pack_proj_weights.restype = i32
    L.isd_pack_proj_weights.argtypes = [vp] * 4 + [i32] * 3 + [vp]
    L.isd_pack_proj_weights_kn.restype = i32
    L.isd_pack_proj_weights_kn.argtypes = [vp] * 4 + [i32] * 3 + [vp]
    L.isd_gated_lora_proj_packed.restype = i32
    L.isd_gated_lora_proj_packed.argtypes = [vp] * 4 + [i32] * 4 + [vp, sz, vp]
    L.isd_commit.restype = ctypes.c_int
    L.isd_commit.argtypes = [vp] * 7 + [i32] * 2 + [vp]
    L.isd_lm_head.restype = i32
    L.isd_lm_head.argtypes = [vp] * 3 + [i32] * 3 + [vp]
    L.isd_lm_head_verify_workspace_bytes.restype = sz
    L.isd_lm_head_verify_workspace_bytes.argtypes = [i32] * 3
    L.isd_lm_head_verify.restype = i32
    L.isd_lm_head_verify.argtypes = [vp] * 6 + [i32] * 4 + [f32] + [vp] * 8 + [vp, sz, vp]
    if L.isd_abi_version() != 1:
        raise RuntimeError("libisd.so ABI version mismatch")
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise IsdError(status, lib().isd_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must live on the GPU ({device})")


_ws_cache: dict = {}


def workspace(kind: str, nbytes: int, device, shape_key=()) -> torch.Tensor:
    """Device workspace, one per (entry point, device, current stream, shape arguments),
    kept for reuse: calls on different streams never share one, since calls that share a
    workspace must not overlap.  The library does not depend on its contents on entry."""
    stream = torch.cuda.current_stream(device).cuda_stream
    key = (kind, str(device), stream, tuple(shape_key))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def _dt(t):
    if t.dtype == torch.bfloat16:
        return ISD_BF16
    if t.dtype == torch.float32:
        return ISD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# ----------------------------------------------------------------------------- attention
def attention_step(q, k_new, v_new, k_cache, v_cache, page_table, ctx_lens, max_ctx_len: int,
                   out=None, scale: float | None = None, ws=None):
    """Strictly causal GQA attention of the 2N-1 block rows over the paged cache; appends the
    block's K/V rows to their slots.  q [B,R,Hq,D]; k_new, v_new [B,R,Hkv,D];
    k_cache [P,Hkv,D/8,16,8], v_cache [P,Hkv,D/16,4,16,4]; page_table [B,maxp] int32;
    ctx_lens [B] int32 (device); max_ctx_len: host bound on ctx_lens."""
    B, R, Hq, D = q.shape
    if R % 2 == 0:
        raise ValueError("q must hold 2N-1 rows per request")
    N = (R + 1) // 2
    Hkv = k_new.shape[2]
    dev = q.device
    _need(q, "q", q.dtype, device=dev)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t, name, q.dtype, (B, R, Hkv, D), dev)
    P = k_cache.shape[0]
    _need(k_cache, "k_cache", q.dtype, (P, Hkv, D // 8, PAGE_SIZE, 8), dev)
    _need(v_cache, "v_cache", q.dtype, (P, Hkv, D // 16, 4, PAGE_SIZE, 4), dev)
    _need(page_table, "page_table", torch.int32, device=dev)
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError(f"page_table: shape {tuple(page_table.shape)}, expected ({B}, max_pages)")
    _need(ctx_lens, "ctx_lens", torch.int32, (B,), dev)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, q.shape, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    L = lib()
    nbytes = L.isd_attention_workspace_bytes(B, N, Hq, Hkv, D, int(max_ctx_len))
    w = ws if ws is not None else workspace("attention", nbytes, dev, (B, N, Hq, Hkv, D, int(max_ctx_len)))
    _check(L.isd_attention_step(_dt(q), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache),
                                _ptr(v_cache), _ptr(page_table), _ptr(ctx_lens), _ptr(out),
                                B, N, Hq, Hkv, D, PAGE_SIZE, page_table.shape[1], P,
                                int(max_ctx_len), float(scale), _ptr(w), w.numel(), _stream(dev)))
    return out


def pack_kv_pages(k_pages, v_pages, k_cache=None, v_cache=None):
    """Logical pages k_pages, v_pages [P, Hkv, 16, D] -> the tile layout attention_step reads
    (k_cache [P, Hkv, D/8, 16, 8], v_cache [P, Hkv, D/16, 4, 16, 4]).  Returns (k_cache, v_cache)."""
    P, Hkv, T, D = k_pages.shape
    dev = k_pages.device
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
        _need(t, name, k_pages.dtype, (P, Hkv, PAGE_SIZE, D), dev)
    if k_cache is None:
        k_cache = torch.empty((P, Hkv, D // 8, PAGE_SIZE, 8), dtype=k_pages.dtype, device=dev)
    if v_cache is None:
        v_cache = torch.empty((P, Hkv, D // 16, 4, PAGE_SIZE, 4), dtype=k_pages.dtype, device=dev)
    _need(k_cache, "k_cache", k_pages.dtype, (P, Hkv, D // 8, PAGE_SIZE, 8), dev)
    _need(v_cache, "v_cache", k_pages.dtype, (P, Hkv, D // 16, 4, PAGE_SIZE, 4), dev)
    _check(lib().isd_pack_kv_pages(_dt(k_pages), _ptr(k_pages), _ptr(v_pages), _ptr(k_cache), _ptr(v_cache),
                                   P, Hkv, D, _stream(dev)))
    return k_cache, v_cache


def unpack_kv_pages(k_cache, v_cache, k_pages=None, v_pages=None):
    """The tile layout back to logical pages [P, Hkv, 16, D].  Returns (k_pages, v_pages)."""
    P, Hkv = k_cache.shape[:2]
    D = k_cache.shape[2] * 8
    dev = k_cache.device
    _need(k_cache, "k_cache", k_cache.dtype, (P, Hkv, D // 8, PAGE_SIZE, 8), dev)
    _need(v_cache, "v_cache", k_cache.dtype, (P, Hkv, D // 16, 4, PAGE_SIZE, 4), dev)
    if k_pages is None:
        k_pages = torch.empty((P, Hkv, PAGE_SIZE, D), dtype=k_cache.dtype, device=dev)
    if v_pages is None:
        v_pages = torch.empty((P, Hkv, PAGE_SIZE, D), dtype=k_cache.dtype, device=dev)
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages)):
        _need(t, name, k_cache.dtype, (P, Hkv, PAGE_SIZE, D), dev)
    _check(lib().isd_unpack_kv_pages(_dt(k_cache), _ptr(k_cache), _ptr(v_cache), _ptr(k_pages), _ptr(v_pages),
                                     P, Hkv, D, _stream(dev)))
    return k_pages, v_pages


def kv_read_sweep(k_cache, v_cache, page_table, ctx_lens, max_ctx_len: int, checksum=None):
    """Read the cached K/V tiles an attention step reads for these requests, once each and
    evenly spread over the GPU, computing nothing from them: the rate reference for
    attention_step.  checksum (one uint32 word on the device, as an int32 tensor of shape
    [1]) is XORed with every 32-bit word read; a new one starts at zero.  Returns it."""
    P, Hkv = k_cache.shape[:2]
    D = k_cache.shape[2] * 8
    dev = k_cache.device
    _need(k_cache, "k_cache", torch.bfloat16, (P, Hkv, D // 8, PAGE_SIZE, 8), dev)
    _need(v_cache, "v_cache", torch.bfloat16, (P, Hkv, D // 16, 4, PAGE_SIZE, 4), dev)
    _need(page_table, "page_table", torch.int32, device=dev)
    if page_table.dim() != 2:
        raise ValueError(f"page_table: shape {tuple(page_table.shape)}, expected (B, max_pages)")
    B = page_table.shape[0]
    _need(ctx_lens, "ctx_lens", torch.int32, (B,), dev)
    if checksum is None:
        checksum = torch.zeros(1, dtype=torch.int32, device=dev)
    _need(checksum, "checksum", torch.int32, (1,), dev)
    _check(lib().isd_kv_read_sweep(_ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(ctx_lens), B, Hkv, D,
                                   page_table.shape[1], P, int(max_ctx_len), _ptr(checksum), _stream(dev)))
    return checksum


# ----------------------------------------------------------------------------- verification
def verify_carry_bytes(B: int, N: int, V: int) -> int:
    """Bytes of one buffer of statistics carried between steps (0 when N == 1)."""
    return lib().isd_verify_carry_bytes(B, N, V)


def verify(logits, draft_logits, draft_ids, uniforms, temperature: float = 1.0,
           with_diagnostics: bool = True, out: dict | None = None, q_stats_prev=None, q_stats_next=None):
    """Vocab-wide verification of one ISD step.  logits [B,2N-1,V]; draft_logits [B,N-1,V]
    or None (argmax drafts); draft_ids [B,N-1] int32; uniforms [B,2N-1] float32.
    Returns a dict of device tensors (n_accept, accept, next_token, argmax_ids,
    sampled_ids, and p_draft, q_draft, row_lse when with_diagnostics).
    q_stats_next / q_stats_prev (uint8 device tensors of verify_carry_bytes): this call's
    statistics of rows N..2N-2 for the next step, and the previous step's for this call's
    draft rows (isd_verify_carry; same outputs as without them)."""
    B, R, V = logits.shape
    if R % 2 == 0:
        raise ValueError("logits must hold 2N-1 rows per request")
    N = (R + 1) // 2
    dev = logits.device
    _need(logits, "logits", logits.dtype, device=dev)
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", logits.dtype, (B, N - 1, V), dev)
    _need(draft_ids, "draft_ids", torch.int32, (B, N - 1), dev)
    _need(uniforms, "uniforms", torch.float32, (B, R), dev)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(n_accept=torch.empty(B, **i32),
                   accept=torch.empty((B, N - 1), dtype=torch.uint8, device=dev),
                   next_token=torch.empty(B, **i32), argmax_ids=torch.empty((B, N), **i32),
                   sampled_ids=torch.empty((B, N), **i32))
        if with_diagnostics:
            f32 = dict(dtype=torch.float32, device=dev)
            out.update(p_draft=torch.empty((B, N - 1), **f32), q_draft=torch.empty((B, N - 1), **f32),
                       row_lse=torch.empty((B, R + N - 1), **f32))
    L = lib()
    nbytes = L.isd_verify_workspace_bytes(B, N, V)
    w = workspace("verify", nbytes, dev, (B, N, V))
    if q_stats_prev is None and q_stats_next is None:
        _check(L.isd_verify(_dt(logits), _ptr(logits), _ptr(draft_logits), _ptr(draft_ids),
                            _ptr(uniforms), B, N, V, float(temperature), _ptr(out["n_accept"]),
                            _ptr(out["accept"]), _ptr(out["next_token"]), _ptr(out["argmax_ids"]),
                            _ptr(out["sampled_ids"]), _ptr(out.get("p_draft")), _ptr(out.get("q_draft")),
                            _ptr(out.get("row_lse")), _ptr(w), w.numel(), _stream(dev)))
        return out
    cb = L.isd_verify_carry_bytes(B, N, V)
    for name, t in (("q_stats_prev", q_stats_prev), ("q_stats_next", q_stats_next)):
        if t is not None:
            _need(t, name, torch.uint8, device=dev)
            if t.numel() < cb:
                raise ValueError(f"{name}: {t.numel()} bytes, need {cb}")
    _check(L.isd_verify_carry(_dt(logits), _ptr(logits), _ptr(draft_logits), _ptr(draft_ids),
                              _ptr(uniforms), B, N, V, float(temperature), _ptr(out["n_accept"]),
                              _ptr(out["accept"]), _ptr(out["next_token"]), _ptr(out["argmax_ids"]),
                              _ptr(out["sampled_ids"]), _ptr(out.get("p_draft")), _ptr(out.get("q_draft")),
                              _ptr(out.get("row_lse")), _ptr(q_stats_prev), _ptr(q_stats_next),
                              _ptr(w), w.numel(), _stream(dev)))
    return out


def verify_noalloc(logits, draft_logits, draft_ids, uniforms, temperature: float = 1.0,
                   out: dict | None = None):
    """verify() without a workspace (isd_verify_noalloc): the library's fixed scratch array
    on the current device serves instead, so the call allocates nothing when `out` is
    given.  Calls that overlap on one GPU race on that array.  Returns verify()'s dict."""
    B, R, V = logits.shape
    if R % 2 == 0:
        raise ValueError("logits must hold 2N-1 rows per request")
    N = (R + 1) // 2
    dev = logits.device
    _need(logits, "logits", logits.dtype, device=dev)
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", logits.dtype, (B, N - 1, V), dev)
    _need(draft_ids, "draft_ids", torch.int32, (B, N - 1), dev)
    _need(uniforms, "uniforms", torch.float32, (B, R), dev)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        out = dict(n_accept=torch.empty(B, **i32),
                   accept=torch.empty((B, N - 1), dtype=torch.uint8, device=dev),
                   next_token=torch.empty(B, **i32), argmax_ids=torch.empty((B, N), **i32),
                   sampled_ids=torch.empty((B, N), **i32), p_draft=torch.empty((B, N - 1), **f32),
                   q_draft=torch.empty((B, N - 1), **f32), row_lse=torch.empty((B, R + N - 1), **f32))
    _check(lib().isd_verify_noalloc(_dt(logits), _ptr(logits), _ptr(draft_logits), _ptr(draft_ids),
                                    _ptr(uniforms), B, N, V, float(temperature), _ptr(out["n_accept"]),
                                    _ptr(out["accept"]), _ptr(out["next_token"]), _ptr(out["argmax_ids"]),
                                    _ptr(out["sampled_ids"]), _ptr(out.get("p_draft")),
                                    _ptr(out.get("q_draft")), _ptr(out.get("row_lse")), _stream(dev)))
    return out


def commit(n_accept, next_token, sampled_ids, draft_ids, ctx_lens, tokens=None, counts=None):
    """Advance every request by one step (isd_commit): ctx_lens grows by the tokens kept,
    draft_ids becomes the next step's drafts (-1 rows: cold).  n_accept, next_token [B],
    sampled_ids [B,N]: isd_verify's outputs; draft_ids [B,N-1], ctx_lens [B] int32 are
    updated in place; tokens [B,N] and counts [B] (int32, optional) receive the kept
    tokens and their number."""
    B, N = sampled_ids.shape
    dev = sampled_ids.device
    for name, t, shape in (("n_accept", n_accept, (B,)), ("next_token", next_token, (B,)),
                           ("draft_ids", draft_ids, (B, N - 1)), ("ctx_lens", ctx_lens, (B,))):
        _need(t, name, torch.int32, shape, dev)
    _need(sampled_ids, "sampled_ids", torch.int32, (B, N), dev)
    if tokens is not None:
        _need(tokens, "tokens", torch.int32, (B, N), dev)
    if counts is not None:
        _need(counts, "counts", torch.int32, (B,), dev)
    L = lib()
    _check(L.isd_commit(_ptr(n_accept), _ptr(next_token), _ptr(sampled_ids), _ptr(draft_ids),
                        _ptr(ctx_lens), _ptr(tokens), _ptr(counts), B, N, _stream(dev)))


# ----------------------------------------------------------------------------- projection
def gated_lora_proj(x, w, a=None, b=None, gate=None, out=None):
    """R-ISD projection y = x W + gate * bf16(x A) B (bf16).  x [M,K]; w [Nout,K] (= W^T);
    a [r,K] (= A^T); b [Nout,r] (= B^T); gate [M] uint8 or None (base only)."""
    M, K = x.shape
    Nout = w.shape[0]
    dev = x.device
    bf = torch.bfloat16
    _need(x, "x", bf, device=dev)
    _need(w, "w", bf, (Nout, K), dev)
    r = 0
    if gate is not None:
        r = a.shape[0]
        _need(a, "a", bf, (r, K), dev)
        _need(b, "b", bf, (Nout, r), dev)
        _need(gate, "gate", torch.uint8, (M,), dev)
    if out is None:
        out = torch.empty((M, Nout), dtype=bf, device=dev)
    _need(out, "out", bf, (M, Nout), dev)
    L = lib()
    nbytes = L.isd_gated_lora_workspace_bytes(M, K, Nout, r)
    ws = workspace("proj", nbytes, dev, (M, K, Nout, r))
    _check(L.isd_gated_lora_proj(_ptr(x), _ptr(w), _ptr(a), _ptr(b), _ptr(gate), _ptr(out),
                                 M, K, Nout, r, _ptr(ws), ws.numel(), _stream(dev)))
    return out


class PackedProj:
    """Projection weights packed once in MFMA fragment order (isd_pack_proj_weights)."""

    def __init__(self, data: torch.Tensor, K: int, Nout: int, r: int):
        self.data, self.K, self.Nout, self.r = data, K, Nout, r


def pack_proj_weights(w, a=None, b=None) -> PackedProj:
    """Pack w [Nout,K] (= W^T), a [r,K] (= A^T), b [Nout,r] (= B^T) for
    gated_lora_proj_packed (a, b None: base weights only)."""
    Nout, K = w.shape
    dev = w.device
    bf = torch.bfloat16
    _need(w, "w", bf, (Nout, K), dev)
    r = 0
    if a is not None or b is not None:
        r = a.shape[0]
        _need(a, "a", bf, (r, K), dev)
        _need(b, "b", bf, (Nout, r), dev)
    L = lib()
    nbytes = L.isd_proj_packed_bytes(K, Nout, r)
    if nbytes == 0:
        raise IsdError(2, f"unsupported projection shape K={K} Nout={Nout} r={r}")
    data = torch.empty(nbytes // 2, dtype=bf, device=dev)
    _check(L.isd_pack_proj_weights(_ptr(w), _ptr(a), _ptr(b), _ptr(data), K, Nout, r, _stream(dev)))
    return PackedProj(data, K, Nout, r)


def pack_proj_weights_kn(w, a=None, b=None) -> PackedProj:
    """The same packed weights from the y = x W storage: w [K,Nout], a [K,r], b [r,Nout]
    (isd_pack_proj_weights_kn; a, b None: base weights only)."""
    K, Nout = w.shape
    dev = w.device
    bf = torch.bfloat16
    _need(w, "w", bf, (K, Nout), dev)
    r = 0
    if a is not None or b is not None:
        r = a.shape[1]
        _need(a, "a", bf, (K, r), dev)
        _need(b, "b", bf, (r, Nout), dev)
    L = lib()
    nbytes = L.isd_proj_packed_bytes(K, Nout, r)
    if nbytes == 0:
        raise IsdError(2, f"unsupported projection shape K={K} Nout={Nout} r={r}")
    data = torch.empty(nbytes // 2, dtype=bf, device=dev)
    _check(L.isd_pack_proj_weights_kn(_ptr(w), _ptr(a), _ptr(b), _ptr(data), K, Nout, r, _stream(dev)))
    return PackedProj(data, K, Nout, r)


def gated_lora_proj_packed(x, packed: PackedProj, gate=None, out=None):
    """gated_lora_proj on packed weights: y = x W + gate * bf16(x A) B (bf16)."""
    M, K = x.shape
    Nout, r = packed.Nout, packed.r
    dev = x.device
    bf = torch.bfloat16
    if K != packed.K:
        raise ValueError(f"x has K={K}, the weights were packed for K={packed.K}")
    _need(x, "x", bf, device=dev)
    if gate is not None:
        _need(gate, "gate", torch.uint8, (M,), dev)
    if out is None:
        out = torch.empty((M, Nout), dtype=bf, device=dev)
    _need(out, "out", bf, (M, Nout), dev)
    L = lib()
    rg = r if gate is not None else 0
    nbytes = L.isd_gated_lora_workspace_bytes(M, K, Nout, rg)
    ws = workspace("proj", nbytes, dev, (M, K, Nout, rg))
    _check(L.isd_gated_lora_proj_packed(_ptr(x), _ptr(packed.data), _ptr(gate), _ptr(out), M, K, Nout, r,
                                        _ptr(ws), ws.numel(), _stream(dev)))
    return out



def lm_head(hidden, w_lm, out=None):
    """logits [M, V] bf16 = hidden [M, Dm] . w_lm [V, Dm]^T (fp32 accumulation, nearest bf16)."""
    M, Dm = hidden.shape
    V = w_lm.shape[0]
    dev = hidden.device
    _need(hidden, "hidden", torch.bfloat16, (M, Dm), dev)
    _need(w_lm, "w_lm", torch.bfloat16, (V, Dm), dev)
    if out is None:
        out = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (M, V), dev)
    _check(lib().isd_lm_head(_ptr(hidden), _ptr(w_lm), _ptr(out), M, Dm, V, _stream(dev)))
    return out


def lm_head_verify(hidden, w_lm, draft_logits, draft_ids, uniforms, temperature: float = 1.0,
                   with_diagnostics: bool = True, out: dict | None = None):
    """The LM head and verification in one pass.  hidden [B (2N-1), Dm] bf16 (request-major),
    w_lm [V, Dm] bf16, then verify()'s arguments.  Returns verify()'s dict plus
    out["logits"] [B, 2N-1, V] bf16."""
    B, R = uniforms.shape
    if R % 2 == 0:
        raise ValueError("uniforms must hold 2N-1 entries per request")
    N = (R + 1) // 2
    M, Dm = hidden.shape
    V = w_lm.shape[0]
    dev = hidden.device
    if M != B * R:
        raise ValueError(f"hidden has {M} rows, expected B (2N-1) = {B * R}")
    _need(hidden, "hidden", torch.bfloat16, (M, Dm), dev)
    _need(w_lm, "w_lm", torch.bfloat16, (V, Dm), dev)
    if draft_logits is not None:
        _need(draft_logits, "draft_logits", torch.bfloat16, (B, N - 1, V), dev)
    _need(draft_ids, "draft_ids", torch.int32, (B, N - 1), dev)
    _need(uniforms, "uniforms", torch.float32, (B, R), dev)
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(logits=torch.empty((B, R, V), dtype=torch.bfloat16, device=dev),
                   n_accept=torch.empty(B, **i32),
                   accept=torch.empty((B, N - 1), dtype=torch.uint8, device=dev),
                   next_token=torch.empty(B, **i32), argmax_ids=torch.empty((B, N), **i32),
                   sampled_ids=torch.empty((B, N), **i32))
        if with_diagnostics:
            f32 = dict(dtype=torch.float32, device=dev)
            out.update(p_draft=torch.empty((B, N - 1), **f32), q_draft=torch.empty((B, N - 1), **f32),
                       row_lse=torch.empty((B, R + N - 1), **f32))
    _need(out["logits"], "logits", torch.bfloat16, (B, R, V), dev)
    L = lib()
    nbytes = L.isd_lm_head_verify_workspace_bytes(B, N, V)
    w = workspace("lm_head_verify", nbytes, dev, (B, N, V))
    _check(L.isd_lm_head_verify(_ptr(hidden), _ptr(w_lm), _ptr(out["logits"]), _ptr(draft_logits),
                                _ptr(draft_ids), _ptr(uniforms), B, N, Dm, V, float(temperature),
                                _ptr(out["n_accept"]), _ptr(out["accept"]), _ptr(out["next_token"]),
                                _ptr(out["argmax_ids"]), _ptr(out["sampled_ids"]), _ptr(out.get("p_draft")),
                                _ptr(out.get("q_draft")), _ptr(out.get("row_lse")), _ptr(w), w.numel(),
                                _stream(dev)))
    return out
