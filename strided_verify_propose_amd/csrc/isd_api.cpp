// C ABI of the ISD hot path: argument validation (host only, before any launch),
// workspace layout, and the launches.  See include/isd.h for the contract.
#include "isd.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_err;

isd_status fail(isd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

isd_status ok() {
  g_err.clear();
  return ISD_OK;
}

isd_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(ISD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- attention workspace
struct AttnWs {
  size_t part_o, part_ml, total;
};

AttnWs attn_ws(int B, int N, int Hq, int Hkv, int D, int max_ctx_len) {
  (void)B; (void)max_ctx_len;
  AttnWs w{};
  const int R = 2 * N - 1, G = Hq / Hkv, RG = R * G;
  const size_t slots = (size_t)isd::ATTN_MAX_WG * 2;
  w.part_o = 0;
  w.part_ml = align256(slots * RG * D * sizeof(float));
  w.total = w.part_ml + align256(slots * RG * 2 * sizeof(float));
  return w;
}

// ---------------------------------------------------------------- verify workspace
struct VerWs {
  int RR, SV, NSUB;
  size_t cmax, cref, cidx, csub, ws, rsub, total;
};

VerWs ver_ws(int B, int N, int V) {
  VerWs w{};
  w.RR = (2 * N - 1) + (N - 1);
  w.SV = (V + isd::VCHUNK - 1) / isd::VCHUNK;
  w.NSUB = (V + isd::VSUB - 1) / isd::VSUB;
  const size_t rows = (size_t)B * w.RR;
  w.cmax = 0;
  w.cref = w.cmax + align256(rows * w.SV * sizeof(float));
  w.cidx = w.cref + align256(rows * w.SV * sizeof(float));
  w.csub = w.cidx + align256(rows * w.SV * sizeof(int32_t));
  w.ws = w.csub + align256(rows * w.NSUB * sizeof(float));
  w.rsub = w.ws + align256((size_t)B * sizeof(isd::WalkState));
  w.total = w.rsub + align256((size_t)B * w.NSUB * sizeof(float));
  return w;
}

// ---------------------------------------------------------------- LM-head workspace
// The verification's records, then the LM head's mini-chunk records of the logits rows.
struct LmhWs {
  VerWs v;
  int NMINI;
  size_t mmax, msum, marg, total;
};

LmhWs lmh_ws(int B, int N, int V) {
  LmhWs w{};
  w.v = ver_ws(B, N, V);
  w.NMINI = (V + isd::LMH_MINI - 1) / isd::LMH_MINI;
  const size_t recs = (size_t)B * (2 * N - 1) * ((w.NMINI + 7) & ~7);
  w.mmax = w.v.total;
  w.msum = w.mmax + align256(recs * sizeof(float));
  w.marg = w.msum + align256(recs * sizeof(float));
  w.total = w.marg + align256(recs * sizeof(int32_t));
  return w;
}

// ---------------------------------------------------------------- projection workspace
struct ProjWs {
  size_t ybase, T, part, total;
  int ksplit, big;
};

ProjWs proj_ws(int M, int K, int Nout, int r) {
  ProjWs w{};
  const int big_split = isd::proj_big_split(M, K, Nout);
  w.big = big_split > 0;
  w.ksplit = w.big ? big_split : isd::proj_ksplit(M, K, Nout);
  w.ybase = 0;
  w.T = align256(r > 0 ? (size_t)M * Nout * sizeof(float) : 0);
  w.part = w.T + align256((size_t)M * (r > 0 ? r : 0) * sizeof(uint16_t));
  w.total = w.part + align256(w.ksplit > 1 ? (size_t)w.ksplit * M * (Nout + r) * sizeof(float) : 0);
  if (w.total == 0) w.total = 256;
  return w;
}

}  // namespace

// ---------------------------------------------------------------- LM head
namespace {

isd_status check_lm_head(const char* who, const void* hidden, const void* w_lm, const void* logits,
                         long long M, int Dm, int V) {
  if (!hidden || !w_lm || !logits) return fail(ISD_ERR_INVALID_ARG, "%s: null tensor pointer", who);
  if (M < 1 || M > 65536) return fail(ISD_ERR_INVALID_ARG, "%s: %lld rows out of [1, 65536]", who, M);
  if (Dm < 32 || Dm > 65536 || Dm % 32)
    return fail(ISD_ERR_UNSUPPORTED, "%s: Dm=%d (multiple of 32 in [32, 65536] required)", who, Dm);
  if (V < 8 || V > (1 << 20) || V % 8)
    return fail(ISD_ERR_UNSUPPORTED, "%s: V=%d (multiple of 8 in [8, 2^20] required)", who, V);
  return ISD_OK;
}

isd::LmhLaunch lmh_launch(const void* hidden, const void* w_lm, void* logits, int M, int Dm, int V,
                          float c2) {
  isd::LmhLaunch p{};
  p.hidden = static_cast<const uint16_t*>(hidden);
  p.w = static_cast<const uint16_t*>(w_lm);
  p.logits = static_cast<uint16_t*>(logits);
  p.M = M; p.Dm = Dm; p.V = V;
  p.NMINI = (V + isd::LMH_MINI - 1) / isd::LMH_MINI;
  p.NMS = (p.NMINI + 7) & ~7;
  p.c2 = c2;
  return p;
}

}  // namespace

extern "C" {

int isd_abi_version(void) { return ISD_ABI_VERSION; }

const char* isd_status_string(isd_status s) {
  switch (s) {
    case ISD_OK: return "ok";
    case ISD_ERR_INVALID_ARG: return "invalid argument";
    case ISD_ERR_UNSUPPORTED: return "unsupported configuration";
    case ISD_ERR_WORKSPACE: return "workspace too small";
    case ISD_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* isd_last_error(void) { return g_err.c_str(); }

// ---------------------------------------------------------------- attention
size_t isd_attention_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int max_ctx_len) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || max_ctx_len < 0) return 0;
  return attn_ws(B, N, Hq, Hkv, D, max_ctx_len).total;
}

isd_status isd_attention_step(isd_dtype dt, const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const int32_t* page_table,
                              const int32_t* ctx_lens, void* out, int B, int N, int Hq, int Hkv,
                              int D, int page_size, int max_pages_per_seq, int num_pages,
                              int max_ctx_len, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (dt != ISD_F32 && dt != ISD_BF16) return fail(ISD_ERR_INVALID_ARG, "attention: unknown dtype %d", (int)dt);
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !page_table || !ctx_lens || !out)
    return fail(ISD_ERR_INVALID_ARG, "attention: null tensor pointer");
  if (B < 1 || B > 65535) return fail(ISD_ERR_INVALID_ARG, "attention: B=%d out of [1, 65535]", B);
  if (N < 1 || N > 64) return fail(ISD_ERR_INVALID_ARG, "attention: N=%d out of [1, 64]", N);
  if (Hq < 1 || Hkv < 1 || Hkv > 65535 || Hq % Hkv)
    return fail(ISD_ERR_INVALID_ARG, "attention: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (D != 64 && D != 128) return fail(ISD_ERR_UNSUPPORTED, "attention: D=%d (supported: 64, 128)", D);
  if (page_size != ISD_PAGE_SIZE)
    return fail(ISD_ERR_UNSUPPORTED, "attention: page_size=%d (supported: 16)", page_size);
  if (max_pages_per_seq < 1 || num_pages < 1)
    return fail(ISD_ERR_INVALID_ARG, "attention: max_pages_per_seq=%d num_pages=%d", max_pages_per_seq, num_pages);
  const int R = 2 * N - 1, G = Hq / Hkv;
  if (max_ctx_len < 0 || (long)max_ctx_len + R > (long)ISD_PAGE_SIZE * max_pages_per_seq)
    return fail(ISD_ERR_INVALID_ARG, "attention: max_ctx_len=%d + %d block rows exceeds %d pages", max_ctx_len, R, max_pages_per_seq);
  if (!std::isfinite(scale)) return fail(ISD_ERR_INVALID_ARG, "attention: scale is not finite");
  if (dt == ISD_BF16 && R * G > 64)
    return fail(ISD_ERR_UNSUPPORTED, "attention: (2N-1)*Hq/Hkv = %d query rows per KV head (max 64)", R * G);
  if (dt == ISD_BF16 && N > 8)
    return fail(ISD_ERR_UNSUPPORTED, "attention: bf16 path takes N <= 8 (the block fits one 16-token tile)");
  if (dt == ISD_BF16 && B > isd::ATTN_MAX_B)
    return fail(ISD_ERR_UNSUPPORTED, "attention: bf16 path takes at most %d requests per call", isd::ATTN_MAX_B);
  if (dt == ISD_F32 && max_ctx_len + R > 16384)
    return fail(ISD_ERR_UNSUPPORTED, "attention: f32 path holds at most 16384 tokens");
  const AttnWs w = attn_ws(B, N, Hq, Hkv, D, max_ctx_len);
  if (dt == ISD_BF16 && (!workspace || workspace_bytes < w.total))
    return fail(ISD_ERR_WORKSPACE, "attention: workspace %zu bytes, need %zu", workspace_bytes, w.total);

  isd::AttnLaunch a{};
  a.dtype = dt == ISD_BF16 ? 1 : 0;
  a.q = q; a.k_new = k_new; a.v_new = v_new; a.k_cache = k_cache; a.v_cache = v_cache;
  a.page_table = page_table; a.ctx_lens = ctx_lens; a.out = out;
  a.B = B; a.N = N; a.R = R; a.Hq = Hq; a.Hkv = Hkv; a.G = G; a.D = D;
  a.max_pages = max_pages_per_seq; a.num_pages = num_pages; a.max_ctx_len = max_ctx_len; a.scale = scale;
  char* ws = static_cast<char*>(workspace);
  a.part_o = ws ? reinterpret_cast<float*>(ws + w.part_o) : nullptr;
  a.part_ml = ws ? reinterpret_cast<float*>(ws + w.part_ml) : nullptr;
  return hip_status(isd::launch_attention(a, static_cast<hipStream_t>(stream)), "attention launch");
}

// ---------------------------------------------------------------- verification
size_t isd_verify_workspace_bytes(int B, int N, int V) {
  if (B < 1 || N < 1 || V < 2) return 0;
  return ver_ws(B, N, V).total;
}

isd_status isd_verify(isd_dtype dt, const void* logits, const void* draft_logits,
                      const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                      float temperature, int32_t* n_accept, uint8_t* accept,
                      int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                      float* p_draft, float* q_draft, float* row_lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (dt != ISD_F32 && dt != ISD_BF16) return fail(ISD_ERR_INVALID_ARG, "verify: unknown dtype %d", (int)dt);
  if (B < 1 || B > 65535) return fail(ISD_ERR_INVALID_ARG, "verify: B=%d out of [1, 65535]", B);
  if (N < 1 || N > 8) return fail(ISD_ERR_UNSUPPORTED, "verify: N=%d (supported: 1..8)", N);
  if (V < 2 || V > (1 << 20)) return fail(ISD_ERR_UNSUPPORTED, "verify: V=%d (supported: 2..2^20)", V);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(ISD_ERR_INVALID_ARG, "verify: temperature must be finite and > 0");
  if (!logits || !uniforms || !n_accept || !next_token || !argmax_ids || !sampled_ids)
    return fail(ISD_ERR_INVALID_ARG, "verify: null tensor pointer");
  if (N > 1 && (!draft_ids || !accept))
    return fail(ISD_ERR_INVALID_ARG, "verify: draft_ids and accept are required when N > 1");
  const VerWs w = ver_ws(B, N, V);
  if (!workspace || workspace_bytes < w.total)
    return fail(ISD_ERR_WORKSPACE, "verify: workspace %zu bytes, need %zu", workspace_bytes, w.total);

  isd::VerifyLaunch v{};
  v.dtype = dt == ISD_BF16 ? 1 : 0;
  v.logits = logits;
  v.draft = (N > 1) ? draft_logits : nullptr;
  v.draft_ids = draft_ids; v.u = uniforms;
  v.B = B; v.N = N; v.R = 2 * N - 1;
  v.RR = v.R + (v.draft ? N - 1 : 0);
  v.V = V; v.SV = w.SV; v.NSUB = w.NSUB;
  v.srow0 = 0; v.snrow = v.RR;
  v.invT = 1.f / temperature;
  v.c2 = (float)(1.4426950408889634 / (double)temperature);
  v.n_accept = n_accept; v.accept = accept; v.next_token = next_token;
  v.argmax_ids = argmax_ids; v.sampled_ids = sampled_ids;
  v.p_draft = p_draft; v.q_draft = q_draft; v.row_lse = row_lse;
  char* ws = static_cast<char*>(workspace);
  v.cmax = reinterpret_cast<float*>(ws + w.cmax);
  v.cref = reinterpret_cast<float*>(ws + w.cref);
  v.cidx = reinterpret_cast<int32_t*>(ws + w.cidx);
  v.csub = reinterpret_cast<float*>(ws + w.csub);
  v.ws = reinterpret_cast<isd::WalkState*>(ws + w.ws);
  v.rsub = reinterpret_cast<float*>(ws + w.rsub);
  return hip_status(isd::launch_verify(v, static_cast<hipStream_t>(stream)), "verify launch");
}

// ---------------------------------------------------------------- gated projection
size_t isd_gated_lora_workspace_bytes(int M, int K, int Nout, int r) {
  if (M < 1 || K < 64 || K % 64 || Nout < 128 || Nout % 128 || r < 0) return 0;
  return proj_ws(M, K, Nout, r).total;
}

isd_status isd_gated_lora_proj(const void* x, const void* w, const void* a, const void* b,
                               const uint8_t* gate, void* y, int M, int K, int Nout, int r,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w || !y) return fail(ISD_ERR_INVALID_ARG, "gated_lora_proj: null tensor pointer");
  if (M < 1 || M > 65536) return fail(ISD_ERR_INVALID_ARG, "gated_lora_proj: M=%d out of [1, 65536]", M);
  if (K < 64 || K % 64) return fail(ISD_ERR_UNSUPPORTED, "gated_lora_proj: K=%d (multiple of 64 required)", K);
  if (Nout < 128 || Nout % 128)
    return fail(ISD_ERR_UNSUPPORTED, "gated_lora_proj: Nout=%d (multiple of 128 required)", Nout);
  const bool lora = gate != nullptr;
  if (lora) {
    if (!a || !b) return fail(ISD_ERR_INVALID_ARG, "gated_lora_proj: gate given without a, b");
    if (r != 128 && r != 256)
      return fail(ISD_ERR_UNSUPPORTED, "gated_lora_proj: r=%d (supported: 128, 256)", r);
  }
  const ProjWs ws_ = proj_ws(M, K, Nout, lora ? r : 0);
  if ((lora || ws_.ksplit > 1) && (!workspace || workspace_bytes < ws_.total))
    return fail(ISD_ERR_WORKSPACE, "gated_lora_proj: workspace %zu bytes, need %zu", workspace_bytes, ws_.total);
  char* ws = static_cast<char*>(workspace);
  isd::ProjLaunch p{};
  p.X = static_cast<const uint16_t*>(x);
  p.W = static_cast<const uint16_t*>(w);
  p.Y = static_cast<uint16_t*>(y);
  p.M = M; p.K = K; p.Nout = Nout; p.r = 0;
  p.ksplit = ws_.ksplit;
  p.big = ws_.big;
  p.part = ws ? reinterpret_cast<float*>(ws + ws_.part) : nullptr;
  if (lora) {
    p.A = static_cast<const uint16_t*>(a);
    p.Bl = static_cast<const uint16_t*>(b);
    p.gate = gate;
    p.r = r;
    p.Ybase = reinterpret_cast<float*>(ws + ws_.ybase);
    p.T = reinterpret_cast<uint16_t*>(ws + ws_.T);
  }
  return hip_status(isd::launch_proj(p, static_cast<hipStream_t>(stream)), "gated_lora_proj launch");
}

// ---------------------------------------------------------------- packed projection weights
size_t isd_proj_packed_bytes(int K, int Nout, int r) {
  if (K < 64 || K % 64 || Nout < 128 || Nout % 128 || (r != 0 && r != 128 && r != 256)) return 0;
  return ((size_t)(Nout + r) * K + (size_t)Nout * r) * sizeof(uint16_t);
}

isd_status isd_commit(const int32_t* n_accept, const int32_t* next_token, const int32_t* sampled_ids,
                      int32_t* draft_ids, int32_t* ctx_lens, int32_t* tokens, int32_t* counts, int B, int N,
                      void* stream) {
  if (B < 1 || B > (1 << 24)) return fail(ISD_ERR_INVALID_ARG, "commit: B=%d out of [1, 2^24]", B);
  if (N < 1 || N > 8) return fail(ISD_ERR_UNSUPPORTED, "commit: N=%d (supported: 1..8)", N);
  if (!n_accept || !next_token || !sampled_ids || !ctx_lens || (N > 1 && !draft_ids))
    return fail(ISD_ERR_INVALID_ARG, "commit: null pointer");
  isd::CommitLaunch c{};
  c.n_accept = n_accept; c.next_token = next_token; c.sampled_ids = sampled_ids;
  c.draft_ids = draft_ids; c.ctx_lens = ctx_lens; c.tokens = tokens; c.counts = counts;
  c.B = B; c.N = N;
  return hip_status(isd::launch_commit(c, static_cast<hipStream_t>(stream)), "commit launch");
}

isd_status isd_pack_proj_weights(const void* w, const void* a, const void* b, void* packed, int K,
                                 int Nout, int r, void* stream) {
  if (!w || !packed) return fail(ISD_ERR_INVALID_ARG, "pack_proj_weights: null tensor pointer");
  if (K < 64 || K % 64) return fail(ISD_ERR_UNSUPPORTED, "pack_proj_weights: K=%d (multiple of 64 required)", K);
  if (Nout < 128 || Nout % 128)
    return fail(ISD_ERR_UNSUPPORTED, "pack_proj_weights: Nout=%d (multiple of 128 required)", Nout);
  if (r != 0 && r != 128 && r != 256)
    return fail(ISD_ERR_UNSUPPORTED, "pack_proj_weights: r=%d (supported: 0, 128, 256)", r);
  if (r > 0 && (!a || !b)) return fail(ISD_ERR_INVALID_ARG, "pack_proj_weights: r > 0 needs a and b");
  return hip_status(isd::launch_pack_proj(static_cast<const uint16_t*>(w), static_cast<const uint16_t*>(a),
                                          static_cast<const uint16_t*>(b), static_cast<uint16_t*>(packed), K,
                                          Nout, r, static_cast<hipStream_t>(stream)),
                    "pack_proj_weights launch");
}

isd_status isd_gated_lora_proj_packed(const void* x, const void* packed, const uint8_t* gate, void* y, int M,
                                      int K, int Nout, int r, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!x || !packed || !y) return fail(ISD_ERR_INVALID_ARG, "gated_lora_proj_packed: null tensor pointer");
  if (M < 1 || M > 65536) return fail(ISD_ERR_INVALID_ARG, "gated_lora_proj_packed: M=%d out of [1, 65536]", M);
  if (K < 64 || K % 64)
    return fail(ISD_ERR_UNSUPPORTED, "gated_lora_proj_packed: K=%d (multiple of 64 required)", K);
  if (Nout < 128 || Nout % 128)
    return fail(ISD_ERR_UNSUPPORTED, "gated_lora_proj_packed: Nout=%d (multiple of 128 required)", Nout);
  if (r != 0 && r != 128 && r != 256)
    return fail(ISD_ERR_UNSUPPORTED, "gated_lora_proj_packed: r=%d (supported: 0, 128, 256)", r);
  if (gate && r == 0) return fail(ISD_ERR_INVALID_ARG, "gated_lora_proj_packed: gate given with r=0");
  const bool lora = gate != nullptr;
  const ProjWs ws_ = proj_ws(M, K, Nout, lora ? r : 0);
  if ((lora || ws_.ksplit > 1) && (!workspace || workspace_bytes < ws_.total))
    return fail(ISD_ERR_WORKSPACE, "gated_lora_proj_packed: workspace %zu bytes, need %zu", workspace_bytes,
                ws_.total);
  char* ws = static_cast<char*>(workspace);
  const uint16_t* pk = static_cast<const uint16_t*>(packed);
  isd::ProjLaunch p{};
  p.X = static_cast<const uint16_t*>(x);
  p.Y = static_cast<uint16_t*>(y);
  p.M = M; p.K = K; p.Nout = Nout; p.r = 0;
  p.Sp = pk;
  p.ksplit = ws_.ksplit;
  p.big = ws_.big;
  p.part = ws ? reinterpret_cast<float*>(ws + ws_.part) : nullptr;
  if (lora) {
    p.gate = gate;
    p.r = r;
    p.Bl = pk + (size_t)(Nout + r) * K;
    p.Ybase = reinterpret_cast<float*>(ws + ws_.ybase);
    p.T = reinterpret_cast<uint16_t*>(ws + ws_.T);
  }
  return hip_status(isd::launch_proj_packed(p, static_cast<hipStream_t>(stream)), "gated_lora_proj_packed launch");
}



isd_status isd_lm_head(const void* hidden, const void* w_lm, void* logits, int M, int Dm, int V,
                       void* stream) {
  const isd_status st = check_lm_head("lm_head", hidden, w_lm, logits, M, Dm, V);
  if (st != ISD_OK) return st;
  const isd::LmhLaunch p = lmh_launch(hidden, w_lm, logits, M, Dm, V, 1.f);
  return hip_status(isd::launch_lm_head(p, static_cast<hipStream_t>(stream)), "lm_head launch");
}

size_t isd_lm_head_verify_workspace_bytes(int B, int N, int V) {
  if (B < 1 || N < 1 || N > 8 || V < 8) return 0;
  return lmh_ws(B, N, V).total;
}

isd_status isd_lm_head_verify(const void* hidden, const void* w_lm, void* logits,
                              const void* draft_logits, const int32_t* draft_ids, const float* uniforms,
                              int B, int N, int Dm, int V, float temperature, int32_t* n_accept,
                              uint8_t* accept, int32_t* next_token, int32_t* argmax_ids,
                              int32_t* sampled_ids, float* p_draft, float* q_draft, float* row_lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 1 || B > 65535) return fail(ISD_ERR_INVALID_ARG, "lm_head_verify: B=%d out of [1, 65535]", B);
  if (N < 1 || N > 8) return fail(ISD_ERR_UNSUPPORTED, "lm_head_verify: N=%d (supported: 1..8)", N);
  const int R = 2 * N - 1;
  const isd_status st = check_lm_head("lm_head_verify", hidden, w_lm, logits, (long long)B * R, Dm, V);
  if (st != ISD_OK) return st;
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(ISD_ERR_INVALID_ARG, "lm_head_verify: temperature must be finite and > 0");
  if (!uniforms || !n_accept || !next_token || !argmax_ids || !sampled_ids)
    return fail(ISD_ERR_INVALID_ARG, "lm_head_verify: null tensor pointer");
  if (N > 1 && (!draft_ids || !accept))
    return fail(ISD_ERR_INVALID_ARG, "lm_head_verify: draft_ids and accept are required when N > 1");
  const LmhWs w = lmh_ws(B, N, V);
  if (!workspace || workspace_bytes < w.total)
    return fail(ISD_ERR_WORKSPACE, "lm_head_verify: workspace %zu bytes, need %zu", workspace_bytes, w.total);
  char* ws = static_cast<char*>(workspace);

  isd::VerifyLaunch v{};
  v.dtype = 1;
  v.logits = logits;
  v.draft = (N > 1) ? draft_logits : nullptr;
  v.draft_ids = draft_ids; v.u = uniforms;
  v.B = B; v.N = N; v.R = R;
  v.RR = R + (v.draft ? N - 1 : 0);
  v.V = V; v.SV = w.v.SV; v.NSUB = w.v.NSUB;
  v.srow0 = R; v.snrow = N - 1;  // the stats pass covers the draft rows only
  v.invT = 1.f / temperature;
  v.c2 = (float)(1.4426950408889634 / (double)temperature);
  v.n_accept = n_accept; v.accept = accept; v.next_token = next_token;
  v.argmax_ids = argmax_ids; v.sampled_ids = sampled_ids;
  v.p_draft = p_draft; v.q_draft = q_draft; v.row_lse = row_lse;
  v.cmax = reinterpret_cast<float*>(ws + w.v.cmax);
  v.cref = reinterpret_cast<float*>(ws + w.v.cref);
  v.cidx = reinterpret_cast<int32_t*>(ws + w.v.cidx);
  v.csub = reinterpret_cast<float*>(ws + w.v.csub);
  v.ws = reinterpret_cast<isd::WalkState*>(ws + w.v.ws);
  v.rsub = reinterpret_cast<float*>(ws + w.v.rsub);

  isd::LmhLaunch p = lmh_launch(hidden, w_lm, logits, B * R, Dm, V, v.c2);
  p.mmax = reinterpret_cast<float*>(ws + w.mmax);
  p.msum = reinterpret_cast<float*>(ws + w.msum);
  p.marg = reinterpret_cast<int32_t*>(ws + w.marg);
  p.N = N; p.R = R; p.RR = v.RR; p.SV = v.SV; p.NSUB = v.NSUB;
  p.cmax = v.cmax; p.cref = v.cref; p.cidx = v.cidx; p.csub = v.csub;

  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (v.draft) e = isd::launch_verify_stats(v, s);
  if (e == hipSuccess) e = isd::launch_lm_head(p, s);
  if (e == hipSuccess) e = isd::launch_lm_head_merge(p, s);
  if (e == hipSuccess) e = isd::launch_verify_tail(v, s);
  return hip_status(e, "lm_head_verify launch");
}

}  // extern "C"
