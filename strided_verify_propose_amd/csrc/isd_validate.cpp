// Host-side argument validation, workspace layouts and launch descriptions for every entry
// point of include/isd.h.  No HIP dependency: isd_api.cpp calls these and then launches;
// tests/c/validate_test.cpp builds this file alone under the sanitizers.
#include "validate.h"

#include <limits.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

namespace isd {

namespace {

thread_local std::string g_err;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// ---------------------------------------------------------------- attention workspace
struct AttnWs {
  size_t part_o, part_ml, rec, total;
};

AttnWs attn_ws(int N, int Hq, int Hkv, int D) {
  AttnWs w{};
  const size_t R = 2 * (size_t)N - 1, G = (size_t)(Hq / Hkv), RG = R * G;
  const size_t slots = (size_t)ATTN_MAX_WG * 2;
  w.part_o = 0;
  w.part_ml = align256(slots * RG * D * sizeof(float));
  w.rec = w.part_ml + align256(slots * RG * 2 * sizeof(float));
  w.total = w.rec + align256((size_t)ATTN_MAX_WG * ATTN_REC_INTS * sizeof(int32_t));
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
  w.SV = (V + VCHUNK - 1) / VCHUNK;
  w.NSUB = (V + VSUB - 1) / VSUB;
  const size_t rows = (size_t)B * w.RR;
  w.cmax = 0;
  w.cref = w.cmax + align256(rows * w.SV * sizeof(float));
  w.cidx = w.cref + align256(rows * w.SV * sizeof(float));
  w.csub = w.cidx + align256(rows * w.SV * sizeof(int32_t));
  w.ws = w.csub + align256(rows * w.NSUB * sizeof(float));
  w.rsub = w.ws + align256((size_t)B * sizeof(WalkState));
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
  w.NMINI = (V + LMH_MINI - 1) / LMH_MINI;
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
  const int big_split = proj_big_split(M, K, Nout);
  w.big = big_split > 0;
  w.ksplit = w.big ? big_split : proj_ksplit(M, K, Nout);
  w.ybase = 0;
  w.T = align256(r > 0 ? (size_t)M * Nout * sizeof(float) : 0);
  w.part = w.T + align256((size_t)M * (r > 0 ? r : 0) * sizeof(uint16_t));
  w.total = w.part + align256(w.ksplit > 1 ? (size_t)w.ksplit * M * (Nout + r) * sizeof(float) : 0);
  if (w.total == 0) w.total = 256;
  return w;
}

void carve_verify(const VerWs& w, void* workspace, VerifyLaunch* v) {
  char* ws = static_cast<char*>(workspace);
  v->cmax = reinterpret_cast<float*>(ws + w.cmax);
  v->cref = reinterpret_cast<float*>(ws + w.cref);
  v->cidx = reinterpret_cast<int32_t*>(ws + w.cidx);
  v->csub = reinterpret_cast<float*>(ws + w.csub);
  v->ws = reinterpret_cast<WalkState*>(ws + w.ws);
  v->rsub = reinterpret_cast<float*>(ws + w.rsub);
}

isd_status check_lm_head(const char* who, const void* hidden, const void* w_lm, const void* logits,
                         long long M, int Dm, int V) {
  if (!hidden || !w_lm || !logits) return set_error(ISD_ERR_INVALID_ARG, "%s: null tensor pointer", who);
  if (M < 1 || M > 65536) return set_error(ISD_ERR_INVALID_ARG, "%s: %lld rows out of [1, 65536]", who, M);
  if (Dm < 32 || Dm > 65536 || Dm % 32)
    return set_error(ISD_ERR_UNSUPPORTED, "%s: Dm=%d (multiple of 32 in [32, 65536] required)", who, Dm);
  if (V < 8 || V > (1 << 20) || V % 8)
    return set_error(ISD_ERR_UNSUPPORTED, "%s: V=%d (multiple of 8 in [8, 2^20] required)", who, V);
  return ISD_OK;
}

LmhLaunch lmh_launch(const void* hidden, const void* w_lm, void* logits, int M, int Dm, int V, float c2) {
  LmhLaunch p{};
  p.hidden = static_cast<const uint16_t*>(hidden);
  p.w = static_cast<const uint16_t*>(w_lm);
  p.logits = static_cast<uint16_t*>(logits);
  p.M = M; p.Dm = Dm; p.V = V;
  p.NMINI = (V + LMH_MINI - 1) / LMH_MINI;
  p.NMS = (p.NMINI + 7) & ~7;
  p.c2 = c2;
  return p;
}

isd_status check_proj_shape(const char* who, int M, int K, int Nout) {
  if (M < 1 || M > 65536) return set_error(ISD_ERR_INVALID_ARG, "%s: M=%d out of [1, 65536]", who, M);
  if (K < 64 || K > (1 << 20) || K % 64)
    return set_error(ISD_ERR_UNSUPPORTED, "%s: K=%d (multiple of 64 in [64, 2^20] required)", who, K);
  if (Nout < 128 || Nout > (1 << 20) || Nout % 128)
    return set_error(ISD_ERR_UNSUPPORTED, "%s: Nout=%d (multiple of 128 in [128, 2^20] required)", who, Nout);
  return ISD_OK;
}

}  // namespace

isd_status set_error(isd_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

isd_status clear_error() {
  g_err.clear();
  return ISD_OK;
}

const char* last_error() { return g_err.c_str(); }

// ---------------------------------------------------------------- sizes
size_t attention_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int max_ctx_len) {
  if (B < 1 || N < 1 || N > 64 || Hq < 1 || Hq > 65535 || Hkv < 1 || Hq % Hkv || D < 1 || D > 128 ||
      max_ctx_len < 0)
    return 0;
  return attn_ws(N, Hq, Hkv, D).total;
}

size_t verify_workspace_bytes(int B, int N, int V) {
  if (B < 1 || B > 65535 || N < 1 || N > 8 || V < 2 || V > (1 << 20)) return 0;
  return ver_ws(B, N, V).total;
}

size_t verify_carry_bytes(int B, int N, int V) {
  if (B < 1 || B > 65535 || N < 2 || N > 8 || V < 2 || V > (1 << 20)) return 0;
  const VerWs w = ver_ws(B, N, V);
  return (size_t)B * (N - 1) * (2 * (size_t)w.SV + w.NSUB) * sizeof(float);
}

size_t lm_head_verify_workspace_bytes(int B, int N, int V) {
  if (B < 1 || B > 65535 || N < 1 || N > 8 || V < 8 || V > (1 << 20)) return 0;
  return lmh_ws(B, N, V).total;
}

size_t proj_workspace_bytes(int M, int K, int Nout, int r) {
  if (M < 1 || M > 65536 || K < 64 || K > (1 << 20) || K % 64 || Nout < 128 || Nout > (1 << 20) || Nout % 128 ||
      r < 0 || r > 256)
    return 0;
  return proj_ws(M, K, Nout, r).total;
}

size_t proj_packed_bytes(int K, int Nout, int r) {
  if (K < 64 || K > (1 << 20) || K % 64 || Nout < 128 || Nout > (1 << 20) || Nout % 128 ||
      (r != 0 && r != 128 && r != 256))
    return 0;
  return ((size_t)(Nout + r) * K + (size_t)Nout * r) * sizeof(uint16_t);
}

int proj_ksplit(int M, int K, int Nout) {
  // the base tiles alone (not the A^T columns) decide, so gated and base-only calls agree
  const long long tiles = (long long)((M + PROJ_BM - 1) / PROJ_BM) * (Nout / PROJ_BN);
  int s = 1;
  while (s < 8 && tiles * s * 2 <= 256 && (K / (2 * s)) % PROJ_BK == 0 && K / (2 * s) >= 4 * PROJ_BK) s *= 2;
  return s;
}

int proj_big_split(int M, int K, int Nout) {
  // tiles counted with room for a rank-128 A^T, so the gated and the base-only call agree
  const long long mt = (M + PROJ_BIG_TBM - 1) / PROJ_BIG_TBM, nt = (Nout + 128LL + PROJ_BIG_TBN - 1) / PROJ_BIG_TBN;
  const long long s = std::min(256 / (mt * nt), (long long)(K / 32) / PROJ_BIG_MIN_STEPS);
  return (M >= PROJ_BIG_MIN_ROWS && s >= 2 && mt * nt * s >= PROJ_BIG_MIN_GRID) ? (int)s : 0;
}

// ---------------------------------------------------------------- attention
isd_status prepare_attention(isd_dtype dt, const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* page_table,
                             const int32_t* ctx_lens, void* out, int B, int N, int Hq, int Hkv,
                             int D, int page_size, int max_pages_per_seq, int num_pages,
                             int max_ctx_len, float scale, void* workspace,
                             size_t workspace_bytes, AttnLaunch* a) {
  if (dt != ISD_F32 && dt != ISD_BF16) return set_error(ISD_ERR_INVALID_ARG, "attention: unknown dtype %d", (int)dt);
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !page_table || !ctx_lens || !out)
    return set_error(ISD_ERR_INVALID_ARG, "attention: null tensor pointer");
  if (B < 1 || B > 65535) return set_error(ISD_ERR_INVALID_ARG, "attention: B=%d out of [1, 65535]", B);
  if (N < 1 || N > 64) return set_error(ISD_ERR_INVALID_ARG, "attention: N=%d out of [1, 64]", N);
  if (Hq < 1 || Hq > 65535 || Hkv < 1 || Hq % Hkv)
    return set_error(ISD_ERR_INVALID_ARG, "attention: Hq=%d, Hkv=%d (Hq a multiple of Hkv, at most 65535)", Hq,
                     Hkv);
  if (D != 64 && D != 128) return set_error(ISD_ERR_UNSUPPORTED, "attention: D=%d (supported: 64, 128)", D);
  if (page_size != ISD_PAGE_SIZE)
    return set_error(ISD_ERR_UNSUPPORTED, "attention: page_size=%d (supported: 16)", page_size);
  if (max_pages_per_seq < 1 || num_pages < 1)
    return set_error(ISD_ERR_INVALID_ARG, "attention: max_pages_per_seq=%d num_pages=%d", max_pages_per_seq,
                     num_pages);
  const int R = 2 * N - 1, G = Hq / Hkv;
  if (max_ctx_len < 0 || (long long)max_ctx_len + R > (long long)ISD_PAGE_SIZE * max_pages_per_seq)
    return set_error(ISD_ERR_INVALID_ARG, "attention: max_ctx_len=%d + %d block rows exceeds %d pages", max_ctx_len,
                     R, max_pages_per_seq);
  if (!std::isfinite(scale)) return set_error(ISD_ERR_INVALID_ARG, "attention: scale is not finite");
  if (dt == ISD_BF16 && R * G > 64)
    return set_error(ISD_ERR_UNSUPPORTED, "attention: (2N-1)*Hq/Hkv = %d query rows per KV head (max 64)", R * G);
  if (dt == ISD_BF16 && N > 8)
    return set_error(ISD_ERR_UNSUPPORTED, "attention: bf16 path takes N <= 8 (the block fits one 16-token tile)");
  if (dt == ISD_BF16 && B > ATTN_MAX_B)
    return set_error(ISD_ERR_UNSUPPORTED, "attention: bf16 path takes at most %d requests per call", ATTN_MAX_B);
  if (dt == ISD_BF16) {
    // the balanced work list's cost prefix is a 32-bit sum over the requests
    const long long cost =
        (long long)B * Hkv * ((max_ctx_len + ATTN_PAGE - 1) / ATTN_PAGE + 1 + ATTN_ITEM_COST);
    if (cost > INT_MAX)
      return set_error(ISD_ERR_UNSUPPORTED,
                       "attention: B*Hkv*(max_ctx_len/16 + %d) = %lld work units exceed 2^31 - 1 per call",
                       1 + ATTN_ITEM_COST, cost);
  }
  if (dt == ISD_F32 && max_ctx_len + R > 16384)
    return set_error(ISD_ERR_UNSUPPORTED, "attention: f32 path holds at most 16384 tokens");
  const AttnWs w = attn_ws(N, Hq, Hkv, D);
  if (dt == ISD_BF16 && (!workspace || workspace_bytes < w.total))
    return set_error(ISD_ERR_WORKSPACE, "attention: workspace %zu bytes, need %zu", workspace_bytes, w.total);

  *a = AttnLaunch{};
  a->dtype = dt == ISD_BF16 ? 1 : 0;
  a->q = q; a->k_new = k_new; a->v_new = v_new; a->k_cache = k_cache; a->v_cache = v_cache;
  a->page_table = page_table; a->ctx_lens = ctx_lens; a->out = out;
  a->B = B; a->N = N; a->R = R; a->Hq = Hq; a->Hkv = Hkv; a->G = G; a->D = D;
  a->max_pages = max_pages_per_seq; a->num_pages = num_pages; a->max_ctx_len = max_ctx_len; a->scale = scale;
  char* ws = static_cast<char*>(workspace);
  a->part_o = ws ? reinterpret_cast<float*>(ws + w.part_o) : nullptr;
  a->part_ml = ws ? reinterpret_cast<float*>(ws + w.part_ml) : nullptr;
  a->rec = ws ? reinterpret_cast<int32_t*>(ws + w.rec) : nullptr;
  return clear_error();
}

// ---------------------------------------------------------------- page layout conversion
isd_status prepare_kv_pages(isd_dtype dt, const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                            int num_pages, int Hkv, int D, int to_tiles, KvPagesLaunch* c) {
  const char* who = to_tiles ? "pack_kv_pages" : "unpack_kv_pages";
  if (dt != ISD_F32 && dt != ISD_BF16) return set_error(ISD_ERR_INVALID_ARG, "%s: unknown dtype %d", who, (int)dt);
  if (!k_src || !v_src || !k_dst || !v_dst) return set_error(ISD_ERR_INVALID_ARG, "%s: null tensor pointer", who);
  if (num_pages < 1 || Hkv < 1 || Hkv > 65535)
    return set_error(ISD_ERR_INVALID_ARG, "%s: num_pages=%d Hkv=%d", who, num_pages, Hkv);
  if (D != 64 && D != 128) return set_error(ISD_ERR_UNSUPPORTED, "%s: D=%d (supported: 64, 128)", who, D);
  if ((long long)num_pages * Hkv * ATTN_PAGE * D > (1LL << 40))
    return set_error(ISD_ERR_UNSUPPORTED, "%s: %d pages x %d heads exceed 2^40 elements per call", who, num_pages,
                     Hkv);
  if (k_src == k_dst || v_src == v_dst || k_src == v_dst || v_src == k_dst)
    return set_error(ISD_ERR_INVALID_ARG, "%s: source and destination must not overlap", who);
  *c = KvPagesLaunch{};
  c->dtype = dt == ISD_BF16 ? 1 : 0;
  c->to_tiles = to_tiles ? 1 : 0;
  c->k_src = k_src; c->v_src = v_src; c->k_dst = k_dst; c->v_dst = v_dst;
  c->num_pages = num_pages; c->Hkv = Hkv; c->D = D;
  return clear_error();
}

// ---------------------------------------------------------------- KV read sweep
isd_status prepare_kv_sweep(const void* k_cache, const void* v_cache, const int32_t* page_table,
                            const int32_t* ctx_lens, int B, int Hkv, int D, int max_pages_per_seq, int num_pages,
                            int max_ctx_len, uint32_t* checksum, KvSweepLaunch* c) {
  if (!k_cache || !v_cache || !page_table || !ctx_lens || !checksum)
    return set_error(ISD_ERR_INVALID_ARG, "kv_read_sweep: null pointer");
  if (B < 1 || B > ATTN_MAX_B)
    return set_error(ISD_ERR_INVALID_ARG, "kv_read_sweep: B=%d out of [1, %d]", B, ATTN_MAX_B);
  if (Hkv < 1 || Hkv > 65535) return set_error(ISD_ERR_INVALID_ARG, "kv_read_sweep: Hkv=%d out of [1, 65535]", Hkv);
  if (D != 64 && D != 128) return set_error(ISD_ERR_UNSUPPORTED, "kv_read_sweep: D=%d (supported: 64, 128)", D);
  if (max_pages_per_seq < 1 || num_pages < 1)
    return set_error(ISD_ERR_INVALID_ARG, "kv_read_sweep: max_pages_per_seq=%d num_pages=%d", max_pages_per_seq,
                     num_pages);
  if (max_ctx_len < 0 || (long long)max_ctx_len > (long long)ATTN_PAGE * max_pages_per_seq)
    return set_error(ISD_ERR_INVALID_ARG, "kv_read_sweep: max_ctx_len=%d exceeds %d pages", max_ctx_len,
                     max_pages_per_seq);
  // the flat tile list is indexed in 32 bits
  const long long tiles = (long long)B * Hkv * ((max_ctx_len + ATTN_PAGE - 1) / ATTN_PAGE);
  if (tiles > INT_MAX)
    return set_error(ISD_ERR_UNSUPPORTED, "kv_read_sweep: %lld tiles exceed 2^31 - 1 per call", tiles);
  *c = KvSweepLaunch{};
  c->k_cache = k_cache; c->v_cache = v_cache; c->page_table = page_table; c->ctx_lens = ctx_lens;
  c->checksum = checksum;
  c->B = B; c->Hkv = Hkv; c->D = D; c->max_pages = max_pages_per_seq; c->num_pages = num_pages;
  c->max_ctx_len = max_ctx_len;
  return clear_error();
}

// ---------------------------------------------------------------- verification
isd_status prepare_verify(isd_dtype dt, const void* logits, const void* draft_logits,
                          const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                          float temperature, int32_t* n_accept, uint8_t* accept,
                          int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                          float* p_draft, float* q_draft, float* row_lse, void* workspace,
                          size_t workspace_bytes, VerifyLaunch* v) {
  if (dt != ISD_F32 && dt != ISD_BF16) return set_error(ISD_ERR_INVALID_ARG, "verify: unknown dtype %d", (int)dt);
  if (B < 1 || B > 65535) return set_error(ISD_ERR_INVALID_ARG, "verify: B=%d out of [1, 65535]", B);
  if (N < 1 || N > 8) return set_error(ISD_ERR_UNSUPPORTED, "verify: N=%d (supported: 1..8)", N);
  if (V < 2 || V > (1 << 20)) return set_error(ISD_ERR_UNSUPPORTED, "verify: V=%d (supported: 2..2^20)", V);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return set_error(ISD_ERR_INVALID_ARG, "verify: temperature must be finite and > 0");
  if (!logits || !uniforms || !n_accept || !next_token || !argmax_ids || !sampled_ids)
    return set_error(ISD_ERR_INVALID_ARG, "verify: null tensor pointer");
  if (N > 1 && (!draft_ids || !accept))
    return set_error(ISD_ERR_INVALID_ARG, "verify: draft_ids and accept are required when N > 1");
  const VerWs w = ver_ws(B, N, V);
  if (!workspace || workspace_bytes < w.total)
    return set_error(ISD_ERR_WORKSPACE, "verify: workspace %zu bytes, need %zu", workspace_bytes, w.total);

  *v = VerifyLaunch{};
  v->dtype = dt == ISD_BF16 ? 1 : 0;
  v->logits = logits;
  v->draft = (N > 1) ? draft_logits : nullptr;
  v->draft_ids = draft_ids; v->u = uniforms;
  v->B = B; v->N = N; v->R = 2 * N - 1;
  v->RR = v->R + (v->draft ? N - 1 : 0);
  v->V = V; v->SV = w.SV; v->NSUB = w.NSUB;
  v->srow0 = 0; v->snrow = v->RR;
  v->invT = 1.f / temperature;
  v->c2 = (float)(1.4426950408889634 / (double)temperature);
  v->n_accept = n_accept; v->accept = accept; v->next_token = next_token;
  v->argmax_ids = argmax_ids; v->sampled_ids = sampled_ids;
  v->p_draft = p_draft; v->q_draft = q_draft; v->row_lse = row_lse;
  v->QS = 2 * w.SV + w.NSUB;
  carve_verify(w, workspace, v);
  return clear_error();
}

isd_status prepare_verify_carry(isd_dtype dt, const void* logits, const void* draft_logits,
                                const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                                float temperature, int32_t* n_accept, uint8_t* accept,
                                int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                                float* p_draft, float* q_draft, float* row_lse, const void* q_stats_prev,
                                void* q_stats_next, void* workspace, size_t workspace_bytes, VerifyLaunch* v) {
  const isd_status st = prepare_verify(dt, logits, draft_logits, draft_ids, uniforms, B, N, V, temperature,
                                       n_accept, accept, next_token, argmax_ids, sampled_ids, p_draft, q_draft,
                                       row_lse, workspace, workspace_bytes, v);
  if (st != ISD_OK) return st;
  if (N < 2 && (q_stats_prev || q_stats_next))
    return set_error(ISD_ERR_INVALID_ARG, "verify_carry: N=1 has no draft rows to carry statistics for");
  if (q_stats_prev && !draft_logits)
    return set_error(ISD_ERR_INVALID_ARG, "verify_carry: carried statistics need draft_logits (sampled drafts)");
  if (q_stats_prev && q_stats_prev == q_stats_next)
    return set_error(ISD_ERR_INVALID_ARG, "verify_carry: q_stats_prev and q_stats_next must be distinct buffers");
  v->qprev = static_cast<const float*>(q_stats_prev);
  v->qnext = static_cast<float*>(q_stats_next);
  if (v->qprev) v->snrow = v->R;  // the draft rows' records come from the previous step
  return clear_error();
}

// ---------------------------------------------------------------- commit
isd_status prepare_commit(const int32_t* n_accept, const int32_t* next_token,
                          const int32_t* sampled_ids, int32_t* draft_ids, int32_t* ctx_lens,
                          int32_t* tokens, int32_t* counts, int B, int N, CommitLaunch* c) {
  if (B < 1 || B > (1 << 24)) return set_error(ISD_ERR_INVALID_ARG, "commit: B=%d out of [1, 2^24]", B);
  if (N < 1 || N > 8) return set_error(ISD_ERR_UNSUPPORTED, "commit: N=%d (supported: 1..8)", N);
  if (!n_accept || !next_token || !sampled_ids || !ctx_lens || (N > 1 && !draft_ids))
    return set_error(ISD_ERR_INVALID_ARG, "commit: null pointer");
  *c = CommitLaunch{};
  c->n_accept = n_accept; c->next_token = next_token; c->sampled_ids = sampled_ids;
  c->draft_ids = draft_ids; c->ctx_lens = ctx_lens; c->tokens = tokens; c->counts = counts;
  c->B = B; c->N = N;
  return clear_error();
}

// ---------------------------------------------------------------- gated projection
isd_status prepare_proj(const void* x, const void* w, const void* a, const void* b,
                        const uint8_t* gate, void* y, int M, int K, int Nout, int r,
                        void* workspace, size_t workspace_bytes, ProjLaunch* p) {
  if (!x || !w || !y) return set_error(ISD_ERR_INVALID_ARG, "gated_lora_proj: null tensor pointer");
  const isd_status st = check_proj_shape("gated_lora_proj", M, K, Nout);
  if (st != ISD_OK) return st;
  const bool lora = gate != nullptr;
  if (lora) {
    if (!a || !b) return set_error(ISD_ERR_INVALID_ARG, "gated_lora_proj: gate given without a, b");
    if (r != 128 && r != 256)
      return set_error(ISD_ERR_UNSUPPORTED, "gated_lora_proj: r=%d (supported: 128, 256)", r);
  }
  const ProjWs ws_ = proj_ws(M, K, Nout, lora ? r : 0);
  if ((lora || ws_.ksplit > 1) && (!workspace || workspace_bytes < ws_.total))
    return set_error(ISD_ERR_WORKSPACE, "gated_lora_proj: workspace %zu bytes, need %zu", workspace_bytes,
                     ws_.total);
  char* ws = static_cast<char*>(workspace);
  *p = ProjLaunch{};
  p->X = static_cast<const uint16_t*>(x);
  p->W = static_cast<const uint16_t*>(w);
  p->Y = static_cast<uint16_t*>(y);
  p->M = M; p->K = K; p->Nout = Nout; p->r = 0;
  p->ksplit = ws_.ksplit;
  p->big = ws_.big;
  p->part = ws ? reinterpret_cast<float*>(ws + ws_.part) : nullptr;
  if (lora) {
    p->A = static_cast<const uint16_t*>(a);
    p->Bl = static_cast<const uint16_t*>(b);
    p->gate = gate;
    p->r = r;
    p->Ybase = reinterpret_cast<float*>(ws + ws_.ybase);
    p->T = reinterpret_cast<uint16_t*>(ws + ws_.T);
  }
  return clear_error();
}

isd_status prepare_pack_proj(const void* w, const void* a, const void* b, void* packed, int K,
                             int Nout, int r) {
  if (!w || !packed) return set_error(ISD_ERR_INVALID_ARG, "pack_proj_weights: null tensor pointer");
  if (K < 64 || K > (1 << 20) || K % 64)
    return set_error(ISD_ERR_UNSUPPORTED, "pack_proj_weights: K=%d (multiple of 64 in [64, 2^20] required)", K);
  if (Nout < 128 || Nout > (1 << 20) || Nout % 128)
    return set_error(ISD_ERR_UNSUPPORTED, "pack_proj_weights: Nout=%d (multiple of 128 in [128, 2^20] required)",
                     Nout);
  if (r != 0 && r != 128 && r != 256)
    return set_error(ISD_ERR_UNSUPPORTED, "pack_proj_weights: r=%d (supported: 0, 128, 256)", r);
  if (r > 0 && (!a || !b)) return set_error(ISD_ERR_INVALID_ARG, "pack_proj_weights: r > 0 needs a and b");
  return clear_error();
}

isd_status prepare_proj_packed(const void* x, const void* packed, const uint8_t* gate, void* y,
                               int M, int K, int Nout, int r, void* workspace,
                               size_t workspace_bytes, ProjLaunch* p) {
  if (!x || !packed || !y) return set_error(ISD_ERR_INVALID_ARG, "gated_lora_proj_packed: null tensor pointer");
  const isd_status st = check_proj_shape("gated_lora_proj_packed", M, K, Nout);
  if (st != ISD_OK) return st;
  if (r != 0 && r != 128 && r != 256)
    return set_error(ISD_ERR_UNSUPPORTED, "gated_lora_proj_packed: r=%d (supported: 0, 128, 256)", r);
  if (gate && r == 0) return set_error(ISD_ERR_INVALID_ARG, "gated_lora_proj_packed: gate given with r=0");
  const bool lora = gate != nullptr;
  const ProjWs ws_ = proj_ws(M, K, Nout, lora ? r : 0);
  if ((lora || ws_.ksplit > 1) && (!workspace || workspace_bytes < ws_.total))
    return set_error(ISD_ERR_WORKSPACE, "gated_lora_proj_packed: workspace %zu bytes, need %zu", workspace_bytes,
                     ws_.total);
  char* ws = static_cast<char*>(workspace);
  const uint16_t* pk = static_cast<const uint16_t*>(packed);
  *p = ProjLaunch{};
  p->X = static_cast<const uint16_t*>(x);
  p->Y = static_cast<uint16_t*>(y);
  p->M = M; p->K = K; p->Nout = Nout; p->r = 0;
  p->Sp = pk;
  p->ksplit = ws_.ksplit;
  p->big = ws_.big;
  p->part = ws ? reinterpret_cast<float*>(ws + ws_.part) : nullptr;
  if (lora) {
    p->gate = gate;
    p->r = r;
    p->Bl = pk + (size_t)(Nout + r) * K;
    p->Ybase = reinterpret_cast<float*>(ws + ws_.ybase);
    p->T = reinterpret_cast<uint16_t*>(ws + ws_.T);
  }
  return clear_error();
}

// ---------------------------------------------------------------- LM head
isd_status prepare_lm_head(const void* hidden, const void* w_lm, void* logits, int M, int Dm, int V,
                           LmhLaunch* p) {
  const isd_status st = check_lm_head("lm_head", hidden, w_lm, logits, M, Dm, V);
  if (st != ISD_OK) return st;
  *p = lmh_launch(hidden, w_lm, logits, M, Dm, V, 1.f);
  return clear_error();
}

isd_status prepare_lm_head_verify(const void* hidden, const void* w_lm, void* logits,
                                  const void* draft_logits, const int32_t* draft_ids,
                                  const float* uniforms, int B, int N, int Dm, int V,
                                  float temperature, int32_t* n_accept, uint8_t* accept,
                                  int32_t* next_token, int32_t* argmax_ids,
                                  int32_t* sampled_ids, float* p_draft, float* q_draft,
                                  float* row_lse, void* workspace, size_t workspace_bytes,
                                  LmhLaunch* p, VerifyLaunch* v) {
  if (B < 1 || B > 65535) return set_error(ISD_ERR_INVALID_ARG, "lm_head_verify: B=%d out of [1, 65535]", B);
  if (N < 1 || N > 8) return set_error(ISD_ERR_UNSUPPORTED, "lm_head_verify: N=%d (supported: 1..8)", N);
  const int R = 2 * N - 1;
  const isd_status st = check_lm_head("lm_head_verify", hidden, w_lm, logits, (long long)B * R, Dm, V);
  if (st != ISD_OK) return st;
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return set_error(ISD_ERR_INVALID_ARG, "lm_head_verify: temperature must be finite and > 0");
  if (!uniforms || !n_accept || !next_token || !argmax_ids || !sampled_ids)
    return set_error(ISD_ERR_INVALID_ARG, "lm_head_verify: null tensor pointer");
  if (N > 1 && (!draft_ids || !accept))
    return set_error(ISD_ERR_INVALID_ARG, "lm_head_verify: draft_ids and accept are required when N > 1");
  const LmhWs w = lmh_ws(B, N, V);
  if (!workspace || workspace_bytes < w.total)
    return set_error(ISD_ERR_WORKSPACE, "lm_head_verify: workspace %zu bytes, need %zu", workspace_bytes, w.total);
  char* ws = static_cast<char*>(workspace);

  *v = VerifyLaunch{};
  v->dtype = 1;
  v->logits = logits;
  v->draft = (N > 1) ? draft_logits : nullptr;
  v->draft_ids = draft_ids; v->u = uniforms;
  v->B = B; v->N = N; v->R = R;
  v->RR = R + (v->draft ? N - 1 : 0);
  v->V = V; v->SV = w.v.SV; v->NSUB = w.v.NSUB;
  v->srow0 = R; v->snrow = N - 1;  // the stats pass covers the draft rows only
  v->invT = 1.f / temperature;
  v->c2 = (float)(1.4426950408889634 / (double)temperature);
  v->n_accept = n_accept; v->accept = accept; v->next_token = next_token;
  v->argmax_ids = argmax_ids; v->sampled_ids = sampled_ids;
  v->p_draft = p_draft; v->q_draft = q_draft; v->row_lse = row_lse;
  carve_verify(w.v, workspace, v);

  *p = lmh_launch(hidden, w_lm, logits, B * R, Dm, V, v->c2);
  p->mmax = reinterpret_cast<float*>(ws + w.mmax);
  p->msum = reinterpret_cast<float*>(ws + w.msum);
  p->marg = reinterpret_cast<int32_t*>(ws + w.marg);
  p->N = N; p->R = R; p->RR = v->RR; p->SV = v->SV; p->NSUB = v->NSUB;
  p->cmax = v->cmax; p->cref = v->cref; p->cidx = v->cidx; p->csub = v->csub;
  return clear_error();
}

}  // namespace isd
