// C ABI of the ISD hot path (include/isd.h): each entry point validates its arguments on
// the host (isd_validate.cpp, before anything is launched), then enqueues its kernels.
#include "isd.h"

#include <hip/hip_runtime.h>

#include "launch.h"
#include "validate.h"

namespace {

isd_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return isd::clear_error();
  return isd::set_error(ISD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

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

const char* isd_last_error(void) { return isd::last_error(); }

// ---------------------------------------------------------------- attention
size_t isd_attention_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int max_ctx_len) {
  return isd::attention_workspace_bytes(B, N, Hq, Hkv, D, max_ctx_len);
}

isd_status isd_attention_step(isd_dtype dt, const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const int32_t* page_table,
                              const int32_t* ctx_lens, void* out, int B, int N, int Hq, int Hkv,
                              int D, int page_size, int max_pages_per_seq, int num_pages,
                              int max_ctx_len, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  isd::AttnLaunch a;
  const isd_status st = isd::prepare_attention(dt, q, k_new, v_new, k_cache, v_cache, page_table, ctx_lens, out, B,
                                               N, Hq, Hkv, D, page_size, max_pages_per_seq, num_pages, max_ctx_len,
                                               scale, workspace, workspace_bytes, &a);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_attention(a, as_stream(stream)), "attention launch");
}

isd_status isd_pack_kv_pages(isd_dtype dt, const void* k_pages, const void* v_pages, void* k_cache,
                             void* v_cache, int num_pages, int Hkv, int D, void* stream) {
  isd::KvPagesLaunch c;
  const isd_status st = isd::prepare_kv_pages(dt, k_pages, v_pages, k_cache, v_cache, num_pages, Hkv, D, 1, &c);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_kv_pages(c, as_stream(stream)), "pack_kv_pages launch");
}

isd_status isd_unpack_kv_pages(isd_dtype dt, const void* k_cache, const void* v_cache, void* k_pages,
                               void* v_pages, int num_pages, int Hkv, int D, void* stream) {
  isd::KvPagesLaunch c;
  const isd_status st = isd::prepare_kv_pages(dt, k_cache, v_cache, k_pages, v_pages, num_pages, Hkv, D, 0, &c);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_kv_pages(c, as_stream(stream)), "unpack_kv_pages launch");
}

isd_status isd_kv_read_sweep(const void* k_cache, const void* v_cache, const int32_t* page_table,
                             const int32_t* ctx_lens, int B, int Hkv, int D, int max_pages_per_seq,
                             int num_pages, int max_ctx_len, uint32_t* checksum, void* stream) {
  isd::KvSweepLaunch c;
  const isd_status st = isd::prepare_kv_sweep(k_cache, v_cache, page_table, ctx_lens, B, Hkv, D, max_pages_per_seq,
                                              num_pages, max_ctx_len, checksum, &c);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_kv_sweep(c, as_stream(stream)), "kv_read_sweep launch");
}

// ---------------------------------------------------------------- verification
size_t isd_verify_workspace_bytes(int B, int N, int V) { return isd::verify_workspace_bytes(B, N, V); }

isd_status isd_verify(isd_dtype dt, const void* logits, const void* draft_logits,
                      const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                      float temperature, int32_t* n_accept, uint8_t* accept,
                      int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                      float* p_draft, float* q_draft, float* row_lse, void* workspace,
                      size_t workspace_bytes, void* stream) {
  isd::VerifyLaunch v;
  const isd_status st = isd::prepare_verify(dt, logits, draft_logits, draft_ids, uniforms, B, N, V, temperature,
                                            n_accept, accept, next_token, argmax_ids, sampled_ids, p_draft, q_draft,
                                            row_lse, workspace, workspace_bytes, &v);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_verify(v, as_stream(stream)), "verify launch");
}

size_t isd_verify_carry_bytes(int B, int N, int V) { return isd::verify_carry_bytes(B, N, V); }

isd_status isd_verify_carry(isd_dtype dt, const void* logits, const void* draft_logits,
                            const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                            float temperature, int32_t* n_accept, uint8_t* accept, int32_t* next_token,
                            int32_t* argmax_ids, int32_t* sampled_ids, float* p_draft, float* q_draft,
                            float* row_lse, const void* q_stats_prev, void* q_stats_next, void* workspace,
                            size_t workspace_bytes, void* stream) {
  isd::VerifyLaunch v;
  const isd_status st = isd::prepare_verify_carry(dt, logits, draft_logits, draft_ids, uniforms, B, N, V,
                                                  temperature, n_accept, accept, next_token, argmax_ids,
                                                  sampled_ids, p_draft, q_draft, row_lse, q_stats_prev,
                                                  q_stats_next, workspace, workspace_bytes, &v);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_verify(v, as_stream(stream)), "verify_carry launch");
}

// ---------------------------------------------------------------- commit
isd_status isd_commit(const int32_t* n_accept, const int32_t* next_token, const int32_t* sampled_ids,
                      int32_t* draft_ids, int32_t* ctx_lens, int32_t* tokens, int32_t* counts, int B, int N,
                      void* stream) {
  isd::CommitLaunch c;
  const isd_status st =
      isd::prepare_commit(n_accept, next_token, sampled_ids, draft_ids, ctx_lens, tokens, counts, B, N, &c);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_commit(c, as_stream(stream)), "commit launch");
}

// ---------------------------------------------------------------- gated projection
size_t isd_gated_lora_workspace_bytes(int M, int K, int Nout, int r) {
  return isd::proj_workspace_bytes(M, K, Nout, r);
}

isd_status isd_gated_lora_proj(const void* x, const void* w, const void* a, const void* b,
                               const uint8_t* gate, void* y, int M, int K, int Nout, int r,
                               void* workspace, size_t workspace_bytes, void* stream) {
  isd::ProjLaunch p;
  const isd_status st = isd::prepare_proj(x, w, a, b, gate, y, M, K, Nout, r, workspace, workspace_bytes, &p);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_proj(p, as_stream(stream)), "gated_lora_proj launch");
}

size_t isd_proj_packed_bytes(int K, int Nout, int r) { return isd::proj_packed_bytes(K, Nout, r); }

isd_status isd_pack_proj_weights(const void* w, const void* a, const void* b, void* packed, int K,
                                 int Nout, int r, void* stream) {
  const isd_status st = isd::prepare_pack_proj(w, a, b, packed, K, Nout, r);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_pack_proj(static_cast<const uint16_t*>(w), static_cast<const uint16_t*>(a),
                                          static_cast<const uint16_t*>(b), static_cast<uint16_t*>(packed), K,
                                          Nout, r, false, as_stream(stream)),
                    "pack_proj_weights launch");
}

isd_status isd_pack_proj_weights_kn(const void* w, const void* a, const void* b, void* packed, int K,
                                    int Nout, int r, void* stream) {
  const isd_status st = isd::prepare_pack_proj(w, a, b, packed, K, Nout, r);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_pack_proj(static_cast<const uint16_t*>(w), static_cast<const uint16_t*>(a),
                                          static_cast<const uint16_t*>(b), static_cast<uint16_t*>(packed), K,
                                          Nout, r, true, as_stream(stream)),
                    "pack_proj_weights_kn launch");
}

isd_status isd_gated_lora_proj_packed(const void* x, const void* packed, const uint8_t* gate, void* y, int M,
                                      int K, int Nout, int r, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  isd::ProjLaunch p;
  const isd_status st =
      isd::prepare_proj_packed(x, packed, gate, y, M, K, Nout, r, workspace, workspace_bytes, &p);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_proj_packed(p, as_stream(stream)), "gated_lora_proj_packed launch");
}

// ---------------------------------------------------------------- LM head
isd_status isd_lm_head(const void* hidden, const void* w_lm, void* logits, int M, int Dm, int V,
                       void* stream) {
  isd::LmhLaunch p;
  const isd_status st = isd::prepare_lm_head(hidden, w_lm, logits, M, Dm, V, &p);
  if (st != ISD_OK) return st;
  return hip_status(isd::launch_lm_head(p, as_stream(stream)), "lm_head launch");
}

size_t isd_lm_head_verify_workspace_bytes(int B, int N, int V) {
  return isd::lm_head_verify_workspace_bytes(B, N, V);
}

isd_status isd_lm_head_verify(const void* hidden, const void* w_lm, void* logits,
                              const void* draft_logits, const int32_t* draft_ids, const float* uniforms,
                              int B, int N, int Dm, int V, float temperature, int32_t* n_accept,
                              uint8_t* accept, int32_t* next_token, int32_t* argmax_ids,
                              int32_t* sampled_ids, float* p_draft, float* q_draft, float* row_lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  isd::LmhLaunch p;
  isd::VerifyLaunch v;
  const isd_status st = isd::prepare_lm_head_verify(
      hidden, w_lm, logits, draft_logits, draft_ids, uniforms, B, N, Dm, V, temperature, n_accept, accept,
      next_token, argmax_ids, sampled_ids, p_draft, q_draft, row_lse, workspace, workspace_bytes, &p, &v);
  if (st != ISD_OK) return st;
  const hipStream_t s = as_stream(stream);
  hipError_t e = hipSuccess;
  if (v.draft) e = isd::launch_verify_stats(v, s);
  if (e == hipSuccess) e = isd::launch_lm_head(p, s);
  if (e == hipSuccess) e = isd::launch_lm_head_merge(p, s);
  if (e == hipSuccess) e = isd::launch_verify_tail(v, s);
  return hip_status(e, "lm_head_verify launch");
}

}  // extern "C"
