// Host-side validation of every entry point's arguments, the workspace layouts, and the
// launch descriptions built from them.  Plain C++ with no HIP dependency, so that it can
// be built and tested on its own (with the address and undefined-behaviour sanitizers).
// Each prepare_* function checks its arguments in the order the C ABI documents and
// either fills the launch description (ISD_OK) or returns the error status with a
// message for isd_last_error(); nothing is launched here.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "isd.h"
#include "launch_types.h"

namespace isd {

// error state of the calling thread
isd_status set_error(isd_status s, const char* fmt, ...);
isd_status clear_error();
const char* last_error();

// Scratch layouts, carved out of one caller buffer (each part 256-byte aligned)
size_t attention_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int max_ctx_len);
size_t verify_workspace_bytes(int B, int N, int V);
size_t lm_head_verify_workspace_bytes(int B, int N, int V);
size_t verify_carry_bytes(int B, int N, int V);
size_t proj_workspace_bytes(int M, int K, int Nout, int r);
size_t proj_packed_bytes(int K, int Nout, int r);

// K split of the 64 x 128 projection kernels for few tiles: a function of (M, K, Nout)
// only, so that a gated call and the base-only call on the same x, w split -- and round --
// alike.
int proj_ksplit(int M, int K, int Nout);
// K ranges of the large-tile path, or 0 when the 64 x 128 kernels serve (M, K, Nout).
int proj_big_split(int M, int K, int Nout);

isd_status prepare_attention(isd_dtype dt, const void* q, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, const int32_t* page_table,
                             const int32_t* ctx_lens, void* out, int B, int N, int Hq, int Hkv,
                             int D, int page_size, int max_pages_per_seq, int num_pages,
                             int max_ctx_len, float scale, void* workspace,
                             size_t workspace_bytes, AttnLaunch* a);

isd_status prepare_kv_pages(isd_dtype dt, const void* k_src, const void* v_src, void* k_dst, void* v_dst,
                            int num_pages, int Hkv, int D, int to_tiles, KvPagesLaunch* c);

isd_status prepare_kv_sweep(const void* k_cache, const void* v_cache, const int32_t* page_table,
                            const int32_t* ctx_lens, int B, int Hkv, int D, int max_pages_per_seq, int num_pages,
                            int max_ctx_len, uint32_t* checksum, KvSweepLaunch* c);

isd_status prepare_verify(isd_dtype dt, const void* logits, const void* draft_logits,
                          const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                          float temperature, int32_t* n_accept, uint8_t* accept,
                          int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                          float* p_draft, float* q_draft, float* row_lse, void* workspace,
                          size_t workspace_bytes, VerifyLaunch* v);

isd_status prepare_verify_carry(isd_dtype dt, const void* logits, const void* draft_logits,
                                const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                                float temperature, int32_t* n_accept, uint8_t* accept,
                                int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                                float* p_draft, float* q_draft, float* row_lse, const void* q_stats_prev,
                                void* q_stats_next, void* workspace, size_t workspace_bytes, VerifyLaunch* v);

isd_status prepare_commit(const int32_t* n_accept, const int32_t* next_token,
                          const int32_t* sampled_ids, int32_t* draft_ids, int32_t* ctx_lens,
                          int32_t* tokens, int32_t* counts, int B, int N, CommitLaunch* c);

isd_status prepare_proj(const void* x, const void* w, const void* a, const void* b,
                        const uint8_t* gate, void* y, int M, int K, int Nout, int r,
                        void* workspace, size_t workspace_bytes, ProjLaunch* p);

isd_status prepare_pack_proj(const void* w, const void* a, const void* b, void* packed, int K,
                             int Nout, int r);

isd_status prepare_proj_packed(const void* x, const void* packed, const uint8_t* gate, void* y,
                               int M, int K, int Nout, int r, void* workspace,
                               size_t workspace_bytes, ProjLaunch* p);

isd_status prepare_lm_head(const void* hidden, const void* w_lm, void* logits, int M, int Dm,
                           int V, LmhLaunch* p);

isd_status prepare_lm_head_verify(const void* hidden, const void* w_lm, void* logits,
                                  const void* draft_logits, const int32_t* draft_ids,
                                  const float* uniforms, int B, int N, int Dm, int V,
                                  float temperature, int32_t* n_accept, uint8_t* accept,
                                  int32_t* next_token, int32_t* argmax_ids,
                                  int32_t* sampled_ids, float* p_draft, float* q_draft,
                                  float* row_lse, void* workspace, size_t workspace_bytes,
                                  LmhLaunch* p, VerifyLaunch* v);

}  // namespace isd
