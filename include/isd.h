/* isd.h -- C ABI of the MI355X (gfx950) hot path of Introspective Strided Decoding.
 *
 * One ISD decode step runs a block of 2N-1 query rows per request: N-1 rows verify the
 * previous step's proposals against the causal anchor distribution p, N [MASK] rows
 * propose new tokens (「首次超越 AR 模型」 "I-DLM 如何解決這些問題"; 「内省扩散语言模型」 "1. 引言"; 「I-DLM – introspektive Diffusion Language Models」
 * "Inference & ISD").  The library provides the three data-parallel parts of that step:
 *
 *   isd_attention_step   strictly causal GQA attention of the block over a paged KV cache
 *   isd_verify           vocab-wide p/q verification, residual resampling, argmax proposals
 *   isd_gated_lora_proj  R-ISD projection: base weights on every row, LoRA delta on gated rows
 *                        (also on weights packed once in MMA fragment order: *_packed)
 *
 * and, around them, isd_commit (what a step keeps, for a loop that stays on the device)
 * and isd_lm_head / isd_lm_head_verify (the vocabulary projection that produces the
 * logits rows, alone or fused with verification's row pass).
 *
 * Conventions for every entry point
 *   - Tensor arguments are DEVICE pointers, dense and row-major in the shapes given, owned
 *     by the caller.  The library allocates nothing and keeps no state between calls.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream).  Nothing is synchronised; outputs are ready when the stream is.
 *   - Shapes, dtypes and pointers are checked on the host before anything is launched.
 *     The *_workspace_bytes and *_bytes queries return 0 for shapes their entry point
 *     does not accept.
 *     A failed check returns ISD_ERR_INVALID_ARG (bad value), ISD_ERR_UNSUPPORTED (valid
 *     but outside what the kernels implement) or ISD_ERR_WORKSPACE (too small), and
 *     launches nothing.  A failed launch returns ISD_ERR_HIP.  isd_last_error() then
 *     holds a message for the calling thread.
 *   - Values stored on the device (context lengths, page ids, draft ids) are
 *     preconditions and are not range-checked there.  Inputs must be finite.
 *   - Results are bitwise reproducible for the same inputs and shapes (fixed reduction
 *     orders, no floating-point atomics).
 *   - Each entry point has its own workspace (device memory, caller-owned, at least the
 *     size its *_workspace_bytes query returns).  Its contents on entry do not matter
 *     unless the entry point says otherwise.  Calls that share a workspace must not run
 *     concurrently.
 *   - bf16 values are IEEE binary32 truncated to their upper 16 bits (uint16 storage).
 */
#ifndef ISD_H
#define ISD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ISD_ABI_VERSION 1
#define ISD_PAGE_SIZE 16

typedef enum {
  ISD_OK = 0,
  ISD_ERR_INVALID_ARG = 1,
  ISD_ERR_UNSUPPORTED = 2,
  ISD_ERR_WORKSPACE = 3,
  ISD_ERR_HIP = 4
} isd_status;

typedef enum { ISD_F32 = 0, ISD_BF16 = 1 } isd_dtype;

int isd_abi_version(void);
const char* isd_status_string(isd_status s);
/* Message for the calling thread's last non-OK status ("" if none). */
const char* isd_last_error(void);

/* ---------------------------------------------------------------- attention
 * Strictly causal GQA attention of the 2N-1 block rows over a paged KV cache.
 * Follows: the block of 2N-1 query positions per forward (「首次超越 AR 模型」 section
 * "為什麼 I-DLM 能在高並發下保持高效"); strictly causal attention, which keeps the model
 * on an AR serving stack (「首次超越 AR 模型」 "實際部署：SGLang 整合"; 「I-DLM – introspektive Diffusion Language Models」 "I-DLM-Methodik"); a
 * paged KV cache read only through its pages (「首次超越 AR 模型」 "實際部署：SGLang 整合"; 「I-DLM – introspektive Diffusion Language Models」
 * "Serving (SGLang)").
 *
 * R = 2N-1, G = Hq/Hkv.  dtype ISD_BF16 or ISD_F32 for every tensor.
 *   q, out        [B, R, Hq, D]      query rows of the block, attention output
 *   k_new, v_new  [B, R, Hkv, D]     the block's keys/values (after any positional transform)
 *   k_cache       [num_pages, Hkv, D/8, 16, 8]      per page and KV head: blocks of 8 dims,
 *                 16 token slots each -- element (page p, head h, slot t, dim d) sits at
 *                 ((p*Hkv + h)*(D/8) + d/8)*128 + t*8 + d%8
 *   v_cache       [num_pages, Hkv, D/16, 4, 16, 4]  element (p, h, t, d) sits at
 *                 ((p*Hkv + h)*(D/16) + d/16)*256 + (t/4)*64 + (d%16)*4 + t%4
 *   page_table    [B, max_pages_per_seq] int32: physical page of logical page j of request b
 *   ctx_lens      [B] int32: tokens cached BEFORE this block (device array)
 * Effect: block row r of request b is written to token slot ctx_lens[b] + r (a bit copy;
 *   no other slot changes), and
 *   out[b,r,h] = sum_j softmax_j(scale * q[b,r,h].k_j) v_j  over tokens j = 0..ctx_lens[b]+r,
 *   KV head h / G.  The block's own keys are used as written, so the result equals attention
 *   read entirely through the pages after the append.  Rejected tokens are rolled back by the
 *   caller simply not advancing ctx_lens; their slots are overwritten by the next step.
 * Requires: page_size == 16, D in {64, 128}, Hq % Hkv == 0, Hq <= 65535,
 *   every page the request touches (ctx_lens[b]+R tokens) present in its page table,
 *   0 <= ctx_lens[b] <= max_ctx_len, max_ctx_len + R <= 16*max_pages_per_seq;
 *   for ISD_BF16 also R*G <= 64, N <= 8, B <= 2048 and
 *   B*Hkv*(ceil(max_ctx_len/16) + 25) <= 2^31 - 1 (the work list's cost units, else
 *   ISD_ERR_UNSUPPORTED); for ISD_F32 max_ctx_len + R <= 16384.
 * scale: usually 1/sqrt(D).  Workspace: isd_attention_workspace_bytes (bf16 only; the
 *   f32 path needs none). */
size_t isd_attention_workspace_bytes(int B, int N, int Hq, int Hkv, int D, int max_ctx_len);
isd_status isd_attention_step(isd_dtype dt, const void* q, const void* k_new, const void* v_new,
                              void* k_cache, void* v_cache, const int32_t* page_table,
                              const int32_t* ctx_lens, void* out, int B, int N, int Hq, int Hkv,
                              int D, int page_size, int max_pages_per_seq, int num_pages,
                              int max_ctx_len, float scale, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- page layout conversion
 * The paged KV cache as the pages state it -- a page table over fixed pages of 16 token
 * slots, each slot one row of D values per KV head (「首次超越 AR 模型」 "實際部署：SGLang 整合",
 * paged KV cache) -- converted to and from the tile layout isd_attention_step reads.
 *   k_pages, v_pages   [num_pages, Hkv, 16, D]: element (page p, head h, slot t, dim d)
 *                      at ((p*Hkv + h)*16 + t)*D + d
 *   k_cache, v_cache   the tile layouts documented at isd_attention_step
 * isd_pack_kv_pages writes k_cache / v_cache from k_pages / v_pages; isd_unpack_kv_pages
 * does the reverse.  Bit copies of every element, asynchronous on `stream`; source and
 * destination must not overlap.  dtype ISD_BF16 or ISD_F32; D in {64, 128}. */
isd_status isd_pack_kv_pages(isd_dtype dt, const void* k_pages, const void* v_pages, void* k_cache,
                             void* v_cache, int num_pages, int Hkv, int D, void* stream);
isd_status isd_unpack_kv_pages(isd_dtype dt, const void* k_cache, const void* v_cache, void* k_pages,
                               void* v_pages, int num_pages, int Hkv, int D, void* stream);

/* ---------------------------------------------------------------- KV read sweep
 * The rate reference for isd_attention_step: reads exactly the cached tiles an attention
 * step reads for the same requests -- pages 0 .. ceil(L_b/16) - 1 of request b, every KV
 * head, K and V, with L_b = min(max(ctx_lens[b], 0), max_ctx_len) -- once each, spread
 * evenly over a resident grid, and computes nothing from them (the paged KV cache of
 * 「首次超越 AR 模型」 "實際部署：SGLang 整合").  Its time is the time this chip takes to read
 * those bytes in the attention's tile order with no balancing loss.
 *   k_cache, v_cache  bf16 tile layouts as at isd_attention_step, num_pages x Hkv tiles
 *   page_table        [B, max_pages_per_seq] int32; ids are clamped into [0, num_pages)
 *   ctx_lens          [B] int32
 *   checksum          one uint32 in device memory, XORed with every 32-bit word read:
 *                     zero it first to obtain the XOR of all the tiles read
 * B in [1, 2048]; D in {64, 128}; max_ctx_len <= 16 * max_pages_per_seq.  Errors are
 * returned before any launch. */
isd_status isd_kv_read_sweep(const void* k_cache, const void* v_cache, const int32_t* page_table,
                             const int32_t* ctx_lens, int B, int Hkv, int D, int max_pages_per_seq,
                             int num_pages, int max_ctx_len, uint32_t* checksum, void* stream);

/* ---------------------------------------------------------------- verification
 * Vocab-wide verification of one ISD step.  Follows: proposals at [MASK] positions from
 * q and verification at clean positions against the anchor p with acceptance
 * min(1, p(x)/q(x)), which keeps the output distribution that of the AR model (「首次超越 AR 模型」
 * "I-DLM 如何解決這些問題"; 「I-DLM – introspektive Diffusion Language Models」 "Inference & ISD"); argmax proposals (「首次超越 AR 模型」
 * "實際部署：SGLang 整合"; 「I-DLM – introspektive Diffusion Language Models」 "Serving (SGLang)").  On a rejection the next token is
 * drawn from the normalised residual max(0, p - q~), the completion that keeps that
 * guarantee (the pages do not print it).
 *
 * Rows per request (R = 2N-1): logits rows 0..N-2 are the anchors p_i verifying draft
 * d_i = draft_ids[b][i]; rows N-1..2N-2 are the proposal rows.  Every row is softmax(l/T).
 *   logits        [B, R, V]      dtype dt
 *   draft_logits  [B, N-1, V]    row i is q~_i, the distribution d_i was drawn from (the
 *                 previous step's proposal row); NULL => argmax drafts: q~_i is one-hot on
 *                 d_i, so a_i = p_i(d_i) and the residual is p_i with d_i removed
 *   draft_ids     [B, N-1] int32 in [0, V); draft_ids[b][0] < 0 marks a cold request (no
 *                 valid drafts: no walk, n_accept 0, P = Q = 0, and next_token is the
 *                 inverse-CDF draw of row 0 -- the anchor of the next position -- at u[b][0])
 *   uniforms      [B, R] float in [0, 1): u[b][i] for draft i's test (reused as
 *                 (u - a)/(1 - a) for the residual draw), u[b][N-1+j] for proposal row j
 * Walk: a_i = 1 if P >= Q else P/Q with P = p_i(d_i), Q = q~_i(d_i); accept iff u < a_i;
 * stop at the first rejection.  Inverse CDF = smallest id k with cumulative mass > u.
 * Outputs (all written for every request):
 *   n_accept      [B] int32 in 0..N-1
 *   accept        [B, N-1] uint8, 0 after the first rejection
 *   next_token    [B] int32: residual draw if n_accept < N-1, else sampled_ids[b][0]
 *   argmax_ids    [B, N] int32: argmax of each proposal row over the raw logits, lowest id on ties
 *   sampled_ids   [B, N] int32: inverse-CDF draw of proposal row j at u[b][N-1+j]
 * Optional outputs (NULL to skip):
 *   p_draft, q_draft [B, N-1] float: P and Q of every draft (Q = 1 for argmax drafts)
 *   row_lse       [B, R + N-1] float: log-sum-exp of l/T per logits row, then per draft row
 *                 (0 for draft rows when draft_logits is NULL)
 * Requires: 1 <= N <= 8, V >= 2, temperature > 0.  Not written on error. */
size_t isd_verify_workspace_bytes(int B, int N, int V);
isd_status isd_verify(isd_dtype dt, const void* logits, const void* draft_logits,
                      const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                      float temperature, int32_t* n_accept, uint8_t* accept,
                      int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                      float* p_draft, float* q_draft, float* row_lse, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- verification across steps
 * A decoding loop's step t+1 verifies drafts drawn from step t's proposal rows N..2N-2
 * (「I-DLM – introspektive Diffusion Language Models」 "Inference & ISD": the forward that
 * proposes is the one whose q the next forward's verification uses).  Step t already
 * reduced those rows to their softmax statistics in order to sample the drafts, so step
 * t+1 need not reduce its draft_logits again.  isd_verify_carry is isd_verify with two
 * more buffers, and the same outputs bit for bit:
 *   q_stats_next  out, may be NULL: this call's statistics of rows N..2N-2 of logits
 *   q_stats_prev  in, may be NULL (then draft_logits rows are reduced here, as in
 *                 isd_verify): q_stats_next of the previous call, made with the same B, N,
 *                 V and temperature, on logits whose rows N..2N-2 are this call's
 *                 draft_logits rows 0..N-2, bit for bit.  draft_logits is still read for
 *                 the residual of rejecting requests.  Cold requests ignore it.
 * Each buffer holds isd_verify_carry_bytes(B, N, V) bytes (0 when N == 1: nothing to
 * carry); its layout is the library's.  The two must be distinct buffers.  q_stats_prev
 * requires draft_logits (sampled drafts) and N >= 2; q_stats_next requires N >= 2.
 * Workspace: isd_verify_workspace_bytes(B, N, V). */
size_t isd_verify_carry_bytes(int B, int N, int V);
isd_status isd_verify_carry(isd_dtype dt, const void* logits, const void* draft_logits,
                            const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                            float temperature, int32_t* n_accept, uint8_t* accept,
                            int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                            float* p_draft, float* q_draft, float* row_lse, const void* q_stats_prev,
                            void* q_stats_next, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- verification, no workspace
 * For callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  isd_verify with the same arguments
 * and results, minus the workspace: its scratch space is a fixed device array of
 * ISD_VERIFY_NOALLOC_MAX_BYTES that the library holds on every GPU it runs on until the
 * process ends.  Nothing is allocated; the first call on a device (with that device
 * current) looks up the array's address there.
 *   - A shape whose isd_verify_workspace_bytes exceeds ISD_VERIFY_NOALLOC_MAX_BYTES returns
 *     ISD_ERR_UNSUPPORTED (B=64, N=4, V=151936 needs about 0.5 MB; the array holds about
 *     1300 such requests).  Every other check and error is isd_verify's.
 *   - Every call on a GPU uses that GPU's one array, which keeps the last call's contents
 *     (nothing in it needs to start at zero).  Calls that overlap on one GPU -- on
 *     concurrent streams or from several threads -- race on it: serialise them.
 *   - `stream` must belong to the current device. */
#define ISD_VERIFY_NOALLOC_MAX_BYTES (8u << 20)
isd_status isd_verify_noalloc(isd_dtype dt, const void* logits, const void* draft_logits,
                              const int32_t* draft_ids, const float* uniforms, int B, int N, int V,
                              float temperature, int32_t* n_accept, uint8_t* accept,
                              int32_t* next_token, int32_t* argmax_ids, int32_t* sampled_ids,
                              float* p_draft, float* q_draft, float* row_lse, void* stream);

/* ---------------------------------------------------------------- commit
 * What one step keeps, per request -- the two-state chain of tokens per forward
 * (「I-DLM – introspektive Diffusion Language Models」 "Speedup Factor Explorer"; the step
 * that cannot verify emits one exact token and fresh proposals, "Inference & ISD").
 * The step's block held the last committed token c (position ctx_len), then the drafts.
 *   n_accept, next_token [B], sampled_ids [B, N]: isd_verify's outputs for the step
 *   draft_ids [B, N-1] in/out: in, the step's drafts (draft_ids[b][0] < 0 marks a cold
 *             request, as in isd_verify); out, the next step's drafts -- sampled_ids[b][1..N-1]
 *             when the step was cold or accepted all N-1 drafts, else -1 (the next step is
 *             cold: those proposals followed a rejected token).  May be NULL when N == 1.
 *   ctx_lens [B] in/out: grows by the number of tokens kept, n_accept + 1 (1 when cold)
 *   tokens [B, N] out, may be NULL: the kept tokens (accepted drafts, then next_token),
 *             padded with -1
 *   counts [B] out, may be NULL: the number kept
 * All device pointers; asynchronous on the stream.  Requires 1 <= N <= 8. */
isd_status isd_commit(const int32_t* n_accept, const int32_t* next_token, const int32_t* sampled_ids,
                      int32_t* draft_ids, int32_t* ctx_lens, int32_t* tokens, int32_t* counts, int B, int N,
                      void* stream);

/* ---------------------------------------------------------------- R-ISD projection
 * Gated residual adaptation of one linear layer: the LoRA delta is applied only on gated
 * ([MASK]) rows and verify rows use the base weights alone, so they equal the base model's
 * output bit for bit (「首次超越 AR 模型」 "無損 R-ISD"; 「内省扩散语言模型」 "1. 引言"; 「I-DLM – introspektive Diffusion Language Models」 "Lossless R-ISD").
 * bf16 only; fp32 accumulation.  Storage follows the linear-layer convention:
 *   x [M, K]; w [Nout, K] (= W^T); a [r, K] (= A^T); b [Nout, r] (= B^T); y [M, Nout]
 *   gate [M] uint8 in {0, 1}; NULL => base-only (a and b may then be NULL)
 * Computes y = x W + gate * (bf16(x A)) B, rounded to bf16.  Rows with gate 0 are
 * bit-identical to the base-only call on the same x, w.
 * Requires: K % 64 == 0 and 64 <= K <= 2^20, Nout % 128 == 0 and 128 <= Nout <= 2^20,
 * r in {128, 256} when gated, 1 <= M <= 65536. */
size_t isd_gated_lora_workspace_bytes(int M, int K, int Nout, int r);
isd_status isd_gated_lora_proj(const void* x, const void* w, const void* a, const void* b,
                               const uint8_t* gate, void* y, int M, int K, int Nout, int r,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- packed projection weights
 * The same R-ISD projection on weights stored once in MFMA fragment order, so that the
 * kernels read every weight byte with fully coalesced 1 KB loads and stage only the
 * activations.  Results are bit-identical to isd_gated_lora_proj on the same x, w, a, b.
 *
 * Packed layout (bf16): S = [w; a] (Nout + r rows of K) as 1 KB fragments -- fragment
 * (nb, kb), nb < (Nout + r)/16, kb < K/32, holds S[16 nb + l % 16][32 kb + 8 (l / 16) + e]
 * at element ((nb (K/32) + kb) 64 + l) 8 + e for l < 64, e < 8 -- followed by b
 * [Nout, r] unchanged.
 *
 * isd_proj_packed_bytes: size of the packed buffer (0 for unsupported shapes).
 * isd_pack_proj_weights: writes the packed buffer from w [Nout,K], a [r,K], b [Nout,r]
 *   (a, b unused when r == 0); asynchronous on `stream`.
 * isd_pack_proj_weights_kn: the same packed buffer, bit for bit, from the y = x W
 *   storage w [K,Nout], a [K,r], b [r,Nout]; a caller holding weights in that
 *   orientation packs them once without a transpose of its own.
 * isd_gated_lora_proj_packed: as isd_gated_lora_proj with the packed buffer in place of
 *   w, a, b; r is the rank the buffer was packed with (gate NULL => base only, any r).
 * Requires: K % 64 == 0 and 64 <= K <= 2^20, Nout % 128 == 0 and 128 <= Nout <= 2^20,
 *   r in {0, 128, 256}, r > 0 when gated, 1 <= M <= 65536.
 *   Workspace: isd_gated_lora_workspace_bytes(M, K, Nout, r). */
size_t isd_proj_packed_bytes(int K, int Nout, int r);
isd_status isd_pack_proj_weights(const void* w, const void* a, const void* b, void* packed, int K,
                                 int Nout, int r, void* stream);
isd_status isd_pack_proj_weights_kn(const void* w, const void* a, const void* b, void* packed, int K,
                                    int Nout, int r, void* stream);
isd_status isd_gated_lora_proj_packed(const void* x, const void* packed, const uint8_t* gate,
                                      void* y, int M, int K, int Nout, int r, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- LM head
 * The vocabulary projection that turns the block's 2N-1 rows into the logits rows that
 * verification reads: anchors on the clean rows, proposals on the [MASK] rows, from one
 * forward (「首次超越 AR 模型」 "I-DLM 如何解決這些問題"; 「I-DLM – introspektive Diffusion Language Models」 "Inference & ISD").
 * bf16 only; fp32 accumulation.
 *   hidden  [M, Dm] bf16: final hidden states of the block rows, request-major (row
 *           b (2N-1) + r is row r of request b)
 *   w_lm    [V, Dm] bf16: the output embedding, one row of Dm weights per vocabulary entry
 *   logits  [M, V] bf16 out (= [B, 2N-1, V]): the fp32-accumulated product hidden . w_lm^T
 *           rounded to the nearest bf16, ties to even
 * isd_lm_head: the logits alone; no workspace.
 *   Requires: Dm % 32 == 0 (32 <= Dm <= 65536), V % 8 == 0 (8 <= V <= 2^20),
 *   1 <= M <= 65536.
 * isd_lm_head_verify: the logits, and verification of them in the same pass: the row
 *   statistics of the logits rows (max, lowest argmax, sums of exponentials per 1024
 *   entries) come from each output tile before it leaves the chip, so the logits rows are
 *   written once and read back only where a draw or the residual needs them.  M = B (2N-1).
 *   Arguments from draft_logits on, and every output, are isd_verify's with dt = ISD_BF16
 *   and logits = the stored logits: argmax ids are identical; P, Q, row_lse and the draws
 *   agree with isd_verify on the same logits up to float rounding (the sums are added in
 *   another order), so an id can differ only where a uniform lies within that rounding of
 *   a boundary.  Requires the above and 1 <= N <= 8, 1 <= B <= 65535, temperature > 0.
 *   Workspace: isd_lm_head_verify_workspace_bytes(B, N, V). */
isd_status isd_lm_head(const void* hidden, const void* w_lm, void* logits, int M, int Dm, int V,
                       void* stream);
size_t isd_lm_head_verify_workspace_bytes(int B, int N, int V);
isd_status isd_lm_head_verify(const void* hidden, const void* w_lm, void* logits,
                              const void* draft_logits, const int32_t* draft_ids, const float* uniforms,
                              int B, int N, int Dm, int V, float temperature, int32_t* n_accept,
                              uint8_t* accept, int32_t* next_token, int32_t* argmax_ids,
                              int32_t* sampled_ids, float* p_draft, float* q_draft, float* row_lse,
                              void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ISD_H */
