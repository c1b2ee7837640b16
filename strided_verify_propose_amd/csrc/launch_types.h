// Plain launch descriptions shared by the host validation (isd_validate.cpp, which has no
// HIP dependency) and the kernels' launch functions (launch.h).  No HIP types here.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace isd {

// ---------------------------------------------------------------- attention
struct AttnLaunch {
  int dtype;  // 0 f32, 1 bf16
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;
  void* v_cache;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  void* out;
  int B, N, R, Hq, Hkv, G, D;
  int max_pages;
  int num_pages;
  int max_ctx_len;
  float scale;
  // workspace carve-up: two partial slots per workgroup of the balanced grid
  float* part_o;         // [ATTN_MAX_WG * 2][R*G][D]
  float* part_ml;        // [ATTN_MAX_WG * 2][R*G][2]
  int32_t* rec;          // [ATTN_MAX_WG][ATTN_REC_INTS] the split item whose first piece a workgroup holds
};
constexpr int ATTN_MAX_WG = 2048;  // workgroups of the balanced attention grid, at most
constexpr int ATTN_MAX_B = 2048;   // requests per bf16 attention call
constexpr int ATTN_PAGE = 16;      // tokens per page
constexpr int ATTN_REC_INTS = 8;   // ints per workgroup record of a split item
// Start-up cost of a piece of the balanced work list, in 16-token tiles: request b with
// L_b cached tokens costs Hkv (ceil(L_b/16) + 1 + ATTN_ITEM_COST) units, and the sum over
// the requests of a call is kept in 32-bit integers.
constexpr int ATTN_ITEM_COST = 24;

// Conversion between logical pages [num_pages][Hkv][16][D] and the attention tile layout.
struct KvPagesLaunch {
  int dtype;             // 0 f32, 1 bf16
  int to_tiles;          // 1: logical -> tiles, 0: tiles -> logical
  const void* k_src;
  const void* v_src;
  void* k_dst;
  void* v_dst;
  int num_pages, Hkv, D;
};

// ---------------------------------------------------------------- KV read sweep
struct KvSweepLaunch {
  const void* k_cache;
  const void* v_cache;
  const int32_t* page_table;   // [B][max_pages]
  const int32_t* ctx_lens;     // [B]
  uint32_t* checksum;          // one word, XORed with every word read
  int B, Hkv, D, max_pages, num_pages, max_ctx_len;
};

// ---------------------------------------------------------------- verification
constexpr int VCHUNK = 16384;   // vocab entries per stats workgroup
constexpr int VSUB = 1024;      // vocab entries per sub-chunk (prefix granularity)
constexpr int VCHUNK_SUBS = VCHUNK / VSUB;

struct WalkState {              // per request, written by the walk, read by the residual pass
  int rej;                      // first rejected draft index, -1 if none / handled in the walk
  int pad;
  double up;                    // (u - a) / (1 - a)
  double zp;                    // Z of p_{rej} (units of 2^(l c2 - kp))
  float kp, kq;                 // row references (max of the chunk references) of p_{rej}, q~_{rej}
  float izp_hi, izp_lo;         // 1/Z of p_{rej}, split hi + lo
  float izq_hi, izq_lo;
};

struct VerifyLaunch {
  int dtype;
  const void* logits;
  const void* draft;            // may be null
  const int32_t* draft_ids;
  const float* u;
  int B, N, R, RR, V, SV, NSUB;
  int srow0, snrow;             // rows srow0 .. srow0 + snrow - 1 of each request get the stats pass
  float invT, c2;               // 1/T and log2(e)/T
  int32_t* n_accept;
  uint8_t* accept;
  int32_t* next_token;
  int32_t* argmax_ids;
  int32_t* sampled_ids;
  float* p_draft;
  float* q_draft;
  float* row_lse;
  // workspace
  float* cmax;                  // [B][RR][SV]  chunk max of raw logits
  float* cref;                  // [B][RR][SV]  chunk reference K = fp32(cmax * c2)
  int32_t* cidx;                // [B][RR][SV]  lowest index of the chunk max
  float* csub;                  // [B][RR][NSUB] sum 2^(l c2 - K) per sub-chunk
  WalkState* ws;                // [B]
  float* rsub;                  // [B][NSUB] residual mass per sub-chunk
  // Statistics carried between the steps of a decoding loop: a step's draft rows are the
  // previous step's proposal rows N .. 2N-2, whose records that step already computed.
  // Per request and carried row i < N-1: [SV] chunk max, [SV] chunk reference, [NSUB]
  // sub-chunk sums (QS floats).
  const float* qprev;           // this call's draft rows' records, or null (computed here)
  float* qnext;                 // receives this call's rows N .. 2N-2, or null
  int QS;                       // floats per carried row: 2 SV + NSUB
};

// ---------------------------------------------------------------- LM head
constexpr int LMH_MINI = 128;   // vocabulary columns per mini-chunk record of the LM head

struct LmhLaunch {
  const uint16_t* hidden;       // [M, Dm] bf16, row b R + r
  const uint16_t* w;            // [V, Dm] bf16
  uint16_t* logits;             // [M, V] bf16 out
  int M, Dm, V, NMINI;          // NMINI = ceil(V / LMH_MINI)
  int NMS;                      // row stride of the mini-chunk records: NMINI rounded up to 8
  float c2;                     // log2(e)/T
  float* mmax;                  // [M][NMS] mini-chunk max; null: logits only
  float* msum;                  // [M][NMS] sum 2^(l c2 - fp32(max c2))
  int32_t* marg;                // [M][NMS] lowest column holding the max
  // merge into the verification's records (rows b RR + r, r < R)
  int N, R, RR, SV, NSUB;
  float* cmax;
  float* cref;
  int32_t* cidx;
  float* csub;
};

// ---------------------------------------------------------------- commit
struct CommitLaunch {
  const int32_t* n_accept;      // [B]
  const int32_t* next_token;    // [B]
  const int32_t* sampled_ids;   // [B][N]
  int32_t* draft_ids;           // [B][N-1] in: this step's drafts; out: the next step's
  int32_t* ctx_lens;            // [B] in/out
  int32_t* tokens;              // [B][N] committed tokens, -1 padded; may be null
  int32_t* counts;              // [B] number committed; may be null
  int B, N;
};

// ---------------------------------------------------------------- gated projection
struct ProjLaunch {
  const uint16_t* X;            // [M, K]
  const uint16_t* W;            // [Nout, K]  (W^T)
  const uint16_t* A;            // [r, K]     (A^T), null when ungated
  const uint16_t* Bl;           // [Nout, r]  (B^T), null when ungated
  const uint8_t* gate;          // [M] or null (base only)
  uint16_t* Y;                  // [M, Nout] bf16
  int M, K, Nout, r;            // r = 0 when ungated
  float* Ybase;                 // workspace [M, Nout] fp32 (rows with gate 1)
  uint16_t* T;                  // workspace [M, r] bf16
  const uint16_t* Sp;           // packed path: [W^T; A^T] in fragment order
  int ksplit;                   // K split into this many equal parts (1: none)
  float* part;                  // workspace [ksplit][M][Nout + r] fp32 partial sums (ksplit > 1)
  int big;                      // 224 x 256 tiles over ksplit ranges of whole k steps
};
// K split of the projection for few tiles: a function of (M, K, Nout) only, so that a
// gated call and the base-only call on the same x, w split -- and round -- alike.
int proj_ksplit(int M, int K, int Nout);
// K ranges of the large-tile path, or 0 when the 64 x 128 kernels serve (M, K, Nout).
int proj_big_split(int M, int K, int Nout);

// Tile shapes that decide the projection's work split on the host.
constexpr int PROJ_BM = 64, PROJ_BN = 128, PROJ_BK = 64;   // 64 x 128 kernels, k step 64
constexpr int PROJ_BIG_TBM = 224, PROJ_BIG_TBN = 256;      // large-tile path
// When the large-tile path is taken (measured against the 64 x 128 kernels, gated calls at
// M = 448: K = 12288 71 vs 83 us, Nout = 12288 82 vs 84 us; M = 1344: 82 vs 91 us; but
// K = Nout = 4096 42 vs 36 us, since 18 k steps per range do not pay for the partials'
// write and read):
constexpr int PROJ_BIG_MIN_ROWS = 192;                     // a 224-row tile at least 6/7 used
constexpr int PROJ_BIG_MIN_STEPS = 48;                     // k steps (of 32) per range
constexpr int PROJ_BIG_MIN_GRID = 192;                     // workgroups: three quarters of the CUs or more

}  // namespace isd
