// Strictly causal GQA attention of the 2N-1 strided block rows over a paged KV cache.
//
// Method (「首次超越 AR 模型」 "為什麼 I-DLM 能在高並發下保持高效": 2N-1 queries per forward; 「首次超越 AR 模型」
// "實際部署：SGLang 整合" and 「I-DLM – introspektive Diffusion Language Models」 "I-DLM-Methodik": strictly causal attention; 「首次超越 AR 模型」
// "實際部署：SGLang 整合" / 「I-DLM – introspektive Diffusion Language Models」 "Serving (SGLang)": paged KV cache, paged-only kernel):
//   out[b,r,h] = softmax_j(scale q[b,r,h].k_j) v_j over tokens j <= ctx_len[b] + r.
//
// bf16 kernel: a resident grid of workgroups over a flattened work list.
//   * The G query heads sharing a KV head and the R block rows form R*G query rows,
//     handled as 16-row MFMA blocks, so every K/V byte read serves all of them.
//   * Page layout is chosen for the MFMA operands: a K page [D/8][16][8] loads, one
//     1 KB-contiguous wave load per 32 dims, straight into the A operand of
//     S^T = K Q^T (16x16x32 bf16); a V page [D/16][4][16][4] loads (512 B per 16 dims)
//     straight into the A operand of O^T = V^T P^T (16x16x16 bf16).  S^T's accumulator
//     layout is exactly P^T's B-operand layout, and O^T keeps one query row per lane,
//     so the online softmax needs no data movement except a 4-lane max.
//   * Work is balanced by estimated time: the (request, KV head) items and their 16-token
//     tiles form one list in which every item also carries a fixed start-up cost, and
//     every workgroup of a grid sized to the resident capacity takes an equal contiguous
//     share.  A workgroup writes the output of every item it holds whole, and an
//     unnormalised partial (max, sum, O) for the at most two items cut by its share's
//     edges; a second kernel merges those in workgroup order.  No workgroup waits on or
//     signals another.
//   * The block's own K/V rows are read from k_new / v_new, and the wave that attends
//     them also stores them into their cache slots.  No piece reads those slots as
//     context, so the stores may land at any time.
//   * Inside a workgroup the group's waves take the tiles of a piece round-robin (the
//     block's own rows and the partial page first), keep the next page's loads in flight
//     while using the current one, and merge their states through LDS in a fixed order,
//     each wave combining and writing a quarter of the head dimension.
#include <algorithm>
#include <atomic>

#include "device.h"
#include "launch.h"

namespace isd {
namespace {

constexpr int PAGE = ATTN_PAGE;
constexpr int THREADS = 256;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ int page_id(const int32_t* pt, int j, int num_pages) {
  return min(max(pt[j], 0), num_pages - 1);
}

// Query rows handled per wave, waves per group and wave groups per workgroup.  Every wave
// keeps all the KV head's 16-row query blocks in registers, so every K/V byte is read from
// memory once.  With at most two blocks one group of eight waves deals the pages (two
// waves per SIMD; one workgroup per CU, so no CU splits its time between two workgroups);
// with three or four blocks (many query heads per KV head) one group of four waves, one
// per SIMD with the whole register file: two groups that split the blocks between them
// and deal the same pages fetched every page twice from HBM (the pairs' loads go out
// together and both miss).
template <int D, int NQB>
struct AttnShape {
  static constexpr int QB = NQB;
  static constexpr int GROUPS = 1;
  static constexpr int WPG = (NQB <= 2 && D / 16 >= 8) ? 8 : 4;  // waves per group
  static constexpr int THREADS = 64 * WPG * GROUPS;
  static constexpr int MIN_BLOCKS = NQB <= 2 ? 2 : 1;           // workgroups per CU the registers allow
};

// One 16-token tile (a cached page or the block) against this wave's query blocks.
// MODE 0: all tokens valid.  MODE 1: tokens t < nvalid valid.  MODE 2: block tile,
// token t valid for query row q iff t <= q / G (causal, diagonal included).
// qf[j] holds the Q^T fragments (B operand) of query block qb0 + j; blocks from nqb on
// do not exist.
template <int D, int QB, int MODE>
__device__ __forceinline__ void attend_tile(const u32x4 (&kf)[D / 32], u32x2 (&vf)[D / 16],
                                            const u32x4 (&qf)[QB][D / 32], int qb0, int nqb,
                                            f32x4 (&o)[QB][D / 16], float (&m)[QB],
                                            float (&l)[QB], float scale_log2, int nvalid,
                                            int G, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  if (MODE == 1) {
    // invalid slots may hold anything: zero their V so P = 0 never meets a non-finite V
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= nvalid) {
          const uint32_t w = vf[n][i >> 1];
          vf[n][i >> 1] = (i & 1) ? (w & 0x0000ffffu) : (w & 0xffff0000u);
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    const int qb = qb0 + j;
    if (qb >= nqb) break;
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) st = mfma16x16x32(kf[c], qf[j][c], st);
    // st[i] = S^T[token 4g+i][query row 16 qb + l16] (unscaled)
    if (MODE != 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * g + i;
        const bool ok = (MODE == 1) ? (t < nvalid) : (t <= (qb * 16 + l16) / G);
        st[i] = ok ? st[i] : neg_inf();
      }
    }
    const float mx = row4_max(fmaxf(fmaxf(st[0], st[1]), fmaxf(st[2], st[3])));
    const float mold = m[j];
    const float mnew = fmaxf(mold, mx * scale_log2);  // running max in log2 units
    // rescale O only when some query row's maximum moved (rare after the first pages)
    if (__builtin_amdgcn_ballot_w64(mnew > mold)) {
      const float alpha = (mold == neg_inf()) ? 0.f : exp2_hw(mold - mnew);
      l[j] *= alpha;
#pragma unroll
      for (int n = 0; n < D / 16; ++n) o[j][n] *= alpha;
    }
    m[j] = mnew;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2_hw(fmaf(st[i], scale_log2, -mnew));
    l[j] += (p[0] + p[1]) + (p[2] + p[3]);
    u32x2 pb;
    pb[0] = cvt_pk_bf16(p[0], p[1]);
    pb[1] = cvt_pk_bf16(p[2], p[3]);
#pragma unroll
    for (int n = 0; n < D / 16; ++n) o[j][n] = mfma16x16x16(vf[n], pb, o[j][n]);
  }
}

// Cached pages are read once per step: non-temporal loads (the nt bit), which read the
// scattered 4 KB tiles of a step about 12 % faster than plain loads on gfx950.
template <int D>
__device__ __forceinline__ void load_kv_page(const uint16_t* kt, const uint16_t* vt, int lane,
                                             u32x4 (&kf)[D / 32], u32x2 (&vf)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    kf[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kt + c * 512 + lane * 8));
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
    vf[n] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vt + n * 256 + lane * 4));
}

// Wave state (m, l, O) -> LDS, lane-contiguous so every access is conflict-free.
template <int D, int QB>
constexpr int state_floats() { return (2 * QB + QB * (D / 16) * 4) * 64; }

template <int D, int QB>
__device__ __forceinline__ void stash_state(const f32x4 (&o)[QB][D / 16], const float (&m)[QB],
                                            const float (&l)[QB], float* buf, int lane) {
#pragma unroll
  for (int j = 0; j < QB; ++j) {
    buf[(j * 2) * 64 + lane] = m[j];
    buf[(j * 2 + 1) * 64 + lane] = l[j];
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) buf[(2 * QB + (j * (D / 16) + n) * 4 + i) * 64 + lane] = o[j][n][i];
  }
}

// ---------------------------------------------------------------- balanced work list
// Item (b, h) -- request b, KV head h -- has u_b = ceil(L_b/16) + 1 units: the cached
// pages, then the block's own rows.  Starting a piece of an item costs a few dependent
// memory round trips, so the list charges every item ITEM_COST extra cost units ahead of
// its real ones: item (b, h) covers cost [s, s + ITEM_COST + u_b) with
// s = pre[b] + h (ITEM_COST + u_b), pre being the exclusive prefix of Hkv (ITEM_COST + u_b),
// and its real units sit at [s + ITEM_COST, s + ITEM_COST + u_b).  Workgroup w of a grid
// of W takes cost [w T / W, (w+1) T / W), so every workgroup gets the same estimated time
// whatever the spread of context lengths and however many items its range touches.
constexpr int MAX_B = ATTN_MAX_B;       // requests per call on the bf16 path (prefix kept in LDS)
constexpr int ITEM_COST = ATTN_ITEM_COST;  // start-up cost of a piece, in 16-token tiles

__device__ __forceinline__ int units_of(int L) { return (L + PAGE - 1) / PAGE + 1; }
__device__ __forceinline__ int cost_of(int L) { return units_of(L) + ITEM_COST; }

__device__ __forceinline__ int clamp_len(const AttnLaunch& a, int b) {
  return min(max(a.ctx_lens[b], 0), a.max_ctx_len);
}

// pre[0..B] in LDS (exclusive prefix of Hkv * cost_of(L_b)); wave 0 builds it.  Ends
// with a barrier.
__device__ void build_prefix(const AttnLaunch& a, int* pre) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (a.B + 63) / 64;
    const int b0 = min(a.B, lane * per), b1 = min(a.B, b0 + per);
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += a.Hkv * cost_of(clamp_len(a, b));
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int run = incl - sum;
    for (int b = b0; b < b1; ++b) {
      pre[b] = run;
      run += a.Hkv * cost_of(clamp_len(a, b));
    }
    if (lane == 63) pre[a.B] = incl;
  }
  __syncthreads();
}

// largest b in [0, B) with pre[b] <= x
__device__ __forceinline__ int find_request(const int* pre, int B, int x) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ int range_lo(int w, int T, int W) {
  return (int)(((long long)w * T) / W);
}

// Workgroup whose share of the cost list [range_lo(w), range_lo(w + 1)) holds position x.
__device__ __forceinline__ int holder(int x, int T, int W) {
  int w = (int)min<long long>(W - 1, ((long long)(x + 1) * W + T - 1) / T - 1);
  while (w > 0 && range_lo(w, T, W) > x) --w;
  while (w + 1 < W && range_lo(w + 1, T, W) <= x) ++w;
  return w;
}

// Share held by the workgroup with id `id` of a grid of W.  Workgroups are dispatched to the
// XCDs round-robin by id, so with W a multiple of 8 XCD x takes the contiguous shares
// x W/8 .. (x+1) W/8 - 1: the pieces of an item split between neighbouring shares are then
// mostly written and merged on one XCD, through one L2.  The combine kernel uses the same
// map.  Shares, and so results, do not depend on it.
__device__ __forceinline__ int share_of(int id, int W) {
  return (W % 8 == 0) ? (id % 8) * (W / 8) + id / 8 : id;
}

// Record of the split item whose first piece a workgroup holds (at most one: the item its
// share ends inside), for the merge kernel: request, KV head, start of the item's cost
// interval, end of its real units, total cost.
constexpr int REC_INTS = ATTN_REC_INTS;

template <int D, int NQB>
__global__ __launch_bounds__((AttnShape<D, NQB>::THREADS), (AttnShape<D, NQB>::MIN_BLOCKS))
void attn_bf16_kernel(const AttnLaunch a) {
  constexpr int QB = AttnShape<D, NQB>::QB;
  constexpr int GROUPS = AttnShape<D, NQB>::GROUPS;
  constexpr int WPG = AttnShape<D, NQB>::WPG;
  constexpr int STATE = state_floats<D, QB>();
  constexpr int NB = D / 16;           // 16-dim output blocks
  constexpr int NPW = NB / WPG;        // output blocks merged and written per wave
  static_assert(NPW * WPG == NB, "the group's waves split the output blocks evenly");
  __shared__ int pre[MAX_B + 1];
  __shared__ float st_buf[GROUPS][WPG][STATE];

  build_prefix(a, pre);
  const int T = pre[a.B];
  const int W = gridDim.x, w = share_of(blockIdx.x, W);
  const int lo = range_lo(w, T, W), hi = range_lo(w + 1, T, W);

  const int R = a.R, G = a.G, Hq = a.Hq, Hkv = a.Hkv, RG = R * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave / WPG, wg = wave % WPG;  // wave group, wave within the group
  const int qb0 = grp * QB;                  // this group's first query block
  const int l16 = lane & 15, g = lane >> 4;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const uint16_t* __restrict__ kn_ = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* __restrict__ vn_ = static_cast<const uint16_t*>(a.v_new);
  const size_t tile = (size_t)PAGE * D;
  const size_t rstride = (size_t)Hkv * D;  // between consecutive block rows

  int first = 1;  // no piece processed yet (selects the partial-result slot)
  if (threadIdx.x == 0) a.rec[w * REC_INTS] = -1;  // no split item starts here (unless found below)
  for (int cur = lo; cur < hi;) {
    // the item (b, kvh) holding cost position `cur`, and this workgroup's piece of it
    const int b = find_request(pre, a.B, cur);
    const int L = clamp_len(a, b);
    const int ncp = (L + PAGE - 1) / PAGE, nfull = L / PAGE, u = ncp + 1;
    const int kvh = (cur - pre[b]) / (u + ITEM_COST);
    const int istart = pre[b] + kvh * (u + ITEM_COST) + ITEM_COST;  // first real unit
    const int seg_end = min(hi, istart + u);
    const int unit0 = max(cur - istart, 0), unit1 = seg_end - istart;
    cur = seg_end;
    if (unit1 <= unit0) continue;  // the range covers only this item's start-up share
    if (unit0 == 0 && unit1 < u && threadIdx.x == 0) {  // the first piece of a split item
      int* r = a.rec + w * REC_INTS;
      r[0] = b;
      r[1] = kvh;
      r[2] = istart - ITEM_COST;
      r[3] = istart + u;
      r[4] = T;
    }
    const int32_t* __restrict__ pt = a.page_table + (size_t)b * a.max_pages;
    const size_t blk = ((size_t)b * R * Hkv + kvh) * D;
    const size_t hoff = (size_t)kvh * tile;
    auto page_off = [&](int id) -> size_t { return (size_t)id * Hkv * tile + hoff; };

    // The piece's units in a fixed order -- the block's own rows (unit ncp) and the
    // partial page (unit nfull) first, then the full pages ascending -- dealt round-robin
    // to the group's waves, so that every wave holds the same number of tiles.
    const bool has_block = unit0 <= ncp && ncp < unit1;
    const bool has_partial = nfull < ncp && unit0 <= nfull && nfull < unit1;
    const int nspecial = (has_block ? 1 : 0) + (has_partial ? 1 : 0);
    const bool do_block = has_block && wg == 0;
    const bool do_partial = has_partial && wg == (has_block ? 1 : 0);
    const int fend = min(unit1, nfull);  // full pages of the piece: [unit0, fend)
    int c0 = unit0 + (wg < nspecial ? wg + WPG - nspecial : wg - nspecial);  // this wave's first

    // Issue first what needs no page id: Q^T fragments (B operand of S^T = K Q^T), the
    // page ids of this wave's first 64 full pages, the partial page's id, the block rows.
    // These loads are unconditional, with indexes clamped into range and the lanes past
    // the end zeroed after the loads: a load under a branch makes the compiler wait for
    // every earlier load at the branch, one full memory round trip each.
    u32x4 qf[QB][D / 32];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int qr = (qb0 + j) * 16 + l16;
      const int qc = min(qr, RG - 1);
      const int r = qc / G, hg = qc - r * G;
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        qf[j][c] = *reinterpret_cast<const u32x4*>(q + (((size_t)b * R + r) * Hq + kvh * G + hg) * D + 32 * c + 8 * g);
    }
    int my_id = page_id(pt, min(c0 + WPG * lane, a.max_pages - 1), a.num_pages);
#pragma unroll
    for (int j = 0; j < QB; ++j)
      if (qb0 + j >= NQB || (qb0 + j) * 16 + l16 >= RG)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) qf[j][c] = u32x4{0u, 0u, 0u, 0u};
    if (c0 + WPG * lane >= fend) my_id = 0;

    f32x4 o[QB][D / 16];
    float m[QB], l[QB];
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      m[j] = neg_inf();
      l[j] = 0.f;
#pragma unroll
      for (int n = 0; n < D / 16; ++n) o[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    u32x4 kf[D / 32], kf2[D / 32];
    u32x2 vf[D / 16], vf2[D / 16];

    int blk_page0 = 0, blk_page1 = 0;  // pages of the block's first and last slot
    if (do_block) {  // the block's own rows, from k_new / v_new (rows past R zeroed)
      blk_page0 = page_id(pt, L / PAGE, a.num_pages);
      blk_page1 = page_id(pt, (L + R - 1) / PAGE, a.num_pages);
#pragma unroll
      for (int c = 0; c < D / 32; ++c)
        kf2[c] = *reinterpret_cast<const u32x4*>(kn_ + blk + min(l16, R - 1) * rstride + 32 * c + 8 * g);
      uint32_t h[D / 16][4];
#pragma unroll
      for (int n = 0; n < D / 16; ++n)
#pragma unroll
        for (int t = 0; t < 4; ++t) h[n][t] = vn_[blk + min(4 * g + t, R - 1) * rstride + 16 * n + l16];
      if (l16 >= R)
#pragma unroll
        for (int c = 0; c < D / 32; ++c) kf2[c] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int n = 0; n < D / 16; ++n) {
#pragma unroll
        for (int t = 0; t < 4; ++t) h[n][t] = (4 * g + t < R) ? h[n][t] : 0u;
        vf2[n][0] = h[n][0] | (h[n][1] << 16);
        vf2[n][1] = h[n][2] | (h[n][3] << 16);
      }
    }
    if (do_partial) {
      const size_t t = page_off(page_id(pt, nfull, a.num_pages));
      load_kv_page<D>(kc + t, vc + t, lane, kf2, vf2);
    }
    // the first full page goes out before the special tile is used
    if (c0 < fend) {
      const size_t t = page_off(__builtin_amdgcn_readlane(my_id, 0));
      load_kv_page<D>(kc + t, vc + t, lane, kf, vf);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (do_block) {
      // The append: the block's rows, already in this wave's registers, go to their page
      // slots ctx_len + r.  No piece reads those slots from the cache (the block is read
      // from k_new / v_new, and slots past the context are masked in the partial page), so
      // the stores may land at any time during the kernel.
      uint16_t* kcw = static_cast<uint16_t*>(a.k_cache);
      uint16_t* vcw = static_cast<uint16_t*>(a.v_cache);
      if (l16 < R) {
        const int j = L + l16;
        const size_t base = page_off(j / PAGE == L / PAGE ? blk_page0 : blk_page1);
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
          *reinterpret_cast<u32x4*>(kcw + base + (4 * c + g) * 128 + (j % PAGE) * 8) = kf2[c];
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (4 * g + t >= R) continue;
        const int j = L + 4 * g + t, slot = j % PAGE;
        const size_t base = page_off(j / PAGE == L / PAGE ? blk_page0 : blk_page1) + (slot / 4) * 64 + (slot % 4);
#pragma unroll
        for (int n = 0; n < D / 16; ++n)
          vcw[base + n * 256 + l16 * 4] = (uint16_t)(vf2[n][t >> 1] >> (16 * (t & 1)));
      }
      attend_tile<D, QB, 2>(kf2, vf2, qf, qb0, NQB, o, m, l, scale_log2, 0, G, lane);
    }
    if (do_partial)
      attend_tile<D, QB, 1>(kf2, vf2, qf, qb0, NQB, o, m, l, scale_log2, L - nfull * PAGE, G, lane);

    // Full pages, 64 page ids at a time (one per lane, read back as scalars).  Two
    // register buffers: the next page's loads are issued before the current page is
    // used, and a scheduling barrier keeps them there.  Loads inside the loop are
    // unconditional, so the compiler's wait counts stay exact (the tail is peeled).
    for (; c0 < fend; c0 += 64 * WPG) {
      const int nu = min(64, (fend - c0 + WPG - 1) / WPG);
      size_t t;
      if (c0 != unit0 + (wg < nspecial ? wg + WPG - nspecial : wg - nspecial)) {
        t = page_off(__builtin_amdgcn_readlane(my_id, 0));
        load_kv_page<D>(kc + t, vc + t, lane, kf, vf);
      }
      int i = 0;
      for (; i + 2 < nu; i += 2) {
        t = page_off(__builtin_amdgcn_readlane(my_id, i + 1));
        load_kv_page<D>(kc + t, vc + t, lane, kf2, vf2);
        __builtin_amdgcn_sched_barrier(0);
        attend_tile<D, QB, 0>(kf, vf, qf, qb0, NQB, o, m, l, scale_log2, PAGE, G, lane);
        t = page_off(__builtin_amdgcn_readlane(my_id, i + 2));
        load_kv_page<D>(kc + t, vc + t, lane, kf, vf);
        __builtin_amdgcn_sched_barrier(0);
        attend_tile<D, QB, 0>(kf2, vf2, qf, qb0, NQB, o, m, l, scale_log2, PAGE, G, lane);
      }
      if (i + 1 < nu) {
        t = page_off(__builtin_amdgcn_readlane(my_id, i + 1));
        load_kv_page<D>(kc + t, vc + t, lane, kf2, vf2);
        __builtin_amdgcn_sched_barrier(0);
        attend_tile<D, QB, 0>(kf, vf, qf, qb0, NQB, o, m, l, scale_log2, PAGE, G, lane);
        attend_tile<D, QB, 0>(kf2, vf2, qf, qb0, NQB, o, m, l, scale_log2, PAGE, G, lane);
      } else {
        attend_tile<D, QB, 0>(kf, vf, qf, qb0, NQB, o, m, l, scale_log2, PAGE, G, lane);
      }
      if (c0 + 64 * WPG < fend) {
        my_id = page_id(pt, min(c0 + 64 * WPG + WPG * lane, a.max_pages - 1), a.num_pages);
        if (c0 + 64 * WPG + WPG * lane >= fend) my_id = 0;
      }
    }

    // Merge the group's wave states: all of them go to LDS, then wave k of the group
    // combines output blocks [k NPW, (k+1) NPW) of every query row over the waves in
    // wave order, and writes them.
#pragma unroll
    for (int j = 0; j < QB; ++j) l[j] = row4_sum(l[j]);
    stash_state<D, QB>(o, m, l, st_buf[grp][wg], lane);
    lds_barrier();
    const bool whole = (unit0 == 0 && unit1 == u);
    const size_t slot = (size_t)w * 2 + (first ? 0 : 1);
    float* po = a.part_o + slot * RG * D;
    float* pml = a.part_ml + slot * RG * 2;
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int j = 0; j < QB; ++j) {
      const int qr = (qb0 + j) * 16 + l16;
      float mw[WPG], fw[WPG];
      float M = neg_inf();
#pragma unroll
      for (int k = 0; k < WPG; ++k) {
        mw[k] = st_buf[grp][k][(j * 2) * 64 + lane];
        M = fmaxf(M, mw[k]);
      }
      float Lsum = 0.f;
#pragma unroll
      for (int k = 0; k < WPG; ++k) {
        fw[k] = (mw[k] == neg_inf()) ? 0.f : exp2_hw(mw[k] - M);
        Lsum += fw[k] * st_buf[grp][k][(j * 2 + 1) * 64 + lane];
      }
      const float inv = 1.f / Lsum;
      const int r = qr / G, hg = qr - r * G;
#pragma unroll
      for (int nn = 0; nn < NPW; ++nn) {
        const int n = wg * NPW + nn;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < WPG; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i] += fw[k] * st_buf[grp][k][(2 * QB + (j * (D / 16) + n) * 4 + i) * 64 + lane];
        if (qb0 + j >= NQB || qr >= RG) continue;
        if (whole) {
          u32x2 wv;
          wv[0] = cvt_pk_bf16(acc[0] * inv, acc[1] * inv);
          wv[1] = cvt_pk_bf16(acc[2] * inv, acc[3] * inv);
          // output row (b, r, head): below B R Hq <= 2048 * 15 * 65535 < 2^32
          const unsigned orow = (unsigned)(b * R + r) * (unsigned)Hq + (unsigned)(kvh * G + hg);
          *reinterpret_cast<u32x2*>(out + (size_t)orow * D + 16 * n + 4 * g) = wv;
        } else {
          *reinterpret_cast<f32x4*>(po + (size_t)qr * D + 16 * n + 4 * g) = acc;
        }
      }
      if (!whole && wg == 0 && g == 0 && qb0 + j < NQB && qr < RG) {
        pml[qr * 2] = M;
        pml[qr * 2 + 1] = Lsum;
      }
    }
    lds_barrier();  // every wave has read the stashed states before they are overwritten
    first = 0;
  }
}

// Merge the pieces of items that crossed workgroup boundaries.  Workgroup w of this grid
// reads the record the main kernel's workgroup w wrote: the split item whose first piece
// it held, if any.  The workgroups holding pieces of that item are w .. w1 (those whose
// share meets the item's real units); each wrote its piece in slot 2k + 1 if its share
// began before the item (it already wrote a piece of an earlier item), else in slot 2k.
// The pieces are merged in workgroup order.
constexpr int COMBINE_THREADS = 256;
static_assert(COMBINE_THREADS == 4 * 64, "the combine's few-piece path maps thread -> (piece, row) as 4 x 64");

template <int D>
__global__ __launch_bounds__(COMBINE_THREADS) void attn_combine_kernel(const AttnLaunch a, int W) {
  const int w0 = share_of(blockIdx.x, W);
  const int tid = threadIdx.x;
  const int* rec = a.rec + (size_t)w0 * REC_INTS;
  const int b = rec[0];
  if (b < 0) return;  // no split item starts in this workgroup's share
  const int kvh = rec[1], c0 = rec[2], iend = rec[3], T = rec[4];
  const int w1 = holder(iend - 1, T, W);  // the last workgroup holding a piece
  const int istart = c0 + ITEM_COST;
  const int R = a.R, G = a.G, Hq = a.Hq, RG = R * G;
  __shared__ int s_slots[2 * ATTN_MAX_WG];
  __shared__ int s_np;
  if (tid < 64) {
    const int lane = tid;
    int n = 0;
    for (int k0 = w0; k0 <= w1; k0 += 64) {
      const int w = k0 + lane;
      const int lo = range_lo(w, T, W), hi = range_lo(w + 1, T, W);
      const bool ok = w <= w1 && max(lo, istart) < min(hi, iend);
      const unsigned long long bal = __ballot(ok);
      if (ok) s_slots[n + __popcll(bal & ((1ull << lane) - 1))] = 2 * w + (lo < c0 ? 1 : 0);
      n += __popcll(bal);
    }
    if (lane == 0) s_np = n;
  }
  lds_barrier();
  const int np = s_np;
  auto slot_of = [&](int k) -> int { return s_slots[k]; };

  // Per query row: the pieces' common maximum M and 1 / sum_k 2^(m_k - M) l_k.  Then every
  // output element is sum_k 2^(m_k - M) O_k / den: the weights of up to CHUNK pieces at a
  // time are staged in LDS, and the O loads of four elements and four pieces go out
  // together.
  constexpr int CHUNK = 32;                  // pieces staged in LDS at a time
  constexpr int PER = 4;                     // elements per thread per pass
  constexpr int KB = 4;                      // pieces per batch of loads
  const int nitems = RG * (D / 4);           // output elements of 4 dims
  __shared__ float s_m[CHUNK][64], s_l[CHUNK][64], s_f[CHUNK][64], s_M[64], s_inv[64];
  uint16_t* out = static_cast<uint16_t*>(a.out);
  if (np <= KB && nitems <= PER * COMBINE_THREADS) {
    // Few pieces, one pass: the O values of every piece and the (m, l) pairs go out in
    // one round trip; the weights follow from LDS.  Same arithmetic as the general path.
    f32x4 ov[PER][KB];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int it = min(e * COMBINE_THREADS + (int)threadIdx.x, nitems - 1);
      const int qr = it / (D / 4), d4 = it - qr * (D / 4);
#pragma unroll
      for (int k = 0; k < KB; ++k)
        ov[e][k] = *reinterpret_cast<const f32x4*>(a.part_o + ((size_t)slot_of(min(k, np - 1)) * RG + qr) * D + 4 * d4);
    }
    {
      const int k = threadIdx.x >> 6, qr = threadIdx.x & 63;  // COMBINE_THREADS = KB * 64
      const float* ml = a.part_ml + ((size_t)slot_of(min(k, np - 1)) * RG + min(qr, RG - 1)) * 2;
      const float m = ml[0], l = ml[1];
      s_m[k][qr] = m;
      s_l[k][qr] = l;
    }
    lds_barrier();
    for (int qr = threadIdx.x; qr < RG; qr += COMBINE_THREADS) {
      float M = neg_inf();
      for (int k = 0; k < np; ++k) M = fmaxf(M, s_m[k][qr]);
      float den = 0.f;
      for (int k = 0; k < np; ++k) {
        const float m = s_m[k][qr];
        den += ((m == neg_inf()) ? 0.f : exp2_hw(m - M)) * s_l[k][qr];
      }
      s_inv[qr] = 1.f / den;
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const float m = s_m[k][qr];
        s_f[k][qr] = (k < np && m != neg_inf()) ? exp2_hw(m - M) : 0.f;
      }
    }
    lds_barrier();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int it = e * COMBINE_THREADS + threadIdx.x;
      if (it >= nitems) break;
      const int qr = it / (D / 4), d4 = it - qr * (D / 4);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KB; ++k) acc += s_f[k][qr] * ov[e][k];
      const float inv = s_inv[qr];
      const int r = qr / G, hg = qr - r * G;
      u32x2 wv;
      wv[0] = cvt_pk_bf16(acc[0] * inv, acc[1] * inv);
      wv[1] = cvt_pk_bf16(acc[2] * inv, acc[3] * inv);
      *reinterpret_cast<u32x2*>(out + (((size_t)b * R + r) * Hq + kvh * G + hg) * D + 4 * d4) = wv;
    }
    return;
  }
  if (np <= CHUNK) {
    for (int idx = threadIdx.x; idx < np * 64; idx += COMBINE_THREADS) {
      const int k = idx >> 6, qr = idx & 63;
      if (qr < RG) {
        const float* ml = a.part_ml + ((size_t)slot_of(k) * RG + qr) * 2;
        s_m[k][qr] = ml[0];
        s_l[k][qr] = ml[1];
      }
    }
    lds_barrier();
  }
  for (int qr = threadIdx.x; qr < RG; qr += COMBINE_THREADS) {
    auto m_of = [&](int k) -> float {
      return np <= CHUNK ? s_m[k][qr] : a.part_ml[((size_t)slot_of(k) * RG + qr) * 2];
    };
    auto l_of = [&](int k) -> float {
      return np <= CHUNK ? s_l[k][qr] : a.part_ml[((size_t)slot_of(k) * RG + qr) * 2 + 1];
    };
    float M = neg_inf();
    for (int k = 0; k < np; ++k) M = fmaxf(M, m_of(k));
    float den = 0.f;
    for (int k = 0; k < np; ++k) {
      const float m = m_of(k);
      den += ((m == neg_inf()) ? 0.f : exp2_hw(m - M)) * l_of(k);
    }
    s_M[qr] = M;
    s_inv[qr] = 1.f / den;
  }
  for (int base = 0; base < nitems; base += PER * COMBINE_THREADS) {
    f32x4 acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < np; c0 += CHUNK) {
      const int nk = min(CHUNK, np - c0);
      const int nkp = (nk + KB - 1) / KB * KB;
      lds_barrier();  // s_M ready; the previous chunk's weights are no longer read
      for (int idx = threadIdx.x; idx < nkp * 64; idx += COMBINE_THREADS) {
        const int k = idx >> 6, qr = idx & 63;
        float f = 0.f;
        if (k < nk && qr < RG) {
          const float m = np <= CHUNK ? s_m[k][qr] : a.part_ml[((size_t)slot_of(c0 + k) * RG + qr) * 2];
          f = (m == neg_inf()) ? 0.f : exp2_hw(m - s_M[qr]);
        }
        s_f[k][qr] = f;
      }
      lds_barrier();
      for (int k0 = 0; k0 < nkp; k0 += KB) {
        f32x4 ov[PER][KB];
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int it = min(base + e * COMBINE_THREADS + (int)threadIdx.x, nitems - 1);
          const int qr = it / (D / 4), d4 = it - qr * (D / 4);
#pragma unroll
          for (int k = 0; k < KB; ++k)
            ov[e][k] = *reinterpret_cast<const f32x4*>(
                a.part_o + ((size_t)slot_of(c0 + min(k0 + k, nk - 1)) * RG + qr) * D + 4 * d4);
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int it = min(base + e * COMBINE_THREADS + (int)threadIdx.x, nitems - 1);
          const int qr = it / (D / 4);
#pragma unroll
          for (int k = 0; k < KB; ++k) acc[e] += s_f[k0 + k][qr] * ov[e][k];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int it = base + e * COMBINE_THREADS + threadIdx.x;
      if (it >= nitems) break;
      const int qr = it / (D / 4), d4 = it - qr * (D / 4);
      const float inv = s_inv[qr];
      const int r = qr / G, hg = qr - r * G;
      u32x2 wv;
      wv[0] = cvt_pk_bf16(acc[e][0] * inv, acc[e][1] * inv);
      wv[1] = cvt_pk_bf16(acc[e][2] * inv, acc[e][3] * inv);
      *reinterpret_cast<u32x2*>(out + (((size_t)b * R + r) * Hq + kvh * G + hg) * D + 4 * d4) = wv;
    }
  }
}

// ---------------------------------------------------------------- fp32 path
// Plain VALU kernel for float32 caches (the small parity configuration).  One workgroup
// per (request, query head); scores staged in LDS.  Same cache layouts, 4-byte elements.
constexpr int F32_MAX_TOKENS = 16384;

__global__ __launch_bounds__(THREADS) void attn_f32_kernel(const AttnLaunch a) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int R = a.R, G = a.G, Hq = a.Hq, Hkv = a.Hkv, D = a.D;
  const int kvh = h / G;
  const int L = min(max(a.ctx_lens[b], 0), a.max_ctx_len);
  const float* q = static_cast<const float*>(a.q);
  const float* kn = static_cast<const float*>(a.k_new);
  const float* vn = static_cast<const float*>(a.v_new);
  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  const int32_t* pt = a.page_table + (size_t)b * a.max_pages;
  const size_t tile = (size_t)PAGE * D;
  __shared__ float sc[F32_MAX_TOKENS];
  __shared__ float qs[128];
  __shared__ float red[THREADS / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  for (int r = 0; r < R; ++r) {
    const int n = L + r + 1;
    for (int d = threadIdx.x; d < D; d += THREADS)
      qs[d] = q[(((size_t)b * R + r) * Hq + h) * D + d];
    __syncthreads();
    float mx = -__builtin_inff();
    for (int j = threadIdx.x; j < n; j += THREADS) {
      float acc = 0.f;
      if (j < L) {
        const float* kt = kc + ((size_t)page_id(pt, j / PAGE, a.num_pages) * Hkv + kvh) * tile + (j % PAGE) * 8;
        for (int d = 0; d < D; ++d) acc += qs[d] * kt[(d / 8) * 128 + (d % 8)];
      } else {
        const float* kr = kn + (((size_t)b * R + (j - L)) * Hkv + kvh) * D;
        for (int d = 0; d < D; ++d) acc += qs[d] * kr[d];
      }
      acc *= a.scale;
      sc[j] = acc;
      mx = fmaxf(mx, acc);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float sum = 0.f;
    for (int j = threadIdx.x; j < n; j += THREADS) {
      const float e = expf(sc[j] - mx);
      sc[j] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    if (lane == 0) red[wave] = sum;
    __syncthreads();
    sum = (red[0] + red[1]) + (red[2] + red[3]);
    for (int d = threadIdx.x; d < D; d += THREADS) {
      float acc = 0.f;
      for (int j = 0; j < n; ++j) {
        float v;
        if (j < L) {
          const int slot = j % PAGE;
          v = vc[((size_t)page_id(pt, j / PAGE, a.num_pages) * Hkv + kvh) * tile + (d / 16) * 256 + (slot / 4) * 64 +
                 (d % 16) * 4 + slot % 4];
        } else {
          v = vn[(((size_t)b * R + (j - L)) * Hkv + kvh) * D + d];
        }
        acc += sc[j] * v;
      }
      float* out = static_cast<float*>(a.out);
      out[(((size_t)b * R + r) * Hq + h) * D + d] = acc / sum;
    }
    __syncthreads();
  }
  // append (one query head per KV head does it, after its reads of cached slots)
  if (h % G == 0) {
    float* kcw = static_cast<float*>(a.k_cache);
    float* vcw = static_cast<float*>(a.v_cache);
    for (int e = threadIdx.x; e < R * D; e += THREADS) {
      const int t = e / D, d = e - t * D;
      const int j = L + t, slot = j % PAGE;
      const size_t base = ((size_t)page_id(pt, j / PAGE, a.num_pages) * Hkv + kvh) * tile;
      const size_t src = (((size_t)b * R + t) * Hkv + kvh) * D + d;
      kcw[base + (d / 8) * 128 + slot * 8 + d % 8] = kn[src];
      vcw[base + (d / 16) * 256 + (slot / 4) * 64 + (d % 16) * 4 + slot % 4] = vn[src];
    }
  }
}

template <int D, int NQB>
hipError_t launch_shape(const AttnLaunch& a, hipStream_t s) {
  constexpr int NT = AttnShape<D, NQB>::THREADS;
  // one workgroup per resident slot (every slot gets an equal share of tiles), fewer
  // when the work is small; the slot count is queried once per device
  static std::atomic<int> slots_of_device[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int slots = (dev >= 0 && dev < 64) ? slots_of_device[dev].load(std::memory_order_relaxed) : 0;
  if (slots <= 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_bf16_kernel<D, NQB>, NT, 0);
    if (e != hipSuccess) return e;
    slots = max(1, per_cu) * max(1, cus);
    if (dev >= 0 && dev < 64) slots_of_device[dev].store(slots, std::memory_order_relaxed);
  }
  const long long units_max = (long long)a.B * a.Hkv * ((a.max_ctx_len + PAGE - 1) / PAGE + 1);
  long long W = slots;
  W = std::min<long long>(W, std::max<long long>(1, (units_max + 15) / 16));
  W = std::min<long long>(W, ATTN_MAX_WG);
  attn_bf16_kernel<D, NQB><<<(int)W, NT, 0, s>>>(a);
  attn_combine_kernel<D><<<(int)W, COMBINE_THREADS, 0, s>>>(a, (int)W);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bf16(const AttnLaunch& a, hipStream_t s) {
  switch ((a.R * a.G + 15) / 16) {
    case 1: return launch_shape<D, 1>(a, s);
    case 2: return launch_shape<D, 2>(a, s);
    case 3: return launch_shape<D, 3>(a, s);
    case 4: return launch_shape<D, 4>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attention(const AttnLaunch& a, hipStream_t s) {
  if (a.dtype == 0) {
    attn_f32_kernel<<<dim3(a.Hq, a.B), THREADS, 0, s>>>(a);
    return hipGetLastError();
  }
  if (a.D == 128) return launch_bf16<128>(a, s);
  if (a.D == 64) return launch_bf16<64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace isd
