// Strictly causal GQA attention of the 2N-1 strided block rows over a paged KV cache.
//
// Method (page 1 "為什麼 I-DLM 能在高並發下保持高效": 2N-1 queries per forward; page 1
// "實際部署：SGLang 整合" and page 5 "I-DLM-Methodik": strictly causal attention; page 1
// "實際部署：SGLang 整合" / page 5 "Serving (SGLang)": paged KV cache, paged-only kernel):
//   out[b,r,h] = softmax_j(scale q[b,r,h].k_j) v_j over tokens j <= ctx_len[b] + r.
//
// bf16 kernel, one workgroup per (request b, KV head, split of cached pages):
//   * The G query heads sharing a KV head and the R block rows form R*G query rows,
//     handled as 16-row MFMA blocks, so every K/V byte read serves all of them.
//   * Page layout is chosen for the MFMA operands: a K page [D/8][16][8] loads, one
//     1 KB-contiguous wave load per 32 dims, straight into the A operand of
//     S^T = K Q^T (16x16x32 bf16); a V page [D/16][4][16][4] loads (512 B per 16 dims)
//     straight into the A operand of O^T = V^T P^T (16x16x16 bf16).  S^T's accumulator
//     layout is exactly P^T's B-operand layout, and O^T keeps one query row per lane,
//     so the online softmax needs no data movement except a 4-lane max.
//   * The 4 waves take interleaved pages and software-prefetch the next one; their
//     partial (max, sum, O) states merge in LDS in a fixed order.
//   * The split holding the block also writes the block's K/V rows into their page
//     slots (after its own page loop) and attends to them from registers with the
//     causal mask.  No other workgroup reads those slots.
//   * A request whose cached pages fit one split writes its output directly; otherwise
//     each split writes an unnormalised partial (max, sum, O) and a small second kernel
//     merges them in split order.  No workgroup waits on or signals another.
#include "device.h"
#include "launch.h"

namespace isd {
namespace {

constexpr int PAGE = 16;
constexpr int THREADS = 256;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ int page_id(const int32_t* pt, int j, int num_pages) {
  return min(max(pt[j], 0), num_pages - 1);
}

// One 16-token tile (a cached page or the block) against every query block.
// MODE 0: all tokens valid.  MODE 1: tokens t < nvalid valid.  MODE 2: block tile,
// token t valid for query row q iff t <= q / G (causal, diagonal included).
template <int D, int NQB, int MODE>
__device__ __forceinline__ void attend_tile(const u32x4 (&kf)[D / 32], u32x2 (&vf)[D / 16],
                                            const u32x4 (&qf)[NQB][D / 32],
                                            f32x4 (&o)[NQB][D / 16], float (&m)[NQB],
                                            float (&l)[NQB], float scale_log2, int nvalid,
                                            int G, int lane) {
  const int l16 = lane & 15, g = lane >> 4;
  if (MODE == 1 && nvalid < PAGE) {
    // invalid slots may hold anything: zero their V so P = 0 never meets a non-finite V
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * g + i >= nvalid) {
          uint32_t w = vf[n][i >> 1];
          vf[n][i >> 1] = (i & 1) ? (w & 0x0000ffffu) : (w & 0xffff0000u);
        }
      }
    }
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 32; ++c) st = mfma16x16x32(kf[c], qf[qb][c], st);
    // st[i] = S^T[token 4g+i][query row 16 qb + l16]
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      bool ok = true;
      if (MODE == 1) ok = t < nvalid;
      if (MODE == 2) ok = t <= (qb * 16 + l16) / G;
      s[i] = ok ? st[i] * scale_log2 : neg_inf();
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m[qb], mx);
    const float alpha = (m[qb] == neg_inf()) ? 0.f : exp2_hw(m[qb] - mnew);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2_hw(s[i] - mnew);
    l[qb] = l[qb] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m[qb] = mnew;
    u32x2 pb;
    pb[0] = pack_bf16x2(p[0], p[1]);
    pb[1] = pack_bf16x2(p[2], p[3]);
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      o[qb][n] *= alpha;
      o[qb][n] = mfma16x16x16(vf[n], pb, o[qb][n]);
    }
  }
}

template <int D>
__device__ __forceinline__ void load_kv_page(const uint16_t* __restrict__ kt,
                                             const uint16_t* __restrict__ vt, int lane,
                                             u32x4 (&kf)[D / 32], u32x2 (&vf)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 32; ++c)
    kf[c] = *reinterpret_cast<const u32x4*>(kt + c * 512 + lane * 8);
#pragma unroll
  for (int n = 0; n < D / 16; ++n)
    vf[n] = *reinterpret_cast<const u32x2*>(vt + n * 256 + lane * 4);
}

template <int D, int NQB>
__device__ __forceinline__ void merge_state(f32x4 (&o)[NQB][D / 16], float (&m)[NQB],
                                            float (&l)[NQB], const float* om, const float* ol,
                                            const float* oo, int lane) {
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const float mb = om[qb * 64 + lane];
    if (mb == neg_inf()) continue;
    const float M = fmaxf(m[qb], mb);
    const float fa = (m[qb] == neg_inf()) ? 0.f : exp2_hw(m[qb] - M);
    const float fb = exp2_hw(mb - M);
    l[qb] = fa * l[qb] + fb * ol[qb * 64 + lane];
    m[qb] = M;
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        o[qb][n][i] = fa * o[qb][n][i] + fb * oo[((qb * (D / 16) + n) * 4 + i) * 64 + lane];
  }
}

template <int D, int NQB>
__device__ __forceinline__ void stash_state(const f32x4 (&o)[NQB][D / 16], const float (&m)[NQB],
                                            const float (&l)[NQB], float* om, float* ol,
                                            float* oo, int lane) {
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    om[qb * 64 + lane] = m[qb];
    ol[qb * 64 + lane] = l[qb];
#pragma unroll
    for (int n = 0; n < D / 16; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) oo[((qb * (D / 16) + n) * 4 + i) * 64 + lane] = o[qb][n][i];
  }
}

// Splits of the cached pages: nsplit = ceil(ceil(L/16) / pages_per_split), at least one.
__device__ __forceinline__ int split_count(int L, int pps) {
  const int ncp = (L + PAGE - 1) / PAGE;
  return ncp == 0 ? 1 : (ncp + pps - 1) / pps;
}

template <int D, int NQB>
__global__ __launch_bounds__(THREADS, (NQB <= 2) ? 2 : 1) void attn_bf16_kernel(const AttnLaunch a) {
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  // device-side preconditions are clamped so a violation cannot address outside buffers
  const int L = min(max(a.ctx_lens[b], 0), a.max_ctx_len);
  const int ncp = (L + PAGE - 1) / PAGE;
  const int pps = a.pages_per_split;
  const int nsplit = split_count(L, pps);
  if (s >= nsplit) return;

  const int R = a.R, G = a.G, Hq = a.Hq, Hkv = a.Hkv, RG = R * G;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  const bool last = (s == nsplit - 1);
  const int p0 = s * pps, p1 = min(ncp, p0 + pps);

  const uint16_t* __restrict__ q = static_cast<const uint16_t*>(a.q);
  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  const int32_t* __restrict__ pt = a.page_table + (size_t)b * a.max_pages;
  const size_t tile = (size_t)PAGE * D;

  // This wave's pages p0 + wave + 4i, i < npw: their physical ids, one per lane, read
  // back as scalars so no page-table load sits between two page loads.
  const int npw = (p1 - p0 - wave + 3) / 4;
  const int my_id = (lane < npw) ? page_id(pt, p0 + wave + 4 * lane, a.num_pages) : 0;

  // Q^T fragments (B operand of S^T = K Q^T): query row 16 qb + l16, dims 32c + 8g ..
  u32x4 qf[NQB][D / 32];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qr = qb * 16 + l16;
    if (qr < RG) {
      const int r = qr / G, hg = qr - r * G;
      const uint16_t* qp = q + (((size_t)b * R + r) * Hq + kvh * G + hg) * D + 8 * g;
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qf[qb][c] = *reinterpret_cast<const u32x4*>(qp + 32 * c);
    } else {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) qf[qb][c] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  f32x4 o[NQB][D / 16];
  float m[NQB], l[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = neg_inf();
    l[qb] = 0.f;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) o[qb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- cached pages, two in flight: buffers A (even i) and B (odd i)
  auto tile_base = [&](int i) -> size_t {
    const int pid = __builtin_amdgcn_readlane(my_id, i);
    return ((size_t)pid * Hkv + kvh) * tile;
  };
  u32x4 kA[D / 32], kB[D / 32];
  u32x2 vA[D / 16], vB[D / 16];
  if (npw > 0) { const size_t t0 = tile_base(0); load_kv_page<D>(kc + t0, vc + t0, lane, kA, vA); }
  if (npw > 1) { const size_t t1 = tile_base(1); load_kv_page<D>(kc + t1, vc + t1, lane, kB, vB); }
  for (int i = 0; i < npw; i += 2) {
    attend_tile<D, NQB, 1>(kA, vA, qf, o, m, l, scale_log2, L - (p0 + wave + 4 * i) * PAGE, G, lane);
    if (i + 2 < npw) { const size_t t = tile_base(i + 2); load_kv_page<D>(kc + t, vc + t, lane, kA, vA); }
    if (i + 1 < npw) {
      attend_tile<D, NQB, 1>(kB, vB, qf, o, m, l, scale_log2, L - (p0 + wave + 4 * (i + 1)) * PAGE, G, lane);
      if (i + 3 < npw) { const size_t t = tile_base(i + 3); load_kv_page<D>(kc + t, vc + t, lane, kB, vB); }
    }
  }

  // ---- the block's own rows (last split only), taken from k_new / v_new
  const uint16_t* __restrict__ kn_ = static_cast<const uint16_t*>(a.k_new);
  const uint16_t* __restrict__ vn_ = static_cast<const uint16_t*>(a.v_new);
  const size_t rstride = (size_t)Hkv * D;  // between consecutive block rows
  const size_t blk = ((size_t)b * R * Hkv + kvh) * D;
  if (last && wave == ((p1 - p0) & 3)) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c)
      kA[c] = (l16 < R) ? *reinterpret_cast<const u32x4*>(kn_ + blk + l16 * rstride + 32 * c + 8 * g)
                        : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * g + i;
        h[i] = (t < R) ? vn_[blk + t * rstride + 16 * n + l16] : 0u;
      }
      vA[n][0] = h[0] | (h[1] << 16);
      vA[n][1] = h[2] | (h[3] << 16);
    }
    attend_tile<D, NQB, 2>(kA, vA, qf, o, m, l, scale_log2, 0, G, lane);
  }

  // ---- merge the four waves in LDS: (w0 + w2) + (w1 + w3)
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    l[qb] += __shfl_xor(l[qb], 16);
    l[qb] += __shfl_xor(l[qb], 32);
  }
  __shared__ float sm[2][NQB * 64], sl[2][NQB * 64];
  __shared__ float so[2][NQB * (D / 16) * 4 * 64];
  if (wave >= 2) stash_state<D, NQB>(o, m, l, sm[wave - 2], sl[wave - 2], so[wave - 2], lane);
  __syncthreads();
  if (wave < 2) merge_state<D, NQB>(o, m, l, sm[wave], sl[wave], so[wave], lane);
  __syncthreads();
  if (wave == 1) stash_state<D, NQB>(o, m, l, sm[0], sl[0], so[0], lane);
  __syncthreads();

  // ---- append the block rows to their page slots (after every read of this split's pages)
  if (last) {
    uint16_t* kcw = static_cast<uint16_t*>(a.k_cache);
    uint16_t* vcw = static_cast<uint16_t*>(a.v_cache);
    // K: 16-byte units of 8 dims; V: single elements
    for (int e = threadIdx.x; e < R * (D / 8); e += THREADS) {
      const int t = e / (D / 8), d8 = e - t * (D / 8);
      const int j = L + t;
      const size_t base = ((size_t)page_id(pt, j / PAGE, a.num_pages) * Hkv + kvh) * tile;
      *reinterpret_cast<u32x4*>(kcw + base + d8 * 128 + (j % PAGE) * 8) =
          *reinterpret_cast<const u32x4*>(kn_ + blk + t * rstride + d8 * 8);
    }
    for (int e = threadIdx.x; e < R * D; e += THREADS) {
      const int t = e / D, d = e - t * D;
      const int j = L + t, slot = j % PAGE;
      const size_t base = ((size_t)page_id(pt, j / PAGE, a.num_pages) * Hkv + kvh) * tile;
      vcw[base + (d / 16) * 256 + (slot / 4) * 64 + (d % 16) * 4 + slot % 4] =
          vn_[blk + t * rstride + d];
    }
  }

  if (wave != 0) return;
  merge_state<D, NQB>(o, m, l, sm[0], sl[0], so[0], lane);
  if (nsplit == 1) {
    uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qr = qb * 16 + l16;
      if (qr >= RG) continue;
      const int r = qr / G, hg = qr - r * G;
      const float inv = 1.f / l[qb];
      uint16_t* op = out + (((size_t)b * R + r) * Hq + kvh * G + hg) * D + 4 * g;
#pragma unroll
      for (int n = 0; n < D / 16; ++n) {
        u32x2 w;
        w[0] = pack_bf16x2(o[qb][n][0] * inv, o[qb][n][1] * inv);
        w[1] = pack_bf16x2(o[qb][n][2] * inv, o[qb][n][3] * inv);
        *reinterpret_cast<u32x2*>(op + 16 * n) = w;
      }
    }
  } else {
    // unnormalised partial state of this split; the combine kernel merges them
    const size_t slot = ((size_t)b * Hkv + kvh) * a.splits_max + s;
    float* po = a.part_o + slot * RG * D;
    float* pml = a.part_ml + slot * RG * 2;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qr = qb * 16 + l16;
      if (qr >= RG) continue;
#pragma unroll
      for (int n = 0; n < D / 16; ++n)
        *reinterpret_cast<f32x4*>(po + (size_t)qr * D + 16 * n + 4 * g) = o[qb][n];
      if (g == 0) {
        pml[qr * 2] = m[qb];
        pml[qr * 2 + 1] = l[qb];
      }
    }
  }
}

// Merge the split partials of one (request, KV head) in split order.  Only requests whose
// cached pages span more than one split have work here.
constexpr int COMBINE_BATCH = 8;

template <int D>
__global__ __launch_bounds__(THREADS) void attn_combine_kernel(const AttnLaunch a) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int L = min(max(a.ctx_lens[b], 0), a.max_ctx_len);
  const int nsplit = split_count(L, a.pages_per_split);
  if (nsplit <= 1) return;
  const int R = a.R, G = a.G, Hq = a.Hq, RG = R * G;
  const size_t slot0 = ((size_t)b * a.Hkv + kvh) * a.splits_max;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  for (int it = threadIdx.x; it < RG * (D / 4); it += THREADS) {
    const int qr = it / (D / 4), d4 = it - qr * (D / 4);
    float M = neg_inf();
    for (int s0 = 0; s0 < nsplit; s0 += COMBINE_BATCH) {
      float mv[COMBINE_BATCH];
#pragma unroll
      for (int k = 0; k < COMBINE_BATCH; ++k)
        mv[k] = (s0 + k < nsplit) ? a.part_ml[((slot0 + s0 + k) * RG + qr) * 2] : neg_inf();
#pragma unroll
      for (int k = 0; k < COMBINE_BATCH; ++k) M = fmaxf(M, mv[k]);
    }
    f32x4 num = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += COMBINE_BATCH) {
      f32x4 ov[COMBINE_BATCH];
      float mv[COMBINE_BATCH], lv[COMBINE_BATCH];
#pragma unroll
      for (int k = 0; k < COMBINE_BATCH; ++k) {
        if (s0 + k < nsplit) {
          const size_t sl = slot0 + s0 + k;
          ov[k] = *reinterpret_cast<const f32x4*>(a.part_o + (sl * RG + qr) * D + 4 * d4);
          mv[k] = a.part_ml[(sl * RG + qr) * 2];
          lv[k] = a.part_ml[(sl * RG + qr) * 2 + 1];
        }
      }
#pragma unroll
      for (int k = 0; k < COMBINE_BATCH; ++k) {
        if (s0 + k < nsplit) {
          const float f = exp2_hw(mv[k] - M);
          den += f * lv[k];
          num += f * ov[k];
        }
      }
    }
    const float inv = 1.f / den;
    const int r = qr / G, hg = qr - r * G;
    u32x2 w;
    w[0] = pack_bf16x2(num[0] * inv, num[1] * inv);
    w[1] = pack_bf16x2(num[2] * inv, num[3] * inv);
    *reinterpret_cast<u32x2*>(out + (((size_t)b * R + r) * Hq + kvh * G + hg) * D + 4 * d4) = w;
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

template <int D>
hipError_t launch_bf16(const AttnLaunch& a, hipStream_t s) {
  const dim3 grid(a.splits_max, a.Hkv, a.B);
  const int nqb = (a.R * a.G + 15) / 16;
  switch (nqb) {
    case 1: attn_bf16_kernel<D, 1><<<grid, THREADS, 0, s>>>(a); break;
    case 2: attn_bf16_kernel<D, 2><<<grid, THREADS, 0, s>>>(a); break;
    case 3: attn_bf16_kernel<D, 3><<<grid, THREADS, 0, s>>>(a); break;
    case 4: attn_bf16_kernel<D, 4><<<grid, THREADS, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  if (a.splits_max > 1) attn_combine_kernel<D><<<dim3(a.Hkv, a.B), THREADS, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

int attention_pages_per_split(int B, int Hkv, int max_ctx_len, int R) {
  (void)B; (void)Hkv; (void)max_ctx_len; (void)R;
  if (const char* e = getenv("ISD_ATTN_PPS")) {
    const int v = atoi(e);
    if (v >= 4 && v <= 4096) return v;
  }
  return 32;
}

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
