// Vocab-wide verification of one ISD step.
//
// Method: [MASK] rows propose from q, clean rows verify earlier proposals against the
// causal anchor p, and a proposal x is kept with probability min(1, p(x)/q(x)), which
// leaves the AR distribution unchanged (「首次超越 AR 模型」 "I-DLM 如何解決這些問題"; 「I-DLM – introspektive Diffusion Language Models」
// "Inference & ISD").  Proposals are argmax ids (「首次超越 AR 模型」 "實際部署：SGLang 整合").  On a
// rejection the next token comes from the normalised residual max(0, p - q~).
//
// Kernels (HBM-streaming reductions over the vocabulary; no MFMA):
//   stats    per 16384-entry chunk of each row: the chunk max M of the raw logits, the
//            lowest id holding it, the chunk reference K = M log2(e)/T rounded to fp32,
//            and for every 1024-entry sub-chunk the sum of 2^(l log2(e)/T - K).  K is
//            used exactly everywhere downstream, so every element weight has one rounding
//            (the fma's) and no chunk carries a bias.  A resident grid walks the chunks
//            with the next one's loads in flight (one workgroup per chunk when rows are not
//            16-byte aligned).  It can cover a subset of each request's rows: in front of
//            the LM head it takes only the draft rows, and the LM head's epilogue supplies
//            the same records for the rows it computes.
//   walk_residual  grid (chunks + 1, request) with sampled drafts, (1, request) with
//            argmax drafts.  Every workgroup takes the request's walk from the chunk
//            statistics in fp64 (row max, argmax, normaliser, acceptance); the last one
//            writes the outputs and takes each inverse-CDF draw from an fp64 prefix over
//            sub-chunk sums plus one re-read sub-chunk; the others sum max(0, p - q~) over
//            their chunk's sub-chunks when the request's sampled draft was rejected.
//   locate   one wave per such request: prefix over those sums, re-read one sub-chunk.
// Argmax drafts need no residual sums: the residual is p with the draft removed, whose
// sub-chunk sums the stats pass already has.
// In a decoding loop a step's draft rows are the previous step's proposal rows N..2N-2:
// the stats pass can hand those rows' records on (qnext), and the next call can take its
// draft rows' records from them (qprev) instead of reducing draft_logits again.
#include <limits.h>

#include <atomic>

#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace isd {
namespace {

constexpr int THREADS = 256;
constexpr int MAX_RR = 22;    // 2N-1 + N-1 rows for N <= 8
constexpr int MAX_SV = 64;    // vocab <= 2^20
constexpr int RPB = 3;        // rows per wave per batch of loads in the walk
constexpr int CSL = 3;        // sub-chunk sums per lane per row held in registers there
constexpr int STASH = 4096;   // sub-chunk sums the walk keeps in LDS
constexpr int RSPLIT = 1;     // residual workgroups per stats chunk (2 and 4 measured slower)

template <typename T> struct VecOf;
template <> struct VecOf<uint16_t> { static constexpr int n = 8; };
template <> struct VecOf<float> { static constexpr int n = 4; };
template <typename T> constexpr int kRounds = VCHUNK / (THREADS * VecOf<T>::n);

__device__ __forceinline__ float to_f(uint16_t h) { return bf16_to_f32(h); }
__device__ __forceinline__ float to_f(float f) { return f; }

// Weight of a logit against a chunk reference K: 2^(l c2 - K), c2 = log2(e)/T, one
// rounding (the fma).  Every kernel computes element weights through this function, so
// a re-read element gets exactly the weight the stats pass summed.
__device__ __forceinline__ float rel_weight(float l, float K, float c2) {
  return exp2_hw(fmaf(l, c2, -K));
}

// Residual weight max(0, p - q~) in fp32 against each row's reference; 1/Z is applied as
// a hi + lo pair so its rounding does not bias p against q~.
__device__ __forceinline__ float residual_weight(float lp, float lq, const WalkState& st, float c2) {
  const float ep = rel_weight(lp, st.kp, c2);
  const float eq = rel_weight(lq, st.kq, c2);
  const float p = fmaf(ep, st.izp_hi, ep * st.izp_lo);
  const float q = fmaf(eq, st.izq_hi, eq * st.izq_lo);
  return fmaxf(0.f, p - q);
}

template <typename T>
__device__ __forceinline__ const T* row_ptr(const VerifyLaunch& v, int b, int rr) {
  if (rr < v.R) return static_cast<const T*>(v.logits) + ((size_t)b * v.R + rr) * v.V;
  return static_cast<const T*>(v.draft) + ((size_t)b * (v.N - 1) + (rr - v.R)) * v.V;
}

// Load one chunk of a row into registers: thread t, round k holds entries
// base + k*THREADS*VE + t*VE + [0, VE).  Entries past V read as -inf.
template <typename T, bool VEC, int ROUNDS = kRounds<T>>
__device__ __forceinline__ void load_chunk(const T* __restrict__ row, int V, int base, int tid,
                                           float (&x)[ROUNDS * VecOf<T>::n]) {
  constexpr int VE = VecOf<T>::n;
#pragma unroll
  for (int k = 0; k < ROUNDS; ++k) {
    const int e0 = base + k * THREADS * VE + tid * VE;
    if (VEC && e0 + VE <= V) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + e0);
      if constexpr (VE == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[k * VE + 2 * i] = bf16_lo(w[i]);
          x[k * VE + 2 * i + 1] = bf16_hi(w[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[k * VE + i] = __uint_as_float(w[i]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < VE; ++j)
        x[k * VE + j] = (e0 + j < V) ? to_f(row[e0 + j]) : -__builtin_inff();
    }
  }
}

// Per-thread round sums -> sub-chunk sums, in a fixed order: the round sums go to LDS,
// then 16 lanes per sub-chunk add their consecutive share and reduce in their 16-lane group.
template <typename T, int ROUNDS = kRounds<T>>
__device__ __forceinline__ void sub_sums(const float (&s)[ROUNDS], float* lds, float* out,
                                         int chunk, int nsub, int tid, float* out2 = nullptr) {
  constexpr int VE = VecOf<T>::n;
  constexpr int TPS = VSUB / VE;              // threads covering one sub-chunk in a round
  constexpr int SPR = THREADS / TPS;          // sub-chunks per round
  constexpr int PER = TPS / 16;               // round sums per lane
  constexpr int SUBS = ROUNDS * SPR;          // sub-chunks of this chunk
#pragma unroll
  for (int k = 0; k < ROUNDS; ++k) lds[k * THREADS + tid] = s[k];
  __syncthreads();
  const int j = tid >> 4, p = tid & 15;       // sub-chunk of this chunk, lane in its group
  if (j >= SUBS) return;
  const float* src = lds + (j / SPR) * THREADS + (j % SPR) * TPS + p * PER;
  float v = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) v += src[i];
  v = row16_sum(v);
  const int sub = chunk * SUBS + j;
  if (p == 0 && sub < nsub) {
    out[sub] = v;
    if (out2) out2[sub] = v;
  }
}

// Chunk maxima, chunk references and sub-chunk sums of row rr of request b: the draft rows'
// come from the previous step when it carried them, every other row's from this call.
struct RowRecords {
  const float* cmax;
  const float* cref;
  const float* csub;
};

__device__ __forceinline__ RowRecords row_records(const VerifyLaunch& v, int b, int rr) {
  if (v.qprev && rr >= v.R) {
    const float* q = v.qprev + ((size_t)b * (v.N - 1) + (rr - v.R)) * v.QS;
    return RowRecords{q, q + v.SV, q + 2 * v.SV};
  }
  const size_t rowid = (size_t)b * v.RR + rr;
  return RowRecords{v.cmax + rowid * v.SV, v.cref + rowid * v.SV, v.csub + rowid * v.NSUB};
}

// Where this call's row rr of request b is also written for the next step, or null: rows
// N .. 2N-2 (the proposal rows whose samples become the next step's drafts).
__device__ __forceinline__ float* carried_row(const VerifyLaunch& v, int b, int rr) {
  if (!v.qnext || rr < v.N || rr >= v.R) return nullptr;
  return v.qnext + ((size_t)b * (v.N - 1) + (rr - v.N)) * v.QS;
}

// ---------------------------------------------------------------- stats pass
template <typename T, bool VEC>
__global__ __launch_bounds__(THREADS) void stats_kernel(const VerifyLaunch v) {
  constexpr int VE = VecOf<T>::n;
  const int chunk = blockIdx.x, rr = v.srow0 + blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = chunk * VCHUNK;
  const T* __restrict__ row = row_ptr<T>(v, b, rr);
  float x[VCHUNK / THREADS];
  load_chunk<T, VEC>(row, v.V, base, tid, x);

  __shared__ float red[4];
  __shared__ int redi[4];
  __shared__ float lds[kRounds<T> * THREADS];
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < VCHUNK / THREADS; ++i) mx = fmaxf(mx, x[i]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float K = M * v.c2;

  const bool proposal = rr >= v.N - 1 && rr < v.R;
  if (proposal) {
    int arg = INT_MAX;
#pragma unroll
    for (int k = 0; k < kRounds<T>; ++k)
#pragma unroll
      for (int j = 0; j < VE; ++j)
        if (x[k * VE + j] == M && arg == INT_MAX) arg = base + k * THREADS * VE + tid * VE + j;
    arg = wave_min_i(arg);
    if (lane == 0) redi[wave] = arg;
  }
  float s[kRounds<T>];
#pragma unroll
  for (int k = 0; k < kRounds<T>; ++k) {
    // started from the first weight: 0 + w = w for every weight (never -0), and the
    // compiler cannot drop an add of +0 itself
    float acc = rel_weight(x[k * VE], K, v.c2);
#pragma unroll
    for (int j = 1; j < VE; ++j) acc += rel_weight(x[k * VE + j], K, v.c2);
    s[k] = acc;
  }
  const size_t rowid = (size_t)b * v.RR + rr;
  float* carry = carried_row(v, b, rr);
  sub_sums<T>(s, lds, v.csub + rowid * v.NSUB, chunk, v.NSUB, tid, carry ? carry + 2 * v.SV : nullptr);
  if (tid == 0) {
    v.cmax[rowid * v.SV + chunk] = M;
    v.cref[rowid * v.SV + chunk] = K;
    v.cidx[rowid * v.SV + chunk] =
        proposal ? min(min(redi[0], redi[1]), min(redi[2], redi[3])) : INT_MAX;
    if (carry) {
      carry[chunk] = M;
      carry[v.SV + chunk] = K;
    }
  }
}

// The same statistics with 16-byte aligned rows, from a resident grid: workgroup w takes
// the (row, chunk) units w, w + W, ... and keeps the next unit's loads in flight while it
// reduces the current one.  Units are numbered (b RR + rr) SV + chunk.
// Unit -> (request, row, chunk): units are numbered (b snrow + (rr - srow0)) SV + chunk.
__device__ __forceinline__ void decode_unit(const VerifyLaunch& v, int unit, int& b, int& rr, int& chunk) {
  const int rl = unit / v.SV;
  chunk = unit - rl * v.SV;
  b = rl / v.snrow;
  rr = v.srow0 + (rl - b * v.snrow);
}

template <typename T>
struct RawChunk {
  u32x4 w[kRounds<T>];  // thread t, round k: 16 bytes at base + k THREADS VE + t VE
};

template <typename T>
__device__ __forceinline__ void load_raw(const VerifyLaunch& v, int unit, int tid, RawChunk<T>& r) {
  constexpr int VE = VecOf<T>::n;
  int b, rr, chunk;
  decode_unit(v, unit, b, rr, chunk);
  const T* __restrict__ row = row_ptr<T>(v, b, rr);
  const int base = chunk * VCHUNK;
#pragma unroll
  for (int k = 0; k < kRounds<T>; ++k) {
    const int e0 = base + k * THREADS * VE + tid * VE;
    // past the row's end: load its first 16 bytes (in bounds), replaced by -inf below;
    // non-temporal: the stats pass reads each logit once
    r.w[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + (e0 < v.V ? e0 : 0)));
  }
}

template <typename T>
__device__ __forceinline__ void stats_of_unit(const VerifyLaunch& v, int unit, int tid,
                                              const RawChunk<T>& r, float* red, int* redi, float* lds) {
  constexpr int VE = VecOf<T>::n;
  constexpr int NE = VCHUNK / THREADS;
  const int lane = tid & 63, wave = tid >> 6;
  int b, rr, chunk;
  decode_unit(v, unit, b, rr, chunk);
  const int rowid = b * v.RR + rr;
  const int base = chunk * VCHUNK;
  float* carry = carried_row(v, b, rr);
  float x[NE];
#pragma unroll
  for (int k = 0; k < kRounds<T>; ++k) {
    if constexpr (VE == 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[k * VE + 2 * i] = bf16_lo(r.w[k][i]);
        x[k * VE + 2 * i + 1] = bf16_hi(r.w[k][i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[k * VE + i] = __uint_as_float(r.w[k][i]);
    }
  }
  if (base + VCHUNK > v.V) {  // the row's last chunk: entries past V read as -inf
#pragma unroll
    for (int k = 0; k < kRounds<T>; ++k)
      if (base + k * THREADS * VE + tid * VE >= v.V)
#pragma unroll
        for (int j = 0; j < VE; ++j) x[k * VE + j] = -__builtin_inff();
  }
  float mloc = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < NE; ++i) mloc = fmaxf(mloc, x[i]);
  const float mw = wave_max(mloc);
  if (lane == 0) red[wave] = mw;
  lds_barrier();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float K = M * v.c2;
  const bool proposal = rr >= v.N - 1 && rr < v.R;
  if (proposal) {
    // lowest id holding M: only lanes whose own maximum is M look for it
    int arg = INT_MAX;
    if (mloc == M) {
#pragma unroll
      for (int k = kRounds<T> - 1; k >= 0; --k)
#pragma unroll
        for (int j = VE - 1; j >= 0; --j)
          if (x[k * VE + j] == M) arg = base + k * THREADS * VE + tid * VE + j;
    }
    arg = wave_min_i(arg);
    if (lane == 0) redi[wave] = arg;
  }
  float s[kRounds<T>];
#pragma unroll
  for (int k = 0; k < kRounds<T>; ++k) {
    // started from the first weight: 0 + w = w for every weight (never -0), and the
    // compiler cannot drop an add of +0 itself
    float acc = rel_weight(x[k * VE], K, v.c2);
#pragma unroll
    for (int j = 1; j < VE; ++j) acc += rel_weight(x[k * VE + j], K, v.c2);
    s[k] = acc;
  }
  // sub-chunk sums (as sub_sums, with an LDS-only barrier)
  {
    constexpr int TPS = VSUB / VE, SPR = THREADS / TPS, PER = TPS / 16;
#pragma unroll
    for (int k = 0; k < kRounds<T>; ++k) lds[k * THREADS + tid] = s[k];
    lds_barrier();
    const int j = tid >> 4, p = tid & 15;
    const float* src = lds + (j / SPR) * THREADS + (j % SPR) * TPS + p * PER;
    float vv = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) vv += src[i];
    vv = row16_sum(vv);
    const int sub = chunk * VCHUNK_SUBS + j;
    if (p == 0 && sub < v.NSUB) {
      v.csub[(size_t)rowid * v.NSUB + sub] = vv;
      if (carry) carry[2 * v.SV + sub] = vv;
    }
  }
  if (tid == 0) {
    v.cmax[(size_t)rowid * v.SV + chunk] = M;
    v.cref[(size_t)rowid * v.SV + chunk] = K;
    v.cidx[(size_t)rowid * v.SV + chunk] = proposal ? min(min(redi[0], redi[1]), min(redi[2], redi[3])) : INT_MAX;
    if (carry) {
      carry[chunk] = M;
      carry[v.SV + chunk] = K;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(THREADS) void stats_resident_kernel(const VerifyLaunch v, int U) {
  __shared__ float red[4];
  __shared__ int redi[4];
  __shared__ float lds[kRounds<T> * THREADS];
  const int tid = threadIdx.x, W = gridDim.x, w = blockIdx.x;
  const int n = (U - w + W - 1) / W;  // units of this workgroup (>= 1: W <= U)
  RawChunk<T> ra, rb;
  load_raw<T>(v, w, tid, ra);
  int i = 0;
  for (; i + 2 < n; i += 2) {
    load_raw<T>(v, w + (i + 1) * W, tid, rb);
    __builtin_amdgcn_sched_barrier(0);
    stats_of_unit<T>(v, w + i * W, tid, ra, red, redi, lds);
    load_raw<T>(v, w + (i + 2) * W, tid, ra);
    __builtin_amdgcn_sched_barrier(0);
    stats_of_unit<T>(v, w + (i + 1) * W, tid, rb, red, redi, lds);
  }
  if (i + 1 < n) {
    load_raw<T>(v, w + (i + 1) * W, tid, rb);
    __builtin_amdgcn_sched_barrier(0);
    stats_of_unit<T>(v, w + i * W, tid, ra, red, redi, lds);
    stats_of_unit<T>(v, w + (i + 1) * W, tid, rb, red, redi, lds);
  } else {
    stats_of_unit<T>(v, w + i * W, tid, ra, red, redi, lds);
  }
}

// ---------------------------------------------------------------- wave-wide locate
// Smallest sub-chunk j with prefix(0..j) > target, weights from subw(j).  Returns the
// prefix before j in `pre`.  If none (rounding at the very end), the last sub-chunk
// with positive weight.
template <class SubW>
__device__ int find_sub(SubW subw, int nsub, double target, int lane, double& pre) {
  const int S = (nsub + 63) / 64;
  const int j0 = min(nsub, lane * S), j1 = min(nsub, j0 + S);
  double part = 0.0;
  for (int j = j0; j < j1; ++j) part += subw(j);
  const double incl = wave_incl_scan_d(part, lane);
  const double excl = incl - part;
  const unsigned long long hit = __ballot(incl > target);
  int jstar = -1;
  double p = 0.0;
  if (hit) {
    const int src = __ffsll((long long)hit) - 1;
    if (lane == src) {
      double acc = excl;
      jstar = j1 - 1;
      for (int j = j0; j < j1; ++j) {
        const double w = subw(j);
        if (acc + w > target) { jstar = j; break; }
        acc += w;
      }
      p = acc;
    }
    jstar = __shfl(jstar, src);
    p = __shfl(p, src);
  } else {
    int last = -1;
    for (int j = j0; j < j1; ++j)
      if (subw(j) > 0.0) last = j;
    // lanes own ascending ranges: the highest lane with a positive sub-chunk wins
    const unsigned long long has = __ballot(last >= 0);
    const int src = has ? 63 - __clzll((long long)has) : 0;
    jstar = __shfl(last, src);
    if (jstar < 0) jstar = 0;
    double acc = 0.0;
    for (int j = lane; j < jstar; j += 64) acc += subw(j);
    p = wave_sum_d(acc);
  }
  pre = p;
  return jstar;
}

// Lane l's 16 consecutive entries k0 = e0 + 16 l .. k0 + 15 of a row (entries from
// `end` on read as -inf); one or two 16-byte loads per lane when rows are 16-byte aligned.
template <typename T, bool VEC>
__device__ __forceinline__ void load16(const T* __restrict__ row, int k0, int end, float (&x)[16]) {
  constexpr int VE = VecOf<T>::n;
  if (VEC && k0 + 16 <= end) {
#pragma unroll
    for (int q = 0; q < 16 / VE; ++q) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(row + k0 + q * VE);
      if constexpr (VE == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[q * 8 + 2 * i] = bf16_lo(w[i]);
          x[q * 8 + 2 * i + 1] = bf16_hi(w[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[q * 4 + i] = __uint_as_float(w[i]);
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < 16; ++t) x[t] = (k0 + t < end) ? to_f(row[k0 + t]) : -__builtin_inff();
  }
}

// Smallest entry k = k0 + t (lane l holds k0 = e0 + 16 l with weights w16[t]) with
// pre + prefix(e0..k) > target.  Fallback: the last entry with positive weight, else e0.
__device__ int find_in16(const double (&w16)[16], int e0, double pre, double target, int lane) {
  const int k0 = e0 + lane * 16;
  double s = 0.0;
#pragma unroll
  for (int t = 0; t < 16; ++t) s += w16[t];
  const double incl = wave_incl_scan_d(s, lane);
  const unsigned long long hit = __ballot(pre + incl > target);
  int ans = -1;
  if (hit) {
    const int src = __ffsll((long long)hit) - 1;
    if (lane == src) {
      double acc = pre + (incl - s);
      for (int t = 0; t < 16; ++t) {
        if (w16[t] > 0.0) ans = k0 + t;
        acc += w16[t];
        if (w16[t] > 0.0 && acc > target) break;
      }
    }
    ans = __shfl(ans, src);
  } else {
    int last = -1;
    for (int t = 0; t < 16; ++t)
      if (w16[t] > 0.0) last = k0 + t;
    const unsigned long long has = __ballot(last >= 0);
    const int src = has ? 63 - __clzll((long long)has) : 0;
    ans = __shfl(last, src);
  }
  return ans < 0 ? e0 : ans;
}

// Inverse-CDF draw from row rr in units of 2^(l c2 - Kmax), optionally with one id
// removed.  fac[c] = 2^(K_c - Kmax) for chunk c of this row.
template <typename T, bool VEC>
__device__ int sample_row(const VerifyLaunch& v, int b, int rr, const double* fac, double target,
                          int excl, int lane, const float* cs_stash = nullptr) {
  const T* __restrict__ row = row_ptr<T>(v, b, rr);
  const size_t rowid = (size_t)b * v.RR + rr;
  const float* __restrict__ cr = v.cref + rowid * v.SV;
  const float* cs = cs_stash ? cs_stash : v.csub + rowid * v.NSUB;
  double wex = 0.0;
  int exsub = -1;
  if (excl >= 0) {
    const int c = excl / VCHUNK;
    wex = (double)rel_weight(to_f(row[excl]), cr[c], v.c2) * fac[c];
    exsub = excl / VSUB;
  }
  auto subw = [&](int j) -> double {
    double w = (double)cs[j] * fac[j / VCHUNK_SUBS];
    if (j == exsub) w = fmax(0.0, w - wex);
    return w;
  };
  double pre;
  const int js = find_sub(subw, v.NSUB, target, lane, pre);
  const int c = js / VCHUNK_SUBS;
  const float Kc = cr[c];
  const double fc = fac[c];
  const int e0 = js * VSUB, end = min(e0 + VSUB, v.V);
  float x[16];
  load16<T, VEC>(row, e0 + lane * 16, end, x);
  double w16[16];
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int k = e0 + lane * 16 + t;
    w16[t] = (k < end && k != excl) ? (double)rel_weight(x[t], Kc, v.c2) * fc : 0.0;
  }
  return find_in16(w16, e0, pre, target, lane);
}

// ---------------------------------------------------------------- walk + residual
// Grid (residual chunks + 1, requests) with sampled drafts, (1, requests) with argmax
// drafts; a residual chunk is 1/RSPLIT of a stats chunk.  Every workgroup takes its
// request's acceptance walk from the row statistics (a few KB, the same arithmetic in
// each); the last workgroup of a request writes the walk's outputs and takes the
// inverse-CDF draws, and with sampled drafts the others each sum their chunk of the
// residual max(0, p - q~) of a rejecting request.
// Workgroups of one request per launch: the residual chunks, then the lead.
__host__ __device__ inline int walk_groups(const VerifyLaunch& v) {
  return v.draft ? (v.NSUB + VCHUNK_SUBS / RSPLIT - 1) / (VCHUNK_SUBS / RSPLIT) + 1 : 1;
}

// One-dimensional grid of XCDS * ceil(B / XCDS) * walk_groups workgroups.  Workgroups are
// dispatched to the XCDs round-robin by id, so id = x + XCDS * slot runs on XCD x; request b
// takes XCD b % XCDS and slots (b / XCDS) * groups + chunk there, so all its workgroups share
// one L2 for the records and the gathers they all read.  Ids past the last request exit.
template <typename T, bool VEC>
__global__ __launch_bounds__(THREADS) void walk_residual_kernel(const VerifyLaunch v) {
  constexpr int WAVES = THREADS / 64;
  const int groups = walk_groups(v);
  const int slot = (int)blockIdx.x / XCDS;
  const int chunk = slot % groups, b = (slot / groups) * XCDS + (int)blockIdx.x % XCDS;
  if (b >= v.B) return;
  const bool lead = chunk == groups - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = v.N, R = v.R, RR = v.RR, SV = v.SV, NSUB = v.NSUB;
  const T* lg = static_cast<const T*>(v.logits);
  const T* dl = static_cast<const T*>(v.draft);
  __shared__ float s_K[MAX_RR];
  __shared__ int s_arg[MAX_RR];
  __shared__ double s_Z[MAX_RR];
  __shared__ double s_fac[MAX_RR][MAX_SV];
  __shared__ float s_cs[STASH];  // sub-chunk sums of every row, when RR * NSUB fits
  __shared__ float s_lp[8], s_lq[8];
  __shared__ int s_rej;
  __shared__ double s_a, s_u;
  __shared__ WalkState s_st;

  __shared__ float s_uu[16];  // the request's uniforms (R <= 15)

  // a cold request (draft_ids[b][0] < 0) has no valid drafts
  const bool cold = N > 1 && v.draft_ids[(size_t)b * (N - 1)] < 0;

  // Loads issued before the row statistics below: the uniforms, and the draft ids whose
  // logits this thread gathers (thread i < N-1: verify row i; thread 64 + i: draft row i).
  // The gather itself goes out right after the statistics' loads, so its round trip
  // overlaps their arithmetic instead of preceding it.
  const float u_pre = (tid < R) ? v.u[(size_t)b * R + tid] : 0.f;
  const T* gsrc = nullptr;
  int gid = 0;
  if (tid < N - 1) {
    gid = v.draft_ids[(size_t)b * (N - 1) + tid];
    gsrc = lg + ((size_t)b * R + tid) * v.V;
  } else if (dl && tid >= 64 && tid < 64 + N - 1) {
    gid = v.draft_ids[(size_t)b * (N - 1) + (tid - 64)];
    gsrc = dl + ((size_t)b * (N - 1) + (tid - 64)) * v.V;
  }
  float glog = 0.f;
  bool gathered = false;

  // A. per row (one wave each; the proposal rows only in the lead workgroup): raw max
  //    and its lowest id, reference Kmax, chunk factors 2^(K_c - Kmax) and
  //    Z = sum_k 2^(l_k c2 - Kmax) over the sub-chunk sums (fp64).  A wave issues the
  //    loads of all its rows of a batch before it uses any, so a batch costs one round
  //    trip; the sub-chunk sums are kept in LDS for the draws when they fit.
  const bool stash = RR * NSUB <= STASH;
  for (int r0 = wave; r0 < RR; r0 += WAVES * RPB) {
    float mv[RPB], kv[RPB], cv[RPB][CSL];
    int iv[RPB];
#pragma unroll
    for (int q = 0; q < RPB; ++q) {
      // rows this workgroup skips below (the proposal rows outside the lead workgroup)
      // load row 0's records again, which the cache already holds: a uniform select,
      // not a branch, so the compiler's wait counts stay exact
      const int rr_ = min(r0 + q * WAVES, RR - 1);
      const int rq = (!lead && rr_ >= N - 1 && rr_ < R) ? 0 : rr_;
      const RowRecords rec = row_records(v, b, rq);
      const int c = min(lane, SV - 1);
      mv[q] = rec.cmax[c];
      kv[q] = rec.cref[c];
      iv[q] = v.cidx[((size_t)b * RR + rq) * SV + c];  // used for the proposal rows only
#pragma unroll
      for (int t = 0; t < CSL; ++t) cv[q][t] = rec.csub[min(t * 64 + lane, NSUB - 1)];
    }
    __builtin_amdgcn_sched_barrier(0);
    if (gsrc && !gathered) {
      glog = to_f(gsrc[min(max(gid, 0), v.V - 1)]);
      gathered = true;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < RPB; ++q) {
      const int rr = r0 + q * WAVES;
      if (rr >= RR || (!lead && rr >= N - 1 && rr < R)) continue;
      const float* cs = row_records(v, b, rr).csub;
      const float m = (lane < SV) ? mv[q] : -__builtin_inff();
      const float k = (lane < SV) ? kv[q] : -__builtin_inff();
      const float M = wave_max(m);
      const float Kmax = wave_max(k);
      const int arg = wave_min_i(m == M && lane < SV ? iv[q] : INT_MAX);
      const double fl = (lane < SV) ? exp2((double)k - (double)Kmax) : 0.0;
      if (lane < SV) s_fac[rr][lane] = fl;
      double z = 0.0;
#pragma unroll
      for (int t = 0; t < CSL; ++t) {
        const int j = t * 64 + lane;
        const double f = __shfl(fl, min(j, NSUB - 1) / VCHUNK_SUBS);
        if (j < NSUB) {
          z += (double)cv[q][t] * f;
          if (stash) s_cs[rr * NSUB + j] = cv[q][t];
        }
      }
      for (int j0 = CSL * 64; j0 < NSUB; j0 += 64) {
        const int j = j0 + lane;
        const double f = __shfl(fl, min(j, NSUB - 1) / VCHUNK_SUBS);
        if (j < NSUB) {
          const float cj = cs[j];
          z += (double)cj * f;
          if (stash) s_cs[rr * NSUB + j] = cj;
        }
      }
      z = wave_sum_d(z);
      if (lane == 0) {
        s_K[rr] = Kmax;
        s_arg[rr] = arg;
        s_Z[rr] = z;
        if (lead && v.row_lse)
          v.row_lse[(size_t)b * (R + N - 1) + rr] = (float)(((double)Kmax + log2(z)) * 0.6931471805599453);
      }
    }
  }
  if (gsrc && !gathered) glog = to_f(gsrc[min(max(gid, 0), v.V - 1)]);
  if (tid < N - 1) s_lp[tid] = glog;
  else if (gsrc) s_lq[tid - 64] = glog;
  if (tid < R) s_uu[tid] = u_pre;
  __syncthreads();

  // rows without statistics (no draft rows with argmax drafts) report 0
  if (lead && v.row_lse && tid >= RR && tid < R + N - 1) v.row_lse[(size_t)b * (R + N - 1) + tid] = 0.f;

  // B. p(d_i), q~(d_i) and the acceptance ratios, one thread per draft; then the walk
  //    (one thread; everything it needs is in LDS)
  //    A cold request (draft_ids[b][0] < 0: no valid drafts) takes no walk.
  __shared__ double s_ratio[8];
  if (tid < N - 1) {
    const int i = tid;
    const double c2 = v.c2;
    const double P = cold ? 0.0 : exp2((double)s_lp[i] * c2 - (double)s_K[i]) / s_Z[i];
    const double Q = cold ? 0.0 : dl ? exp2((double)s_lq[i] * c2 - (double)s_K[R + i]) / s_Z[R + i] : 1.0;
    if (lead && v.p_draft) v.p_draft[(size_t)b * (N - 1) + i] = (float)P;
    if (lead && v.q_draft) v.q_draft[(size_t)b * (N - 1) + i] = (float)Q;
    s_ratio[i] = (P >= Q) ? 1.0 : P / Q;
  }
  __syncthreads();
  if (tid == 0) {
    int rej = -1;
    double ra = 1.0, ru = 0.0;
    for (int i = 0; i < N - 1 && !cold; ++i) {
      const double a = s_ratio[i];
      uint8_t acc = 0;
      if (rej < 0) {
        const double u = (double)s_uu[i];
        if (u < a) {
          acc = 1;
        } else {
          rej = i;
          ra = a;
          ru = u;
        }
      }
      if (lead) v.accept[(size_t)b * (N - 1) + i] = acc;
    }
    if (lead && cold)
      for (int i = 0; i < N - 1; ++i) v.accept[(size_t)b * (N - 1) + i] = 0;
    if (lead) v.n_accept[b] = cold ? 0 : (rej < 0) ? N - 1 : rej;
    s_rej = rej;
    s_a = ra;
    s_u = ru;
    WalkState st;
    st.rej = -1;
    st.pad = 0;
    st.up = 0.0;
    st.zp = 1.0;
    st.kp = st.kq = 0.f;
    st.izp_hi = st.izp_lo = st.izq_hi = st.izq_lo = 0.f;
    if (rej >= 0 && dl) {
      st.rej = rej;
      st.up = (ru - ra) / (1.0 - ra);
      st.zp = s_Z[rej];
      st.kp = s_K[rej];
      st.kq = s_K[R + rej];
      const double izp = 1.0 / s_Z[rej], izq = 1.0 / s_Z[R + rej];
      st.izp_hi = (float)izp;
      st.izp_lo = (float)(izp - (double)st.izp_hi);
      st.izq_hi = (float)izq;
      st.izq_lo = (float)(izq - (double)st.izq_hi);
    }
    s_st = st;
    if (lead) v.ws[b] = st;
  }
  __syncthreads();
  const int rej = s_rej;

  if (!lead) {
    // C. this chunk's residual sums of a rejecting request (sampled drafts)
    const WalkState st = s_st;
    if (st.rej < 0) return;
    constexpr int VE = VecOf<T>::n;
    constexpr int RR_ = kRounds<T> / RSPLIT;  // rounds of a residual chunk
    const int base = chunk * (VCHUNK / RSPLIT);
    float xp[RR_ * VE], xq[RR_ * VE];
    load_chunk<T, VEC, RR_>(row_ptr<T>(v, b, st.rej), v.V, base, tid, xp);
    load_chunk<T, VEC, RR_>(row_ptr<T>(v, b, v.R + st.rej), v.V, base, tid, xq);
    __shared__ float lds[RR_ * THREADS];
    float sr[RR_];
#pragma unroll
    for (int k = 0; k < RR_; ++k) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < VE; ++j) acc += residual_weight(xp[k * VE + j], xq[k * VE + j], st, v.c2);
      sr[k] = acc;
    }
    sub_sums<T, RR_>(sr, lds, v.rsub + (size_t)b * v.NSUB, chunk, v.NSUB, tid);
    return;
  }

  // D. inverse-CDF draws, one wave each: N proposal rows, plus the argmax-draft residual
  const bool argmax_residual = (rej >= 0) && (dl == nullptr);
  const int jobs = N + ((argmax_residual || cold) ? 1 : 0);
  for (int jb = wave; jb < jobs; jb += WAVES) {
    int k;
    if (jb < N) {
      const int rr = N - 1 + jb;
      const double u = (double)s_uu[rr];
      k = sample_row<T, VEC>(v, b, rr, s_fac[rr], u * s_Z[rr], -1, lane, stash ? s_cs + rr * NSUB : nullptr);
      if (lane == 0) {
        v.sampled_ids[(size_t)b * N + jb] = k;
        v.argmax_ids[(size_t)b * N + jb] = s_arg[rr];
        if (jb == 0 && rej < 0 && !cold) v.next_token[b] = k;
      }
    } else if (cold) {
      // no valid drafts: the exact token of the next position from row 0 at u_0
      k = sample_row<T, VEC>(v, b, 0, s_fac[0], (double)s_uu[0] * s_Z[0], -1, lane,
                             stash ? s_cs : nullptr);
      if (lane == 0) v.next_token[b] = k;
    } else {
      // residual of a one-hot q~: p_rej with the draft removed, drawn at (u - a)/(1 - a)
      const int d = min(max(v.draft_ids[(size_t)b * (N - 1) + rej], 0), v.V - 1);
      const T* row = row_ptr<T>(v, b, rej);
      const float* cr = v.cref + ((size_t)b * RR + rej) * SV;
      const int c = d / VCHUNK;
      const double wd = (double)rel_weight(to_f(row[d]), cr[c], v.c2) * s_fac[rej][c];
      const double W = s_Z[rej] - wd;
      const double up = (s_u - s_a) / (1.0 - s_a);
      const float* cst = stash ? s_cs + rej * NSUB : nullptr;
      if (W > 0.0)
        k = sample_row<T, VEC>(v, b, rej, s_fac[rej], up * W, d, lane, cst);
      else
        k = sample_row<T, VEC>(v, b, rej, s_fac[rej], up * s_Z[rej], -1, lane, cst);
      if (lane == 0) v.next_token[b] = k;
    }
  }
}

// ---------------------------------------------------------------- residual draw
template <typename T, bool VEC>
__global__ __launch_bounds__(64) void locate_kernel(const VerifyLaunch v) {
  const int b = blockIdx.x, lane = threadIdx.x;
  // the walk state and the residual sums in one round trip; the sums go to LDS
  const WalkState st = v.ws[b];
  const float* rs = v.rsub + (size_t)b * v.NSUB;
  __shared__ float s_rs[MAX_SV * VCHUNK_SUBS];
  float rv[CSL];
#pragma unroll
  for (int t = 0; t < CSL; ++t) rv[t] = rs[min(t * 64 + lane, v.NSUB - 1)];
  if (st.rej < 0) return;
  double W = 0.0;
#pragma unroll
  for (int t = 0; t < CSL; ++t) {
    const int j = t * 64 + lane;
    if (j < v.NSUB) {
      W += (double)rv[t];
      s_rs[j] = rv[t];
    }
  }
  for (int j = CSL * 64 + lane; j < v.NSUB; j += 64) {
    const float r = rs[j];
    W += (double)r;
    s_rs[j] = r;
  }
  W = wave_sum_d(W);
  __syncthreads();
  int k;
  if (W > 0.0) {
    const T* rp = row_ptr<T>(v, b, st.rej);
    const T* rq = row_ptr<T>(v, b, v.R + st.rej);
    const double target = st.up * W;
    auto subw = [&](int j) -> double { return (double)s_rs[j]; };
    double pre;
    const int js = find_sub(subw, v.NSUB, target, lane, pre);
    const int e0 = js * VSUB, end = min(e0 + VSUB, v.V);
    float xp[16], xq[16];
    load16<T, VEC>(rp, e0 + lane * 16, end, xp);
    load16<T, VEC>(rq, e0 + lane * 16, end, xq);
    double w16[16];
#pragma unroll
    for (int t = 0; t < 16; ++t)
      w16[t] = (e0 + lane * 16 + t < end) ? (double)residual_weight(xp[t], xq[t], st, v.c2) : 0.0;
    k = find_in16(w16, e0, pre, target, lane);
  } else {
    // p <= q~ everywhere (only by rounding): draw from p itself
    const size_t rowid = (size_t)b * v.RR + st.rej;
    const float* cr = v.cref + rowid * v.SV;
    __shared__ double s_fac[MAX_SV];
    if (lane < v.SV) s_fac[lane] = exp2((double)cr[lane] - (double)st.kp);
    __syncthreads();
    k = sample_row<T, VEC>(v, b, st.rej, s_fac, st.up * st.zp, -1, lane);
  }
  if (lane == 0) v.next_token[b] = k;
}

template <typename T>
hipError_t launch_stats_typed(const VerifyLaunch& v, hipStream_t s) {
  const bool vec = ((size_t)v.V * sizeof(T)) % 16 == 0;
  const dim3 g1(v.SV, v.snrow, v.B);
  if (vec) {
    // a resident grid: a few workgroups per CU, each streaming its units
    static std::atomic<int> slots_of_device[64];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    int slots = (dev >= 0 && dev < 64) ? slots_of_device[dev].load(std::memory_order_relaxed) : 0;
    if (slots <= 0) {
      int cus = 0, per_cu = 0;
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, stats_resident_kernel<T>, THREADS, 0);
      if (e != hipSuccess) return e;
      slots = max(1, per_cu) * max(1, cus);
      if (dev >= 0 && dev < 64) slots_of_device[dev].store(slots, std::memory_order_relaxed);
    }
    const int U = v.B * v.snrow * v.SV;
    stats_resident_kernel<T><<<min(U, slots), THREADS, 0, s>>>(v, U);
  } else {
    stats_kernel<T, false><<<g1, THREADS, 0, s>>>(v);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_tail_typed(const VerifyLaunch& v, hipStream_t s) {
  const bool vec = ((size_t)v.V * sizeof(T)) % 16 == 0;
  const unsigned g2 = (unsigned)(XCDS * ((v.B + XCDS - 1) / XCDS) * walk_groups(v));
  if (vec) walk_residual_kernel<T, true><<<g2, THREADS, 0, s>>>(v);
  else walk_residual_kernel<T, false><<<g2, THREADS, 0, s>>>(v);
  if (v.draft) {
    if (vec) locate_kernel<T, true><<<v.B, 64, 0, s>>>(v);
    else locate_kernel<T, false><<<v.B, 64, 0, s>>>(v);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_stats(const VerifyLaunch& v, hipStream_t s) {
  if (v.SV > MAX_SV || v.RR > MAX_RR || v.srow0 < 0 || v.snrow < 1 || v.srow0 + v.snrow > v.RR)
    return hipErrorInvalidValue;
  return v.dtype == 1 ? launch_stats_typed<uint16_t>(v, s) : launch_stats_typed<float>(v, s);
}

hipError_t launch_verify_tail(const VerifyLaunch& v, hipStream_t s) {
  if (v.SV > MAX_SV || v.RR > MAX_RR) return hipErrorInvalidValue;
  return v.dtype == 1 ? launch_tail_typed<uint16_t>(v, s) : launch_tail_typed<float>(v, s);
}

hipError_t launch_verify(const VerifyLaunch& v, hipStream_t s) {
  const hipError_t e = launch_verify_stats(v, s);
  if (e != hipSuccess) return e;
  return launch_verify_tail(v, s);
}

}  // namespace isd
