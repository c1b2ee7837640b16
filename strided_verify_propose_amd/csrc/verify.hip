// Vocab-wide verification of one ISD step.
//
// Method: [MASK] rows propose from q, clean rows verify earlier proposals against the
// causal anchor p, and a proposal x is kept with probability min(1, p(x)/q(x)), which
// leaves the AR distribution unchanged (page 1 "I-DLM 如何解決這些問題"; page 5
// "Inference & ISD").  Proposals are argmax ids (page 1 "實際部署：SGLang 整合").  On a
// rejection the next token comes from the normalised residual max(0, p - q~).
//
// Kernels (all HBM-streaming, no MFMA: this is a reduction over the vocabulary):
//   stats    grid (chunk, row, request): one 16384-entry chunk of one row per workgroup.
//            Chunk max of the raw logits, the lowest id holding it, and for every
//            1024-entry sub-chunk the sum of 2^((l - chunk max) * log2(e)/T) (fp32).
//   walk     one workgroup per request: combines chunk statistics in fp64 (row max,
//            log-sum-exp), runs the acceptance walk, and draws every inverse-CDF sample
//            from the fp64 prefix over sub-chunk sums plus one re-read sub-chunk.
//   residual grid (chunk, request), only for requests whose sampled draft was rejected:
//            per sub-chunk sums of max(0, p - q~) over the two rows involved.
//   locate   one wave per such request: prefix over those sums, re-read one sub-chunk.
// Argmax drafts (no draft rows) need no residual pass: the residual is p with the draft
// removed, whose sub-chunk sums the stats pass already has.
#include <limits.h>

#include "device.h"
#include "launch.h"

namespace isd {
namespace {

constexpr int THREADS = 256;
constexpr int MAX_RR = 22;    // 2N-1 + N-1 rows for N <= 8
constexpr int MAX_SV = 64;    // vocab <= 2^20

template <typename T> struct VecOf;
template <> struct VecOf<uint16_t> { static constexpr int n = 8; };
template <> struct VecOf<float> { static constexpr int n = 4; };

__device__ __forceinline__ float to_f(uint16_t h) { return bf16_to_f32(h); }
__device__ __forceinline__ float to_f(float f) { return f; }

// Weight of a logit relative to a reference (a chunk or row maximum), 2^((l - ref) c2),
// c2 = log2(e)/T.  Every kernel computes element weights through this one function, so
// a re-read element gets exactly the weight the stats pass summed.
__device__ __forceinline__ float rel_weight(float l, float ref, float c2) {
  return exp2_hw((l - ref) * c2);
}

// Residual weight max(0, p - q~) in fp32; 1/Z is applied as a hi + lo pair so its
// rounding does not bias p against q~.
__device__ __forceinline__ float residual_weight(float lp, float lq, const WalkState& st, float c2) {
  const float ep = rel_weight(lp, st.mp, c2);
  const float eq = rel_weight(lq, st.mq, c2);
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
template <typename T, bool VEC>
__device__ __forceinline__ void load_chunk(const T* __restrict__ row, int V, int base, int tid,
                                           float (&x)[VCHUNK / THREADS]) {
  constexpr int VE = VecOf<T>::n;
  constexpr int ROUNDS = VCHUNK / (THREADS * VE);
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

// Per-round wave sums -> per sub-chunk sums, in a fixed order.
template <typename T>
__device__ __forceinline__ void write_sub_sums(const float (&rs)[VCHUNK / (THREADS * VecOf<T>::n)][4],
                                               float* out, int chunk, int nsub, int tid) {
  constexpr int VE = VecOf<T>::n;
  constexpr int SPR = THREADS * VE / VSUB;  // sub-chunks per round
  constexpr int WPS = 4 / SPR;              // waves per sub-chunk
  if (tid < VCHUNK_SUBS) {
    const int k = tid / SPR, part = tid % SPR;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < WPS; ++w) s += rs[k][part * WPS + w];
    const int sub = chunk * VCHUNK_SUBS + tid;
    if (sub < nsub) out[sub] = s;
  }
}

// ---------------------------------------------------------------- stats pass
template <typename T, bool VEC>
__global__ __launch_bounds__(THREADS) void stats_kernel(const VerifyLaunch v) {
  constexpr int VE = VecOf<T>::n;
  constexpr int ROUNDS = VCHUNK / (THREADS * VE);
  const int chunk = blockIdx.x, rr = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = chunk * VCHUNK;
  const T* __restrict__ row = row_ptr<T>(v, b, rr);
  float x[VCHUNK / THREADS];
  load_chunk<T, VEC>(row, v.V, base, tid, x);

  __shared__ float red[4];
  __shared__ int redi[4];
  __shared__ float rs[ROUNDS][4];
  float mx = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < VCHUNK / THREADS; ++i) mx = fmaxf(mx, x[i]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  const bool proposal = rr >= v.N - 1 && rr < v.R;
  int arg = INT_MAX;
  if (proposal) {
#pragma unroll
    for (int k = 0; k < ROUNDS; ++k)
#pragma unroll
      for (int j = 0; j < VE; ++j)
        if (x[k * VE + j] == M && arg == INT_MAX) arg = base + k * THREADS * VE + tid * VE + j;
    arg = wave_min_i(arg);
    if (lane == 0) redi[wave] = arg;
  }
#pragma unroll
  for (int k = 0; k < ROUNDS; ++k) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < VE; ++j) s += rel_weight(x[k * VE + j], M, v.c2);
    s = wave_sum(s);
    if (lane == 0) rs[k][wave] = s;
  }
  __syncthreads();
  const size_t rowid = (size_t)b * v.RR + rr;
  write_sub_sums<T>(rs, v.csub + rowid * v.NSUB, chunk, v.NSUB, tid);
  if (tid == 0) {
    v.cmax[rowid * v.SV + chunk] = M;
    v.cidx[rowid * v.SV + chunk] =
        proposal ? min(min(redi[0], redi[1]), min(redi[2], redi[3])) : INT_MAX;
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

// Smallest entry k in [e0, e0 + cnt) with pre + prefix(e0..k) > target; lane l takes 16
// consecutive entries.  Fallback: the last entry with positive weight.
template <class ElemW>
__device__ int find_elem(ElemW elw, int e0, int cnt, double pre, double target, int lane) {
  const int k0 = e0 + lane * 16;
  double w16[16];
  double s = 0.0;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    const int k = k0 + t;
    w16[t] = (k < e0 + cnt) ? elw(k) : 0.0;
    s += w16[t];
  }
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
    if (ans < 0) ans = e0;
  }
  return ans;
}

// Inverse-CDF draw from row rr (weights 2^((l - M) c2)), optionally with one id removed.
template <typename T>
__device__ int sample_row(const VerifyLaunch& v, int b, int rr, float M, double target, int excl,
                          int lane) {
  const T* __restrict__ row = row_ptr<T>(v, b, rr);
  const size_t rowid = (size_t)b * v.RR + rr;
  const float* __restrict__ cm = v.cmax + rowid * v.SV;
  const float* __restrict__ cs = v.csub + rowid * v.NSUB;
  const double c2 = v.c2;
  double wex = 0.0;
  int exsub = -1;
  if (excl >= 0) {
    const int c = excl / VCHUNK;
    wex = (double)rel_weight(to_f(row[excl]), cm[c], v.c2) * exp2((double)(cm[c] - M) * c2);
    exsub = excl / VSUB;
  }
  auto subw = [&](int j) -> double {
    const int c = j / VCHUNK_SUBS;
    double w = (double)cs[j] * exp2((double)(cm[c] - M) * c2);
    if (j == exsub) w = fmax(0.0, w - wex);
    return w;
  };
  double pre;
  const int js = find_sub(subw, v.NSUB, target, lane, pre);
  const int c = js / VCHUNK_SUBS;
  const float ref = cm[c];
  const double fc = exp2((double)(ref - M) * c2);
  auto elw = [&](int k) -> double {
    if (k == excl) return 0.0;
    return (double)rel_weight(to_f(row[k]), ref, v.c2) * fc;
  };
  const int e0 = js * VSUB;
  return find_elem(elw, e0, min(VSUB, v.V - e0), pre, target, lane);
}

// ---------------------------------------------------------------- walk
template <typename T>
__global__ __launch_bounds__(THREADS) void walk_kernel(const VerifyLaunch v) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = v.N, R = v.R, RR = v.RR, SV = v.SV, NSUB = v.NSUB;
  const double c2 = v.c2;
  __shared__ float s_M[MAX_RR];
  __shared__ int s_arg[MAX_RR];
  __shared__ double s_Z[MAX_RR];
  __shared__ int s_rej;
  __shared__ double s_a, s_u;

  // A. per row: max, argmax, Z = sum_k 2^((l_k - M) c2) (fp64 over chunk factors)
  for (int rr = wave; rr < RR; rr += 4) {
    const size_t rowid = (size_t)b * RR + rr;
    const float* cm = v.cmax + rowid * SV;
    const int32_t* ci = v.cidx + rowid * SV;
    const float* cs = v.csub + rowid * NSUB;
    float M = -__builtin_inff();
    for (int c = lane; c < SV; c += 64) M = fmaxf(M, cm[c]);
    M = wave_max(M);
    int arg = INT_MAX;
    for (int c = lane; c < SV; c += 64)
      if (cm[c] == M) arg = min(arg, ci[c]);
    arg = wave_min_i(arg);
    double z = 0.0;
    for (int j = lane; j < NSUB; j += 64)
      z += (double)cs[j] * exp2((double)(cm[j / VCHUNK_SUBS] - M) * c2);
    z = wave_sum_d(z);
    if (lane == 0) {
      s_M[rr] = M;
      s_arg[rr] = arg;
      s_Z[rr] = z;
    }
  }
  __syncthreads();

  // B. the acceptance walk (one thread)
  if (tid == 0) {
    const T* lg = static_cast<const T*>(v.logits);
    const T* dl = static_cast<const T*>(v.draft);
    if (v.row_lse) {
      for (int rr = 0; rr < R + N - 1; ++rr)
        v.row_lse[(size_t)b * (R + N - 1) + rr] =
            (rr < RR) ? (float)((double)s_M[rr] * v.invT + log(s_Z[rr])) : 0.f;
    }
    int rej = -1;
    double ra = 1.0, ru = 0.0;
    for (int i = 0; i < N - 1; ++i) {
      const int d = min(max(v.draft_ids[(size_t)b * (N - 1) + i], 0), v.V - 1);
      const float lp = to_f(lg[((size_t)b * R + i) * v.V + d]);
      const double P = exp2(((double)lp - s_M[i]) * c2) / s_Z[i];
      double Q = 1.0;
      if (dl) {
        const float lq = to_f(dl[((size_t)b * (N - 1) + i) * v.V + d]);
        Q = exp2(((double)lq - s_M[R + i]) * c2) / s_Z[R + i];
      }
      if (v.p_draft) v.p_draft[(size_t)b * (N - 1) + i] = (float)P;
      if (v.q_draft) v.q_draft[(size_t)b * (N - 1) + i] = (float)Q;
      const double a = (P >= Q) ? 1.0 : P / Q;
      uint8_t acc = 0;
      if (rej < 0) {
        const double u = (double)v.u[(size_t)b * R + i];
        if (u < a) {
          acc = 1;
        } else {
          rej = i;
          ra = a;
          ru = u;
        }
      }
      v.accept[(size_t)b * (N - 1) + i] = acc;
    }
    v.n_accept[b] = (rej < 0) ? N - 1 : rej;
    s_rej = rej;
    s_a = ra;
    s_u = ru;
    WalkState st;
    st.rej = -1;
    st.pad = 0;
    st.up = 0.0;
    st.mp = st.mq = 0.f;
    st.izp_hi = st.izp_lo = st.izq_hi = st.izq_lo = 0.f;
    if (rej >= 0 && dl) {
      st.rej = rej;
      st.up = (ru - ra) / (1.0 - ra);
      st.mp = s_M[rej];
      st.mq = s_M[R + rej];
      const double izp = 1.0 / s_Z[rej], izq = 1.0 / s_Z[R + rej];
      st.izp_hi = (float)izp;
      st.izp_lo = (float)(izp - (double)st.izp_hi);
      st.izq_hi = (float)izq;
      st.izq_lo = (float)(izq - (double)st.izq_hi);
    }
    v.ws[b] = st;
  }
  __syncthreads();

  // C. inverse-CDF draws: N proposal rows, plus the argmax-draft residual
  const int rej = s_rej;
  const bool argmax_residual = (rej >= 0) && (v.draft == nullptr);
  const int jobs = N + (argmax_residual ? 1 : 0);
  for (int jb = wave; jb < jobs; jb += 4) {
    int k;
    if (jb < N) {
      const int rr = N - 1 + jb;
      const double u = (double)v.u[(size_t)b * R + rr];
      k = sample_row<T>(v, b, rr, s_M[rr], u * s_Z[rr], -1, lane);
      if (lane == 0) {
        v.sampled_ids[(size_t)b * N + jb] = k;
        v.argmax_ids[(size_t)b * N + jb] = s_arg[rr];
        if (jb == 0 && rej < 0) v.next_token[b] = k;
      }
    } else {
      // residual of a one-hot q~: p_rej with the draft removed, drawn at (u - a)/(1 - a)
      const int d = min(max(v.draft_ids[(size_t)b * (N - 1) + rej], 0), v.V - 1);
      const T* row = row_ptr<T>(v, b, rej);
      const float* cm = v.cmax + ((size_t)b * RR + rej) * SV;
      const float M = s_M[rej];
      const int c = d / VCHUNK;
      const double wd = (double)rel_weight(to_f(row[d]), cm[c], v.c2) *
                        exp2((double)(cm[c] - M) * c2);
      const double W = s_Z[rej] - wd;
      const double up = (s_u - s_a) / (1.0 - s_a);
      if (W > 0.0)
        k = sample_row<T>(v, b, rej, M, up * W, d, lane);
      else
        k = sample_row<T>(v, b, rej, M, up * s_Z[rej], -1, lane);
      if (lane == 0) v.next_token[b] = k;
    }
  }
}

// ---------------------------------------------------------------- residual (sampled drafts)
template <typename T, bool VEC>
__global__ __launch_bounds__(THREADS) void residual_kernel(const VerifyLaunch v) {
  constexpr int VE = VecOf<T>::n;
  constexpr int ROUNDS = VCHUNK / (THREADS * VE);
  const int chunk = blockIdx.x, b = blockIdx.y;
  const WalkState st = v.ws[b];
  if (st.rej < 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = chunk * VCHUNK;
  float xp[VCHUNK / THREADS], xq[VCHUNK / THREADS];
  load_chunk<T, VEC>(row_ptr<T>(v, b, st.rej), v.V, base, tid, xp);
  load_chunk<T, VEC>(row_ptr<T>(v, b, v.R + st.rej), v.V, base, tid, xq);
  __shared__ float rs[ROUNDS][4];
#pragma unroll
  for (int k = 0; k < ROUNDS; ++k) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < VE; ++j) s += residual_weight(xp[k * VE + j], xq[k * VE + j], st, v.c2);
    s = wave_sum(s);
    if (lane == 0) rs[k][wave] = s;
  }
  __syncthreads();
  write_sub_sums<T>(rs, v.rsub + (size_t)b * v.NSUB, chunk, v.NSUB, tid);
}

template <typename T>
__global__ __launch_bounds__(64) void locate_kernel(const VerifyLaunch v) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const WalkState st = v.ws[b];
  if (st.rej < 0) return;
  const float* rs = v.rsub + (size_t)b * v.NSUB;
  double W = 0.0;
  for (int j = lane; j < v.NSUB; j += 64) W += (double)rs[j];
  W = wave_sum_d(W);
  int k;
  if (W > 0.0) {
    const T* rp = row_ptr<T>(v, b, st.rej);
    const T* rq = row_ptr<T>(v, b, v.R + st.rej);
    const double target = st.up * W;
    auto subw = [&](int j) -> double { return (double)rs[j]; };
    double pre;
    const int js = find_sub(subw, v.NSUB, target, lane, pre);
    auto elw = [&](int e) -> double {
      return (double)residual_weight(to_f(rp[e]), to_f(rq[e]), st, v.c2);
    };
    const int e0 = js * VSUB;
    k = find_elem(elw, e0, min(VSUB, v.V - e0), pre, target, lane);
  } else {
    // p <= q~ everywhere (only by rounding): draw from p itself
    const double Zp = 1.0 / ((double)st.izp_hi + (double)st.izp_lo);
    k = sample_row<T>(v, b, st.rej, st.mp, st.up * Zp, -1, lane);
  }
  if (lane == 0) v.next_token[b] = k;
}

template <typename T>
hipError_t launch_typed(const VerifyLaunch& v, hipStream_t s) {
  const bool vec = ((size_t)v.V * sizeof(T)) % 16 == 0;
  const dim3 g1(v.SV, v.RR, v.B);
  if (vec) stats_kernel<T, true><<<g1, THREADS, 0, s>>>(v);
  else stats_kernel<T, false><<<g1, THREADS, 0, s>>>(v);
  walk_kernel<T><<<v.B, THREADS, 0, s>>>(v);
  if (v.draft) {
    const dim3 g3(v.SV, v.B);
    if (vec) residual_kernel<T, true><<<g3, THREADS, 0, s>>>(v);
    else residual_kernel<T, false><<<g3, THREADS, 0, s>>>(v);
    locate_kernel<T><<<v.B, 64, 0, s>>>(v);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_verify(const VerifyLaunch& v, hipStream_t s) {
  if (v.SV > MAX_SV || v.RR > MAX_RR) return hipErrorInvalidValue;
  return v.dtype == 1 ? launch_typed<uint16_t>(v, s) : launch_typed<float>(v, s);
}

}  // namespace isd
