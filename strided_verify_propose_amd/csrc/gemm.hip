// R-ISD gated projection on gfx950 MFMA:  Y = X W + gate * bf16(X A) B   (bf16 in/out).
//
// R-ISD (「首次超越 AR 模型」 "無損 R-ISD"; 「内省扩散语言模型」 "1. 引言"; 「I-DLM – introspektive Diffusion Language Models」 "Lossless R-ISD"): the LoRA
// delta is added only on gated ([MASK]) rows; verify rows keep the base product bit
// for bit.  Two kernels, no workgroup ever waits on another:
//   base_kernel  one GEMM over the stacked weights [W^T; A^T] (Nout + r rows of K):
//                tiles of W^T give the base product -- written as bf16 for ungated rows
//                (exactly what a gate-free call writes) and kept in fp32 for gated
//                rows -- and the tiles of A^T give T = bf16(X A).
//   lora_kernel  gated rows only: Y = bf16(base + T B) with T B on MFMA (K = r, every
//                step's loads at once).
// Tiles: 64 x 128 per workgroup, 4 waves of 32 x 64 (2 x 4 MFMA 16x16x32 blocks), K in
// steps of 64: three steps of global loads in flight, one step staged in LDS, and the
// next step's MFMA fragments read from LDS while the current step's MFMAs run.  Workgroups are
// numbered so that the tiles sharing a weight-column block land on the same XCD and
// reuse it from that XCD's L2.
#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace isd {
namespace {

constexpr int BM = PROJ_BM, BN = PROJ_BN, BK = PROJ_BK;
constexpr int THREADS = 256;
constexpr int PROJ_RING = 4;  // register stages of the load pipeline
constexpr int A_LOADS = BM * BK / 8 / THREADS;  // 16-byte loads per thread per k step
constexpr int B_LOADS = BN * BK / 8 / THREADS;

// One k step (64) of operand data in flight for one thread.  Loads are row-contiguous:
// eight consecutive lanes read one row's 128 bytes.
struct Stage {
  u32x4 a[A_LOADS];
  u32x4 b[B_LOADS];
};

// LDS tile of one operand: MFMA fragments [k half][16-row block][slot], 16 bytes per
// slot.  Row r, 16-byte k chunk c (0..7) lives in fragment (c / 4, r / 16) at slot
// (c % 4) * 16 + ((r % 16) ^ c).  The xor spreads the eight chunks of a row, written
// by eight consecutive lanes, over all banks, and an MFMA operand read (lane l takes
// slot l ^ c) stays one conflict-free 1 KB sweep.
template <int ROWS>
struct OpTile {
  u32x4 f[2][ROWS / 16][64];
};
struct Tiles {
  OpTile<BM> a;
  OpTile<BN> b;
};

__device__ __forceinline__ int chunk_slot(int r, int c) { return (c & 3) * 16 + ((r & 15) ^ c); }

__device__ __forceinline__ void issue(Stage& st, const uint16_t* const (&pa)[A_LOADS],
                                      const uint16_t* const (&pb)[B_LOADS], int k) {
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) st.a[i] = *reinterpret_cast<const u32x4*>(pa[i] + k);
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) st.b[i] = *reinterpret_cast<const u32x4*>(pb[i] + k);
}

__device__ __forceinline__ void put(Tiles& t, const Stage& st, int tid) {
  const int c = tid & 7;
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int r = (tid >> 3) + 32 * i;
    t.a.f[c >> 2][r >> 4][chunk_slot(r, c)] = st.a[i];
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int r = (tid >> 3) + 32 * i;
    t.b.f[c >> 2][r >> 4][chunk_slot(r, c)] = st.b[i];
  }
}

// MFMA operand fragments of one k step for this wave (rows 32 wm + 16 i, columns
// 64 wn + 16 j), read from LDS one step ahead of their use.
struct Frags {
  u32x4 a[2][2];  // [k half][i]
  u32x4 b[2][4];  // [k half][j]
};

__device__ __forceinline__ void fetch_frags(Frags& f, const Tiles& t, int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int slot = lane ^ (kk * 4 + (lane >> 4));
#pragma unroll
    for (int i = 0; i < 2; ++i) f.a[kk][i] = t.a.f[kk][wm * 2 + i][slot];
#pragma unroll
    for (int j = 0; j < 4; ++j) f.b[kk][j] = t.b.f[kk][wn * 4 + j][slot];
  }
}

__device__ __forceinline__ void mma(const Frags& f, f32x4 (&acc)[2][4]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(f.a[kk][i], f.b[kk][j], acc[i][j]);
}

// acc = sum over k < K of X[row][k] Wt[col][k] for the 64 x 128 tile at X, Wt.  X rows
// past `mrows` read row mrows - 1 (never stored).  Three pipelines overlap at step s:
// global loads for step s + RING - 1 go out (RING register stages), step s + 2 goes from
// registers to LDS, step s + 1's fragments come from LDS into registers, and step s's
// MFMAs run on fragments already in registers.  LDS is double-buffered.
template <int RING>
__device__ void gemm_tile(Tiles (&lds)[2], const uint16_t* __restrict__ X, int ldx, int mrows,
                          const uint16_t* __restrict__ Wt, int ldw, int K, int tid, int wm, int wn,
                          int lane, f32x4 (&acc)[2][4]) {
  const uint16_t* pa[A_LOADS];
  const uint16_t* pb[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i)
    pa[i] = X + (size_t)min((tid >> 3) + 32 * i, mrows - 1) * ldx + (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) pb[i] = Wt + (size_t)((tid >> 3) + 32 * i) * ldw + (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  static_assert(RING % 2 == 0, "fragment buffers alternate with the step parity");
  const int S = K / BK;
  Stage r[RING];
  Frags f[2];
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) issue(r[u], pa, pb, min(u, S - 1) * BK);
  put(lds[0], r[0], tid);
  put(lds[1], r[1], tid);
  lds_barrier();
  fetch_frags(f[0], lds[0], wm, wn, lane);
  lds_barrier();  // every wave has read buffer 0 before step 0 refills it with step 2
  // Steps past the end re-load and re-stage the last step (unconditional loads keep the
  // compiler's wait counts exact); only the MFMAs are skipped.
  for (int s0 = 0; s0 < S; s0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      const int s = s0 + u;
      issue(r[(u + RING - 1) % RING], pa, pb, min(s + RING - 1, S - 1) * BK);
      fetch_frags(f[(u + 1) & 1], lds[(s + 1) & 1], wm, wn, lane);
      put(lds[s & 1], r[(u + 2) % RING], tid);
      if (s < S) mma(f[u & 1], acc);
      lds_barrier();
    }
  }
}

__global__ __launch_bounds__(THREADS) void base_kernel(const ProjLaunch p) {
  const int mt = (p.M + BM - 1) / BM, nt = (p.Nout + p.r) / BN;
  int tm, tn;
  if (!tile_of(blockIdx.x, mt, nt * p.ksplit, tm, tn)) return;
  const int ks = tn % p.ksplit, klen = p.K / p.ksplit, k0 = ks * klen;  // this part of K
  tn /= p.ksplit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, gq = lane >> 4;
  const int m0 = tm * BM, n0 = tn * BN;
  const int mrows = min(BM, p.M - m0);
  const bool lowrank = n0 >= p.Nout;  // this tile computes T = X A
  const uint16_t* Bsrc = (lowrank ? p.A + (size_t)(n0 - p.Nout) * p.K : p.W + (size_t)n0 * p.K) + k0;
  __shared__ Tiles lds[2];
  f32x4 acc[2][4];
  gemm_tile<PROJ_RING>(lds, p.X + (size_t)m0 * p.K + k0, p.K, mrows, Bsrc, p.K, klen, tid, wm, wn, lane, acc);
  if (p.ksplit > 1) {  // partial sums; proj_reduce_kernel adds them in order and stores
    const int ncols = p.Nout + p.r;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wm * 32 + i * 16 + 4 * gq + e;
        if (row >= mrows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          p.part[((size_t)ks * p.M + m0 + row) * ncols + n0 + wn * 64 + j * 16 + l16] = acc[i][j][e];
      }
    return;
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = wm * 32 + i * 16 + 4 * gq + e;
      if (row >= mrows) continue;
      const int gr = m0 + row;
      const bool gated = p.gate != nullptr && p.gate[gr] != 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + l16;
        const float v = acc[i][j][e];
        if (lowrank)
          p.T[(size_t)gr * p.r + (col - p.Nout)] = (uint16_t)f32_to_bf16_bits(v);
        else if (gated)
          p.Ybase[(size_t)gr * p.Nout + col] = v;
        else
          p.Y[(size_t)gr * p.Nout + col] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
}

// acc as gemm_tile computes it, for a short K = S BK (the delta's K = r): every step's
// loads go out at once, each step has its own LDS buffer, and one barrier separates the
// staging from the MFMAs, which run in the same order as in gemm_tile.  With the ring,
// K = r spent most of its time in the ring's refills past the last step.
template <int S>
__device__ void gemm_tile_short(Tiles (&lds)[S], const uint16_t* __restrict__ X, int ldx, int mrows,
                                const uint16_t* __restrict__ Wt, int ldw, int tid, int wm, int wn, int lane,
                                f32x4 (&acc)[2][4]) {
  const uint16_t* pa[A_LOADS];
  const uint16_t* pb[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i)
    pa[i] = X + (size_t)min((tid >> 3) + 32 * i, mrows - 1) * ldx + (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) pb[i] = Wt + (size_t)((tid >> 3) + 32 * i) * ldw + (tid & 7) * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  Stage r[S];
#pragma unroll
  for (int s = 0; s < S; ++s) issue(r[s], pa, pb, s * BK);
#pragma unroll
  for (int s = 0; s < S; ++s) put(lds[s], r[s], tid);
  lds_barrier();
#pragma unroll
  for (int s = 0; s < S; ++s) {
    Frags f;
    fetch_frags(f, lds[s], wm, wn, lane);
    mma(f, acc);
  }
}

template <int S>
__global__ __launch_bounds__(THREADS) void lora_kernel(const ProjLaunch p) {
  // tiles numbered over the base grid's Nout + r columns, so that tile (tm, tn) runs on the
  // XCD whose base-kernel workgroup wrote its fp32 base product (one L2); the A^T column
  // tiles have no delta
  const int mt = (p.M + BM - 1) / BM, ntb = (p.Nout + p.r) / BN;
  int tm, tn;
  if (!tile_of(blockIdx.x, mt, ntb, tm, tn) || tn >= p.Nout / BN) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, gq = lane >> 4;
  const int m0 = tm * BM, n0 = tn * BN;
  const int mrows = min(BM, p.M - m0);
  // The gate flags and the base product of this lane's elements are loaded first (rows
  // past the tile's end read its last row and are never written), so their round trip
  // overlaps the delta's loads instead of following its product.
  bool gated[2][4];
  float yb[2][4][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = wm * 32 + i * 16 + 4 * gq + e;
      const int gr = m0 + min(row, mrows - 1);
      gated[i][e] = p.gate[gr] != 0 && row < mrows;
#pragma unroll
      for (int j = 0; j < 4; ++j) yb[i][j][e] = p.Ybase[(size_t)gr * p.Nout + n0 + wn * 64 + j * 16 + l16];
    }
  __shared__ Tiles lds[S];
  f32x4 acc[2][4];
  gemm_tile_short<S>(lds, p.T + (size_t)m0 * p.r, p.r, mrows, p.Bl + (size_t)n0 * p.r, p.r, tid, wm, wn, lane, acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!gated[i][e]) continue;
      const int gr = m0 + wm * 32 + i * 16 + 4 * gq + e;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t o = (size_t)gr * p.Nout + n0 + wn * 64 + j * 16 + l16;
        p.Y[o] = (uint16_t)f32_to_bf16_bits(yb[i][j][e] + acc[i][j][e]);
      }
    }
}

int grid_of(int M, int ncols) { return tile_grid((M + BM - 1) / BM, ncols / BN); }

// Sum of the K parts, in part order, then the base kernel's stores: T for the A^T
// columns, the fp32 base product for gated rows, bf16 for the others.  Four columns
// per thread.
__global__ __launch_bounds__(256) void proj_reduce_kernel(const ProjLaunch p) {
  const int ncols = p.Nout + p.r, q4 = ncols / 4;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)p.M * q4) return;
  const int row = (int)(idx / q4), col = (int)(idx - (long long)row * q4) * 4;
  f32x4 v = *reinterpret_cast<const f32x4*>(p.part + (size_t)row * ncols + col);
  for (int s = 1; s < p.ksplit; ++s)
    v += *reinterpret_cast<const f32x4*>(p.part + ((size_t)s * p.M + row) * ncols + col);
  if (col >= p.Nout) {
    uint16_t* t = p.T + (size_t)row * p.r + (col - p.Nout);
    for (int i = 0; i < 4; ++i) t[i] = (uint16_t)f32_to_bf16_bits(v[i]);
  } else if (p.gate != nullptr && p.gate[row] != 0) {
    *reinterpret_cast<f32x4*>(p.Ybase + (size_t)row * p.Nout + col) = v;
  } else {
    u32x2 w;
    w[0] = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
    w[1] = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<u32x2*>(p.Y + (size_t)row * p.Nout + col) = w;
  }
}

}  // namespace

hipError_t launch_proj_reduce(const ProjLaunch& p, hipStream_t s) {
  const long long n = (long long)p.M * ((p.Nout + p.r) / 4);
  proj_reduce_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_lora(const ProjLaunch& p, hipStream_t s) {
  // K = r, one lora_kernel per supported rank (validated: 128 or 256)
  if (p.r == 2 * BK) lora_kernel<2><<<grid_of(p.M, p.Nout + p.r), THREADS, 0, s>>>(p);
  else if (p.r == 4 * BK) lora_kernel<4><<<grid_of(p.M, p.Nout + p.r), THREADS, 0, s>>>(p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_proj(const ProjLaunch& p, hipStream_t s) {
  if (p.big) return launch_proj_big(p, false, s);
  base_kernel<<<grid_of(p.M, (p.Nout + p.r) * p.ksplit), THREADS, 0, s>>>(p);
  if (p.ksplit > 1) {
    const hipError_t e = launch_proj_reduce(p, s);
    if (e != hipSuccess) return e;
  }
  if (p.gate) return launch_lora(p, s);
  return hipGetLastError();
}

}  // namespace isd
