// R-ISD gated projection on gfx950 MFMA:  Y = X W + gate * bf16(X A) B   (bf16 in/out).
//
// R-ISD (page 1 "無損 R-ISD"; page 3 "1. 引言"; page 5 "Lossless R-ISD"): the LoRA
// delta is added only on gated ([MASK]) rows; verify rows keep the base product bit
// for bit.  Two kernels, no workgroup ever waits on another:
//   base_kernel  one GEMM over the stacked weights [W^T; A^T] (Nout + r rows of K):
//                tiles of W^T give the base product -- written as bf16 for ungated rows
//                (exactly what a gate-free call writes) and kept in fp32 for gated
//                rows -- and the tiles of A^T give T = bf16(X A).
//   lora_kernel  gated rows only: Y = bf16(base + T B) with T B on MFMA (K = r).
// Tiles: 64 x 128 per workgroup, 4 waves of 32 x 64 (2 x 4 MFMA 16x16x32 blocks), K in
// steps of 64 through LDS with register prefetch of the next step.  Workgroups are
// numbered so that the tiles sharing a weight-column block land on the same XCD and
// reuse it from that XCD's L2.
#include "device.h"
#include "launch.h"

namespace isd {
namespace {

constexpr int BM = 64, BN = 128, BK = 64;
constexpr int LDP = BK + 8;  // padded LDS row (elements)
constexpr int THREADS = 256;
constexpr int XCDS = 8;

struct Tiles {
  uint16_t a[BM][LDP];
  uint16_t b[BN][LDP];
};

// Global -> registers: rows x 64 bf16 per operand tile, 16 B per thread per pass.
template <int ROWS>
__device__ __forceinline__ void fetch(const uint16_t* __restrict__ src, int rows_valid, int ld,
                                      int k, int tid, u32x4 (&r)[ROWS / 32]) {
#pragma unroll
  for (int p = 0; p < ROWS / 32; ++p) {
    const int idx = tid + THREADS * p;
    const int row = idx >> 3, c8 = idx & 7;
    r[p] = (row < rows_valid) ? *reinterpret_cast<const u32x4*>(src + (size_t)row * ld + k + c8 * 8)
                              : u32x4{0u, 0u, 0u, 0u};
  }
}
template <int ROWS>
__device__ __forceinline__ void stash(uint16_t (*dst)[LDP], int tid, const u32x4 (&r)[ROWS / 32]) {
#pragma unroll
  for (int p = 0; p < ROWS / 32; ++p) {
    const int idx = tid + THREADS * p;
    *reinterpret_cast<u32x4*>(&dst[idx >> 3][(idx & 7) * 8]) = r[p];
  }
}

// acc(32 x 64 per wave) += A_tile * B_tile^T over one BK step.  Wave (wm, wn) owns rows
// 32 wm .. and columns 64 wn ..
__device__ __forceinline__ void mma_step(const Tiles& t, int wm, int wn, int lane,
                                         f32x4 (&acc)[2][4]) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < BK / 32; ++kk) {
    u32x4 af[2], bf[4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(&t.a[wm * 32 + i * 16 + l16][kk * 32 + 8 * g]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const u32x4*>(&t.b[wn * 64 + j * 16 + l16][kk * 32 + 8 * g]);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
  }
}

// acc = sum over k in [0, K) of A[m0 + r, k] B[n0 + c, k]
__device__ void gemm_tile(Tiles& t, const uint16_t* __restrict__ A, int lda, int mrows,
                          const uint16_t* __restrict__ B, int ldb, int K, int tid, int wm, int wn,
                          int lane, f32x4 (&acc)[2][4]) {
  u32x4 ra[BM / 32], rb[BN / 32];
  fetch<BM>(A, mrows, lda, 0, tid, ra);
  fetch<BN>(B, BN, ldb, 0, tid, rb);
  for (int k = 0; k < K; k += BK) {
    __syncthreads();
    stash<BM>(t.a, tid, ra);
    stash<BN>(t.b, tid, rb);
    __syncthreads();
    if (k + BK < K) {
      fetch<BM>(A, mrows, lda, k + BK, tid, ra);
      fetch<BN>(B, BN, ldb, k + BK, tid, rb);
    }
    mma_step(t, wm, wn, lane, acc);
  }
}

// Linear workgroup id -> (m tile, n tile): XCD x (= id % 8, the dispatch order) takes the
// column blocks x, x + 8, ... with all their row tiles.
__device__ __forceinline__ bool tile_of(int id, int mt, int nt, int& m, int& n) {
  const int x = id % XCDS, k = id / XCDS;
  n = x + XCDS * (k / mt);
  m = k % mt;
  return n < nt;
}

__global__ __launch_bounds__(THREADS) void base_kernel(const ProjLaunch p) {
  const int mt = (p.M + BM - 1) / BM, nt = (p.Nout + p.r) / BN;
  int tm, tn;
  if (!tile_of(blockIdx.x, mt, nt, tm, tn)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, gq = lane >> 4;
  const int m0 = tm * BM, n0 = tn * BN;
  const int mrows = min(BM, p.M - m0);
  const bool lowrank = n0 >= p.Nout;  // this tile computes T = X A
  const uint16_t* Bsrc = lowrank ? p.A + (size_t)(n0 - p.Nout) * p.K : p.W + (size_t)n0 * p.K;
  __shared__ Tiles t;
  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile(t, p.X + (size_t)m0 * p.K, p.K, mrows, Bsrc, p.K, p.K, tid, wm, wn, lane, acc);

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

__global__ __launch_bounds__(THREADS) void lora_kernel(const ProjLaunch p) {
  const int mt = (p.M + BM - 1) / BM, nt = p.Nout / BN;
  int tm, tn;
  if (!tile_of(blockIdx.x, mt, nt, tm, tn)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, gq = lane >> 4;
  const int m0 = tm * BM, n0 = tn * BN;
  const int mrows = min(BM, p.M - m0);
  // skip tiles without gated rows
  __shared__ int s_any;
  if (tid == 0) s_any = 0;
  __syncthreads();
  if (tid < mrows && p.gate[m0 + tid]) s_any = 1;
  __syncthreads();
  if (!s_any) return;
  __shared__ Tiles t;
  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile(t, p.T + (size_t)m0 * p.r, p.r, mrows, p.Bl + (size_t)n0 * p.r, p.r, p.r, tid, wm, wn,
            lane, acc);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = wm * 32 + i * 16 + 4 * gq + e;
      if (row >= mrows) continue;
      const int gr = m0 + row;
      if (!p.gate[gr]) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t o = (size_t)gr * p.Nout + n0 + wn * 64 + j * 16 + l16;
        p.Y[o] = (uint16_t)f32_to_bf16_bits(p.Ybase[o] + acc[i][j][e]);
      }
    }
}

int grid_of(int M, int ncols) {
  const int mt = (M + BM - 1) / BM, nt = ncols / BN;
  return XCDS * ((nt + XCDS - 1) / XCDS) * mt;
}

}  // namespace

hipError_t launch_proj(const ProjLaunch& p, hipStream_t s) {
  base_kernel<<<grid_of(p.M, p.Nout + p.r), THREADS, 0, s>>>(p);
  if (p.gate) lora_kernel<<<grid_of(p.M, p.Nout), THREADS, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace isd
