// bf16 GEMM C[M,N] = A[M,K] B[N,K]^T on gfx950 MFMA, with the R-ISD gated-LoRA epilogue.
//
// R-ISD (page 1 "無損 R-ISD"; page 5 "Lossless R-ISD"): the LoRA delta is added only on
// gated ([MASK]) rows; verify rows keep the base product, bit for bit.  Here the delta
// T B^T (T = bf16(X A), computed by a first call of the same kernel) is added in the
// epilogue of the base product, after the base accumulation is complete, and selected
// per row -- so rows with gate 0 leave exactly the bits of a gate-free call.
//
// Tiling: 128x128 workgroup tile, 4 waves of 64x64 (4x4 MFMA 16x16x32 blocks), K in
// steps of 64 through LDS with register prefetch of the next step.  Split-K for
// occupancy: each split writes an fp32 partial; the last split of a tile to finish
// (counter in the workspace) sums the partials in split order, so results do not
// depend on timing.
#include "device.h"
#include "launch.h"

namespace isd {
namespace {

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;
constexpr int LDP = BK + 8;  // padded LDS row (elements)
constexpr int THREADS = 256;

struct Tiles {
  uint16_t a[BM][LDP];
  uint16_t b[BN][LDP];
};

// Global -> registers: 4 x 16 B per thread for each operand tile.
__device__ __forceinline__ void fetch(const uint16_t* __restrict__ src, int rows_valid, int ld,
                                      int k, int tid, u32x4 (&r)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = tid + THREADS * p;
    const int row = idx >> 3, c8 = idx & 7;
    r[p] = (row < rows_valid) ? *reinterpret_cast<const u32x4*>(src + (size_t)row * ld + k + c8 * 8)
                              : u32x4{0u, 0u, 0u, 0u};
  }
}
__device__ __forceinline__ void stash(uint16_t (*dst)[LDP], int tid, const u32x4 (&r)[4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = tid + THREADS * p;
    *reinterpret_cast<u32x4*>(&dst[idx >> 3][(idx & 7) * 8]) = r[p];
  }
}

// acc += A_tile[rows of this wave] * B_tile[cols of this wave]^T over one BK step.
__device__ __forceinline__ void mma_step(const Tiles& t, int wm, int wn, int lane,
                                         f32x4 (&acc)[4][4]) {
  const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < BK / 32; ++kk) {
    u32x4 af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      af[i] = *reinterpret_cast<const u32x4*>(&t.a[wm * 64 + i * 16 + l16][kk * 32 + 8 * g]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const u32x4*>(&t.b[wn * 64 + j * 16 + l16][kk * 32 + 8 * g]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
  }
}

// acc = sum over k in [k0, k1) of A[m0.., k] B[n0.., k]
__device__ void gemm_range(Tiles& t, const uint16_t* __restrict__ A, int lda, int mrows,
                           const uint16_t* __restrict__ B, int ldb, int nrows, int k0, int k1,
                           int tid, int wm, int wn, int lane, f32x4 (&acc)[4][4]) {
  u32x4 ra[4], rb[4];
  fetch(A, mrows, lda, k0, tid, ra);
  fetch(B, nrows, ldb, k0, tid, rb);
  for (int k = k0; k < k1; k += BK) {
    __syncthreads();
    stash(t.a, tid, ra);
    stash(t.b, tid, rb);
    __syncthreads();
    if (k + BK < k1) {
      fetch(A, mrows, lda, k + BK, tid, ra);
      fetch(B, nrows, ldb, k + BK, tid, rb);
    }
    mma_step(t, wm, wn, lane, acc);
  }
}

__global__ __launch_bounds__(THREADS) void gemm_kernel(const GemmLaunch g) {
  const int tn = blockIdx.x, tm = blockIdx.y, ks = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l16 = lane & 15, gq = lane >> 4;
  const int m0 = tm * BM, n0 = tn * BN;
  const int mrows = min(BM, g.M - m0);
  __shared__ Tiles t;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kper = g.K / g.splits;
  gemm_range(t, g.A + (size_t)m0 * g.K, g.K, mrows, g.B + (size_t)n0 * g.K, g.K, BN,
             ks * kper, (ks + 1) * kper, tid, wm, wn, lane, acc);

  if (g.splits > 1) {
    float* part = g.part + (size_t)ks * g.M * g.N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = wm * 64 + i * 16 + 4 * gq + e;
          if (row < mrows)
            part[(size_t)(m0 + row) * g.N + n0 + wn * 64 + j * 16 + l16] = acc[i][j][e];
        }
    __threadfence();
    __shared__ int s_last;
    __syncthreads();
    if (tid == 0) {
      const uint32_t prev = atomicAdd(&g.counters[tm * gridDim.x + tn], 1u);
      s_last = (prev == (uint32_t)(g.splits - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = wm * 64 + i * 16 + 4 * gq + e;
          float s = 0.f;
          if (row < mrows)
            for (int z = 0; z < g.splits; ++z)
              s += g.part[((size_t)z * g.M + m0 + row) * g.N + n0 + wn * 64 + j * 16 + l16];
          acc[i][j][e] = s;
        }
    if (tid == 0) g.counters[tm * gridDim.x + tn] = 0u;
  }

  // gated low-rank delta on the finished base product
  const bool lora = g.T != nullptr && g.gate != nullptr;
  f32x4 dl[4][4];
  if (lora) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) dl[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    gemm_range(t, g.T + (size_t)m0 * g.r, g.r, mrows, g.Bl + (size_t)n0 * g.r, g.r, BN, 0, g.r,
               tid, wm, wn, lane, dl);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = wm * 64 + i * 16 + 4 * gq + e;
        if (row >= mrows) continue;
        float y = acc[i][j][e];
        if (lora && g.gate[m0 + row]) y = y + dl[i][j][e];
        g.C[(size_t)(m0 + row) * g.N + n0 + wn * 64 + j * 16 + l16] = (uint16_t)f32_to_bf16_bits(y);
      }
}

}  // namespace

hipError_t launch_gemm(const GemmLaunch& g, hipStream_t s) {
  const dim3 grid(g.N / BN, (g.M + BM - 1) / BM, g.splits);
  gemm_kernel<<<grid, THREADS, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace isd
