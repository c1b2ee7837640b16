// R-ISD gated projection on weights packed in MFMA fragment order (bf16 in/out):
//   Y = X W + gate * bf16(X A) B,
// the same product and the same rows-with-gate-0-are-base-only guarantee as the row-major
// kernels (「首次超越 AR 模型」 "無損 R-ISD"; 「内省扩散语言模型」 "1. 引言";
// 「I-DLM – introspektive Diffusion Language Models」 "Lossless R-ISD").
//
// Packed layout.  A weight matrix S of n rows (output columns) by k (the contraction)
// is stored as 1 KB fragments: fragment (nb, kb), nb < n/16, kb < k/32, holds
// S[16 nb + l % 16][32 kb + 8 (l / 16) + e] at element ((nb (k/32) + kb) 64 + l) 8 + e,
// i.e. exactly the B operand of v_mfma_f32_16x16x32_bf16 for lane l.  The packed buffer
// holds S = [W^T; A^T] (Nout + r rows of K) in that order, then B^T (Nout rows of r)
// row-major: the second kernel (K = r, two k steps) is the row-major one.
//
// With the weights in that order every wave loads its B operands straight from memory
// with 1 KB fully coalesced loads, and only the activation tile goes through LDS (stored
// as fragments with the same conflict-free xor swizzle as the row-major kernels).
// Tiles: 64 x 128 per workgroup, 8 waves of 64 x 16 (4 x 1 MFMA 16x16x32 blocks) when the
// grid is one round, else 4 waves of 64 x 32 (4 x 2 blocks); K in steps of 64 with three
// steps of loads in flight.
#include "device.h"
#include "launch.h"
#include "tiles.h"

namespace isd {
namespace {

constexpr int BM = PROJ_BM, BN = PROJ_BN, BK = PROJ_BK;
constexpr int RING = 4;                         // register stages of the load pipeline
constexpr int FRAG = 64 * 8;                    // elements in one packed 16 x 32 fragment

// ---------------------------------------------------------------- packing
// One thread per 16 bytes of the packed buffer: S = [W^T; A^T] in fragment order, then
// B^T as it is (the second kernel reads it row-major).  KN = false reads the
// linear-layer storage w [Nout, K], a [r, K], b [Nout, r]; KN = true reads the
// y = x W storage w [K, Nout], a [K, r], b [r, Nout] (eight strided 2-byte reads per
// thread; sixteen lanes read sixteen consecutive columns of one row, and packing is done
// once per weight set).
template <bool KN>
__global__ __launch_bounds__(256) void pack_kernel(const uint16_t* __restrict__ w,
                                                   const uint16_t* __restrict__ a,
                                                   const uint16_t* __restrict__ b,
                                                   uint16_t* __restrict__ packed, int K, int Nout,
                                                   int r) {
  const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long gS = (long long)(Nout + r) * K / 8, gB = (long long)Nout * r / 8;
  if (g >= gS + gB) return;
  u32x4 v;
  if (g >= gS) {
    const long long h = g - gS;  // elements 8h .. 8h + 7 of B^T: row n, ranks j .. j + 7
    if constexpr (KN) {
      const int n = (int)(h * 8 / r), j = (int)(h * 8 % r);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = (uint32_t)b[(size_t)(j + 2 * e) * Nout + n] | ((uint32_t)b[(size_t)(j + 2 * e + 1) * Nout + n] << 16);
    } else {
      v = *reinterpret_cast<const u32x4*>(b + (size_t)h * 8);
    }
    *reinterpret_cast<u32x4*>(packed + (size_t)(Nout + r) * K + (size_t)h * 8) = v;
    return;
  }
  const int lane = (int)(g & 63);
  const long long frag = g >> 6;
  const int kb = (int)(frag % (K / 32)), nb = (int)(frag / (K / 32));
  const int row = nb * 16 + (lane & 15), col = kb * 32 + 8 * (lane >> 4);  // S[row][col .. col + 7]
  if constexpr (KN) {
    const uint16_t* src = row < Nout ? w + (size_t)col * Nout + row : a + (size_t)col * r + (row - Nout);
    const size_t ld = row < Nout ? (size_t)Nout : (size_t)r;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (uint32_t)src[(2 * e) * ld] | ((uint32_t)src[(2 * e + 1) * ld] << 16);
  } else {
    const uint16_t* src = row < Nout ? w + (size_t)row * K + col : a + (size_t)(row - Nout) * K + col;
    v = *reinterpret_cast<const u32x4*>(src);
  }
  *reinterpret_cast<u32x4*>(packed + (size_t)g * 8) = v;
}

// ---------------------------------------------------------------- product
// The tile's 128 columns are split over WAVES waves (4: 32 columns each, 8: 16 each).
// Every output element gets the same MFMA sequence either way, so the results do not
// depend on the wave count; 8 waves hide more latency when the grid is one round.
template <int WAVES>
struct Shape {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int CBW = BN / 16 / WAVES;            // column blocks per wave
  static constexpr int A_LOADS = BM * BK / 8 / THREADS;  // 16-byte activation loads per thread per k step
  static constexpr int ROWS = THREADS / 8;               // activation rows per load round
};

template <int WAVES>
struct Stage {
  u32x4 a[Shape<WAVES>::A_LOADS];
  u32x4 b[Shape<WAVES>::CBW][2];  // this wave's weight fragments [column block][k half]
};

// LDS activation tile: MFMA fragments [k half][16-row block][slot].  Row r, 16-byte k chunk
// c (0..7) lives in fragment (c / 4, r / 16) at slot (c % 4) * 16 + ((r % 16) ^ c).
struct ATile {
  u32x4 f[2][BM / 16][64];
};

__device__ __forceinline__ int chunk_slot(int r, int c) { return (c & 3) * 16 + ((r & 15) ^ c); }

template <int WAVES>
__device__ __forceinline__ void issue(Stage<WAVES>& st, const uint16_t* const (&pa)[Shape<WAVES>::A_LOADS],
                                      const uint16_t* const (&pb)[Shape<WAVES>::CBW], int s) {
#pragma unroll
  for (int i = 0; i < Shape<WAVES>::A_LOADS; ++i) st.a[i] = *reinterpret_cast<const u32x4*>(pa[i] + s * BK);
#pragma unroll
  for (int cb = 0; cb < Shape<WAVES>::CBW; ++cb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      st.b[cb][kk] = *reinterpret_cast<const u32x4*>(pb[cb] + (size_t)(2 * s + kk) * FRAG);
}

template <int WAVES>
__device__ __forceinline__ void put(ATile& t, const Stage<WAVES>& st, int tid) {
  const int c = tid & 7;
#pragma unroll
  for (int i = 0; i < Shape<WAVES>::A_LOADS; ++i) {
    const int r = (tid >> 3) + Shape<WAVES>::ROWS * i;
    t.f[c >> 2][r >> 4][chunk_slot(r, c)] = st.a[i];
  }
}

struct Frags {
  u32x4 a[2][BM / 16];  // [k half][row block]
};

__device__ __forceinline__ void fetch_frags(Frags& f, const ATile& t, int lane) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int slot = lane ^ (kk * 4 + (lane >> 4));
#pragma unroll
    for (int rb = 0; rb < BM / 16; ++rb) f.a[kk][rb] = t.f[kk][rb][slot];
  }
}

template <int WAVES>
__device__ __forceinline__ void mma(const Frags& f, const Stage<WAVES>& st,
                                    f32x4 (&acc)[BM / 16][Shape<WAVES>::CBW]) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int rb = 0; rb < BM / 16; ++rb)
#pragma unroll
      for (int cb = 0; cb < Shape<WAVES>::CBW; ++cb)
        acc[rb][cb] = mfma16x16x32(f.a[kk][rb], st.b[cb][kk], acc[rb][cb]);
}

// acc[rb][cb] = sum over k < K of X[16 rb + row][k] S[16 (CBW wave + cb) + col][k] for the
// 64 x 128 tile at X and the packed fragments at Sp (the tile's first 16-column block, at
// the first k of the part; Kfull is the weights' full K).
// X rows past `mrows` read row mrows - 1 (never stored).  At step s: loads for step
// s + RING - 1 go out, step s + 2's activations go to LDS, step s + 1's activation
// fragments come from LDS, and step s's MFMAs run.
template <int WAVES>
__device__ void gemm_tile(ATile (&lds)[2], const uint16_t* __restrict__ X, int ldx, int mrows,
                          const uint16_t* __restrict__ Sp, int Kfull, int K, int tid, int wave, int lane,
                          f32x4 (&acc)[BM / 16][Shape<WAVES>::CBW]) {
  static_assert(RING % 2 == 0 && RING >= 4, "fragment buffers alternate with the step parity");
  constexpr int A_LOADS = Shape<WAVES>::A_LOADS, CBW = Shape<WAVES>::CBW;
  const int KB = Kfull / 32;  // fragments per 16-column block of the packed weights
  const uint16_t* pa[A_LOADS];
  const uint16_t* pb[CBW];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i)
    pa[i] = X + (size_t)min((tid >> 3) + Shape<WAVES>::ROWS * i, mrows - 1) * ldx + (tid & 7) * 8;
#pragma unroll
  for (int cb = 0; cb < CBW; ++cb) pb[cb] = Sp + ((size_t)(CBW * wave + cb) * KB) * FRAG + lane * 8;
#pragma unroll
  for (int rb = 0; rb < BM / 16; ++rb)
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int S = K / BK;
  Stage<WAVES> r[RING];
  Frags f[2];
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) issue<WAVES>(r[u], pa, pb, min(u, S - 1));
  put<WAVES>(lds[0], r[0], tid);
  put<WAVES>(lds[1], r[1], tid);
  lds_barrier();
  fetch_frags(f[0], lds[0], lane);
  lds_barrier();  // every wave has read buffer 0 before step 0 refills it with step 2
  // Steps past the end re-load and re-stage the last step (unconditional loads keep the
  // compiler's wait counts exact); only the MFMAs are skipped.
  for (int s0 = 0; s0 < S; s0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      const int s = s0 + u;
      issue<WAVES>(r[(u + RING - 1) % RING], pa, pb, min(s + RING - 1, S - 1));
      fetch_frags(f[(u + 1) & 1], lds[(s + 1) & 1], lane);
      put<WAVES>(lds[s & 1], r[(u + 2) % RING], tid);
      if (s < S) mma<WAVES>(f[u & 1], r[u], acc);
      lds_barrier();
    }
  }
}

template <int WAVES>
__global__ __launch_bounds__(Shape<WAVES>::THREADS) void base_kernel_packed(const ProjLaunch p) {
  constexpr int CBW = Shape<WAVES>::CBW;
  const int mt = (p.M + BM - 1) / BM, nt = (p.Nout + p.r) / BN;
  int tm, tn;
  if (!tile_of(blockIdx.x, mt, nt * p.ksplit, tm, tn)) return;
  const int ks = tn % p.ksplit, klen = p.K / p.ksplit, k0 = ks * klen;  // this part of K
  tn /= p.ksplit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int m0 = tm * BM, n0 = tn * BN;
  const int mrows = min(BM, p.M - m0);
  const bool lowrank = n0 >= p.Nout;  // this tile computes T = X A
  const size_t blk = (size_t)(p.K / 32) * FRAG;  // elements per packed 16-column block
  __shared__ ATile lds[2];
  f32x4 acc[BM / 16][CBW];
  gemm_tile<WAVES>(lds, p.X + (size_t)m0 * p.K + k0, p.K, mrows, p.Sp + (size_t)(n0 / 16) * blk + (size_t)(k0 / 32) * FRAG,
            p.K, klen, tid, wave, lane, acc);
  if (p.ksplit > 1) {  // partial sums; the reduce kernel adds them in order and stores
    const int ncols = p.Nout + p.r;
#pragma unroll
    for (int rb = 0; rb < BM / 16; ++rb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rb * 16 + 4 * gq + e;
        if (row >= mrows) continue;
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb)
          p.part[((size_t)ks * p.M + m0 + row) * ncols + n0 + wave * 16 * CBW + cb * 16 + l16] = acc[rb][cb][e];
      }
    return;
  }
#pragma unroll
  for (int rb = 0; rb < BM / 16; ++rb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = rb * 16 + 4 * gq + e;
      if (row >= mrows) continue;
      const int gr = m0 + row;
      const bool gated = p.gate != nullptr && p.gate[gr] != 0;
#pragma unroll
      for (int cb = 0; cb < CBW; ++cb) {
        const int col = n0 + wave * 16 * CBW + cb * 16 + l16;
        const float v = acc[rb][cb][e];
        if (lowrank)
          p.T[(size_t)gr * p.r + (col - p.Nout)] = (uint16_t)f32_to_bf16_bits(v);
        else if (gated)
          p.Ybase[(size_t)gr * p.Nout + col] = v;
        else
          p.Y[(size_t)gr * p.Nout + col] = (uint16_t)f32_to_bf16_bits(v);
      }
    }
}

}  // namespace

hipError_t launch_proj_packed(const ProjLaunch& p, hipStream_t s) {
  if (p.big) return launch_proj_big(p, true, s);
  const int mt = (p.M + BM - 1) / BM, tiles = mt * (p.Nout + p.r) / BN * p.ksplit;
  // eight waves per tile when every tile gets a CU of its own (at most one workgroup of
  // 8 waves is resident per CU), else four, two workgroups sharing a CU
  if (tiles <= 256)
    base_kernel_packed<8><<<tile_grid(mt, (p.Nout + p.r) / BN * p.ksplit), Shape<8>::THREADS, 0, s>>>(p);
  else
    base_kernel_packed<4><<<tile_grid(mt, (p.Nout + p.r) / BN * p.ksplit), Shape<4>::THREADS, 0, s>>>(p);
  if (p.ksplit > 1) {
    const hipError_t e = launch_proj_reduce(p, s);
    if (e != hipSuccess) return e;
  }
  if (p.gate) return launch_lora(p, s);  // K = r: the row-major kernel on B^T as stored
  return hipGetLastError();
}

hipError_t launch_pack_proj(const uint16_t* w, const uint16_t* a, const uint16_t* b, uint16_t* packed,
                            int K, int Nout, int r, bool kn, hipStream_t s) {
  const long long groups = (long long)(Nout + r) * K / 8 + (long long)Nout * r / 8;
  const unsigned grid = (unsigned)((groups + 255) / 256);
  if (kn)
    pack_kernel<true><<<grid, 256, 0, s>>>(w, a, b, packed, K, Nout, r);
  else
    pack_kernel<false><<<grid, 256, 0, s>>>(w, a, b, packed, K, Nout, r);
  return hipGetLastError();
}

}  // namespace isd
