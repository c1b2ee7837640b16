// Large-tile, split-K base product of the R-ISD gated projection (bf16 in, fp32 partial
// sums out), for calls whose 64 x 128 tiles would read many times the weight from L2 and
// whose K is long enough to pay for partial sums: e.g. 448 rows (64 requests x 7) against
// the 12288-wide down projection of a Qwen3-8B layer.
//
// The product is the one of the 64 x 128 kernels: the stacked weight S = [W^T; A^T]
// (Nout + r rows of K), whose W^T rows give the base product and whose A^T rows give
// T = X A for the delta on gated rows (「首次超越 AR 模型」 "無損 R-ISD"; 「内省扩散语言模型」
// "1. 引言"; 「I-DLM – introspektive Diffusion Language Models」 "Lossless R-ISD").
//
// Output tiles are 224 x 256 and K is cut into `ksplit` ranges of whole 32-wide steps,
// so that tiles x ranges fill the chip in one round.  Workgroup (tile, range) runs the LM
// head's pipeline over its range -- 8 waves, two per SIMD, each 112 x 64 = 7 x 4 blocks of
// v_mfma_f32_16x16x32_bf16, operand fragments streamed into an LDS ring by
// global_load_lds with RING - 1 steps in flight -- and writes its fp32 sums to
// part[range].  proj_reduce_kernel then adds the ranges in order and stores as the
// 64 x 128 kernels do (bf16 Y on rows with gate 0, fp32 on gated rows, bf16 T), and
// lora_kernel adds the delta on gated rows.
//
// A 32-wide k step of a 224 x 256 tile loads 30 KB for 3.67 MFLOP, against 12 KB for
// 0.52 MFLOP at 64 x 128: 2.7 times fewer operand bytes per flop.  The price is the fp32
// partials, ksplit x M x (Nout + r) x 4 bytes written once and read once.
//
// Row-major weights load with the coalesced lane mapping of lds_dma.h; packed weights
// (fragment order) are already one contiguous 1 KB block per fragment, lane l's 16 bytes
// being MFMA lane l's operand.  Both put the same values into the same MFMA lanes in the
// same order, so the two layouts give bit-identical results.
#include "device.h"
#include "launch.h"
#include "lds_dma.h"
#include "tiles.h"

namespace isd {
namespace {

constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int TBM = PROJ_BIG_TBM;              // rows per workgroup
constexpr int TBN = PROJ_BIG_TBN;              // stacked weight rows (output columns) per workgroup
constexpr int WM = TBM / 2;                    // 112 rows per wave (waves 2 in M x 4 in N)
constexpr int WN = TBN / 4;                    // 64 columns per wave
constexpr int RB = WM / 16;                    // 7 row blocks per wave
constexpr int CB = WN / 16;                    // 4 column blocks per wave
constexpr int AF = TBM / 16;                   // 14 activation fragments per k step
constexpr int BF = TBN / 16;                   // 16 weight fragments per k step
constexpr int NF = AF + BF;                    // 30 fragments (1 KB each) per k step
constexpr int LPW = (NF + WAVES - 1) / WAVES;  // loads per wave per step: 4 (waves 0..5), 3 (6..7)
constexpr int RING = 4;                        // LDS slots: RING - 1 k steps of loads in flight
constexpr int SLOT = NF * 1024;                // bytes per slot
constexpr int PFRAG = 64 * 8;                  // elements of one packed fragment

template <bool PACKED>
__global__ __launch_bounds__(THREADS, 1) void base_big_kernel(const ProjLaunch p) {
  const int ncols = p.Nout + p.r;  // stacked weight rows computed (r = 0: base only)
  const int mt = (p.M + TBM - 1) / TBM, nt = (ncols + TBN - 1) / TBN;
  int tm, tq;
  // tiles numbered range-major (tq = range nt + column tile), so the workgroups an XCD
  // runs share one or two activation ranges, and each weight range is read by the row
  // tiles next to it
  if (!tile_of(blockIdx.x, mt, nt * p.ksplit, tm, tq)) return;
  const int ks = tq / nt, tn = tq - ks * nt;
  const int S = p.K / 32;
  const int s0 = (int)((long long)ks * S / p.ksplit);
  const int n = (int)((long long)(ks + 1) * S / p.ksplit) - s0;  // k steps in this range, >= 1
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int wm = wave >> 2, wn = wave & 3;
  const int m0 = tm * TBM, n0 = tn * TBN;

  __shared__ __attribute__((aligned(16))) unsigned char smem[RING * SLOT];

  // This wave's fragment loads: fragment f = wave + 8 i (i < LPW, f < NF); f < AF is row
  // block f of X, else block f - AF of the stacked weight rows.  Rows past M read row M - 1
  // and stacked rows past Nout + r read the last one (in bounds; never stored).  Nout is a
  // multiple of 16, so every weight fragment lies wholly in W^T or wholly in A^T.
  const uint16_t* src[LPW];
  int stride[LPW];  // elements from one k step to the next
  int dst[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int f = min(wave + WAVES * i, NF - 1);
    if (f < AF) {
      src[i] = p.X + (size_t)min(m0 + 16 * f + frag_row(lane), p.M - 1) * p.K + 8 * frag_chunk(lane) + 32 * s0;
      stride[i] = 32;
    } else if (PACKED) {
      const int nb = min(n0 / 16 + (f - AF), ncols / 16 - 1);
      src[i] = p.Sp + ((size_t)nb * S + s0) * PFRAG + 8 * lane;
      stride[i] = PFRAG;
    } else {
      const int row = min(n0 + 16 * (f - AF) + frag_row(lane), ncols - 1);
      const uint16_t* base = row < p.Nout ? p.W + (size_t)row * p.K : p.A + (size_t)(row - p.Nout) * p.K;
      src[i] = base + 8 * frag_chunk(lane) + 32 * s0;
      stride[i] = 32;
    }
    dst[i] = f * 1024;
  }
  const bool extra = wave < NF - (LPW - 1) * WAVES;  // this wave has an LPW-th fragment
  auto issue = [&](int t) {
    unsigned char* slot = smem + (t % RING) * SLOT;
    const int k = min(t, n - 1);  // steps past the range re-load its last one (dead slots)
#pragma unroll
    for (int i = 0; i < LPW - 1; ++i) load_frag(src[i] + (size_t)k * stride[i], slot + dst[i]);
    if (extra) load_frag(src[LPW - 1] + (size_t)k * stride[LPW - 1], slot + dst[LPW - 1]);
  };

  f32x4 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragments of step t + 1 are read from LDS while step t's MFMAs run: at step t the wait
  // covers step t + 1's loads, and the barrier makes every wave's loads of it visible.
  struct Frag { u32x4 a[RB], b[CB]; };
  const int rda = frag_read_slot(lane);
  const int rdb = PACKED ? lane : rda;
  auto read = [&](Frag& F, int t) {
    const u32x4* fr = reinterpret_cast<const u32x4*>(smem + (t % RING) * SLOT);
#pragma unroll
    for (int j = 0; j < CB; ++j) F.b[j] = fr[(AF + CB * wn + j) * 64 + rdb];
#pragma unroll
    for (int i = 0; i < RB; ++i) F.a[i] = fr[(RB * wm + i) * 64 + rda];
  };
  auto sync_next = [&]() {
    if (extra) stage_barrier<LPW>();
    else stage_barrier<LPW - 1>();
  };
  auto body = [&](int t, const Frag& cur, Frag& nxt) {
    sync_next();
    issue(t + RING - 1);
    read(nxt, t + 1);
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) acc[i][j] = mfma16x16x32(cur.a[i], cur.b[j], acc[i][j]);
  };
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) issue(u);
  Frag F0, F1;
  sync_next();
  read(F0, 0);
  int t = 0;
  for (; t + 2 <= n; t += 2) {
    body(t, F0, F1);
    body(t + 1, F1, F0);
  }
  if (t < n) body(t, F0, F1);
  wait_vmcnt<0>();  // the dead loads of the last steps land before the workgroup ends

  // fp32 partial sums of this range: lane (l16, g) of block (i, j) holds rows 4 g .. 4 g + 3
  // of column l16, so 16 lanes store 64 contiguous bytes of a row
  const int l16 = lane & 15, g = lane >> 4;
  float* part = p.part + (size_t)ks * p.M * ncols;
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + WM * wm + 16 * i + 4 * g + e;
      if (row >= p.M) continue;
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        const int col = n0 + WN * wn + 16 * j + l16;
        if (col < ncols) part[(size_t)row * ncols + col] = acc[i][j][e];
      }
    }
}

}  // namespace

hipError_t launch_proj_big(const ProjLaunch& p, bool packed, hipStream_t s) {
  const int mt = (p.M + TBM - 1) / TBM, nt = (p.Nout + p.r + TBN - 1) / TBN;
  const int grid = tile_grid(mt, nt * p.ksplit);
  if (packed) base_big_kernel<true><<<grid, THREADS, 0, s>>>(p);
  else base_big_kernel<false><<<grid, THREADS, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_proj_reduce(p, s);
  if (e != hipSuccess || !p.gate) return e;
  return launch_lora(p, s);
}

}  // namespace isd
