// LM head in front of verification (bf16): logits = hidden . w_lm^T, stored as bf16, with
// the verification's row statistics taken from the tile while it is still on chip.
//
// One ISD forward yields the anchor p on the clean rows and the proposal q on the [MASK]
// rows from the same block of 2N-1 rows (「首次超越 AR 模型」 "I-DLM 如何解決這些問題";
// 「I-DLM – introspektive Diffusion Language Models」 "Inference & ISD"); the vocabulary
// projection that produces those rows is this product.
//
// lmh_kernel   One workgroup per 224-row x 256-column tile, (2 x 112) x (4 x 64) over 8
//              waves, two per SIMD, each wave 7 x 4 blocks of v_mfma_f32_16x16x32_bf16.
//              Both operands are K-contiguous (hidden rows, w_lm rows), so a k step of 32
//              is 30 MFMA fragments of 16 rows x 64 bytes (14 of hidden, 16 of w_lm), which
//              the waves load straight into LDS
//              (global_load_lds_dwordx4: lane l's 16 bytes land at slot l).  For coalescing,
//              four consecutive lanes read one row's 64 contiguous bytes: lane l takes row
//              l / 4 of the fragment and 16-byte chunk (l % 4) ^ (row / 4), so chunk c of
//              row r sits at slot 4 r + (c ^ (r / 4)), where the MFMA lane holding
//              (r, c) reads it -- the xor keeps every 16-lane read on distinct banks.  A
//              ring of RING slots keeps RING - 1 steps of loads in flight; one barrier per
//              step, after which the waves read the next step's fragments while the current
//              step's MFMAs run.
//              The epilogue rounds the tile to bf16 (nearest even), passes it through LDS so
//              that every lane stores 32 contiguous bytes of a row, and -- when statistics are
//              asked for -- reduces each row's 128 values to a mini-chunk record: the max m of
//              the stored values, the lowest column holding it, and the sum of
//              2^(l c2 - K) with K = fp32(m c2).
// lmh_merge_kernel  One wave per row and 64 sub-chunks: mini-chunk records -> the verification's chunk
//              records (16384 columns: max, lowest argmax, K = fp32(max c2)) and sub-chunk
//              sums (1024 columns) against the chunk's K, rescaled and added in fp64 in
//              column order.  The walk, residual and draw kernels then run unchanged.
#include <limits.h>

#include "device.h"
#include "launch.h"
#include "lds_dma.h"
#include "tiles.h"

namespace isd {
namespace {

constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int TBM = 224;            // rows per workgroup
constexpr int TBN = 256;            // columns per workgroup
constexpr int WM = TBM / 2;         // 112 rows per wave (waves 2 in M x 4 in N)
constexpr int WN = TBN / 4;         // 64 columns per wave
constexpr int BN = LMH_MINI;        // 128 columns per mini-chunk record
constexpr int RB = WM / 16;         // 7 row blocks per wave
constexpr int CB = WN / 16;         // 4 column blocks per wave
constexpr int AF = TBM / 16;        // 14 hidden fragments per k step
constexpr int BF = TBN / 16;        // 16 w_lm fragments per k step
constexpr int NF = AF + BF;         // 30 fragments (1 KB each) per k step
constexpr int LPW = (NF + WAVES - 1) / WAVES;  // loads per wave per step: 4 (waves 0..5), 3 (6..7)
constexpr int RING = 4;             // LDS slots: RING - 1 k steps of loads in flight
constexpr int SLOT = NF * 1024;     // bytes per slot
constexpr int LROW = TBN + 8;       // LDS row stride of the epilogue tile, in bf16
static_assert(BN == 128 && TBN == 2 * BN && TBM % 16 == 0, "tile shape: two mini-chunks per row");
static_assert(VCHUNK % BN == 0 && VSUB % BN == 0, "mini-chunks tile the chunks");
static_assert((size_t)TBM * LROW * 2 <= (size_t)RING * SLOT, "the epilogue tile fits in the ring");

__global__ __launch_bounds__(THREADS, 1) void lmh_kernel(const LmhLaunch p) {
  const int mt = (p.M + TBM - 1) / TBM, nt = (p.NMINI + 1) / 2;
  int tm, tn;
  if (!tile_of(blockIdx.x, mt, nt, tm, tn)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int wm = wave >> 2, wn = wave & 3;
  const int l16 = lane & 15;
  const int m0 = tm * TBM, n0 = tn * TBN;
  const int S = p.Dm / 32;

  // LDS: RING slots of NF fragments during the K loop, then the bf16 output tile.
  __shared__ __attribute__((aligned(16))) unsigned char smem[RING * SLOT];

  // This wave's fragment loads: fragment f = wave + 8 i (i < LPW, f < NF); f < AF is
  // hidden row block f, else w_lm block f - AF.  Rows past M read row M-1 and columns
  // past V read row V-1 of w_lm (in bounds; never stored).  Lane l loads row l / 4 of the
  // fragment, chunk (l % 4) ^ (row / 4).
  const uint16_t* src[LPW];
  int dst[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int f = min(wave + WAVES * i, NF - 1);
    const int fr_row = lane >> 2, fr_chunk = (lane & 3) ^ (fr_row >> 2);
    src[i] = f < AF ? p.hidden + (size_t)min(m0 + 16 * f + fr_row, p.M - 1) * p.Dm + 8 * fr_chunk
                    : p.w + (size_t)min(n0 + 16 * (f - AF) + fr_row, p.V - 1) * p.Dm + 8 * fr_chunk;
    dst[i] = f * 1024;
  }
  const bool extra = wave < NF - (LPW - 1) * WAVES;  // this wave has an LPW-th fragment
  auto issue = [&](int step) {
    unsigned char* slot = smem + (step % RING) * SLOT;
    const int k = 32 * min(step, S - 1);  // steps past the end re-load the last (dead slots)
#pragma unroll
    for (int i = 0; i < LPW - 1; ++i) load_frag(src[i] + k, slot + dst[i]);
    if (extra) load_frag(src[LPW - 1] + k, slot + dst[LPW - 1]);
  };

  f32x4 acc[RB][CB];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Fragments of step s + 1 are read from LDS while step s's MFMAs run: at step s the
  // wait covers step s + 1's loads, and the barrier then makes them visible.
  struct Frag { u32x4 a[RB], b[CB]; };
  auto read = [&](Frag& F, int step) {
    const u32x4* fr = reinterpret_cast<const u32x4*>(smem + (step % RING) * SLOT);
    const int rd = 4 * l16 + ((lane >> 4) ^ (l16 >> 2));
#pragma unroll
    for (int j = 0; j < CB; ++j) F.b[j] = fr[(AF + CB * wn + j) * 64 + rd];
#pragma unroll
    for (int i = 0; i < RB; ++i) F.a[i] = fr[(RB * wm + i) * 64 + rd];
  };
  auto sync_next = [&]() {
    if (extra) wait_vmcnt<LPW>();
    else wait_vmcnt<LPW - 1>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  };
  auto body = [&](int s, const Frag& cur, Frag& nxt) {
    sync_next();
    issue(s + RING - 1);
    read(nxt, s + 1);
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int j = 0; j < CB; ++j) acc[i][j] = mfma16x16x32(cur.a[i], cur.b[j], acc[i][j]);
  };
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) issue(u);
  Frag F0, F1;
  if (extra) wait_vmcnt<LPW>();
  else wait_vmcnt<LPW - 1>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  read(F0, 0);
  int s = 0;
  for (; s + 2 <= S; s += 2) {
    body(s, F0, F1);
    body(s + 1, F1, F0);
  }
  if (s < S) body(s, F0, F1);
  wait_vmcnt<0>();
  __syncthreads();  // the ring is dead: reuse it as the output tile

  // ---- epilogue: bf16 tile through LDS, coalesced stores, mini-chunk records
  uint16_t(*t)[LROW] = reinterpret_cast<uint16_t(*)[LROW]>(smem);
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < CB; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        t[WM * wm + 16 * i + 4 * (lane >> 4) + e][WN * wn + 16 * j + l16] =
            (uint16_t)f32_to_bf16_bits(acc[i][j][e]);
  __syncthreads();

  // wave w: tile rows 28 w .. 28 w + 27, sixteen lanes per row (16 columns each); lanes
  // 0..7 and 8..15 of a row are its two mini-chunks
  constexpr int RPW = TBM / WAVES;
  const int q = lane & 15;
  const float c2 = p.c2;
  for (int pass = 0; pass < RPW / 4; ++pass) {
    const int rl = RPW * wave + 4 * pass + (lane >> 4);
    const int row = m0 + rl;
    const int cbase = n0 + 16 * q;
    const int mini = 2 * tn + (q >> 3);
    u32x4 w2[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) w2[h] = *reinterpret_cast<const u32x4*>(&t[rl][16 * q + 8 * h]);
    if (row < p.M) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c0 = cbase + 8 * h;  // V % 8 == 0: a 16-byte group is all in or all out
        if (c0 < p.V) *reinterpret_cast<u32x4*>(p.logits + (size_t)row * p.V + c0) = w2[h];
      }
    }
    if (!p.mmax) continue;
    float x[16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * h + 2 * e] = bf16_lo(w2[h][e]);
        x[8 * h + 2 * e + 1] = bf16_hi(w2[h][e]);
      }
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (cbase + k >= p.V) x[k] = -__builtin_inff();
    float m = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < 16; ++k) m = fmaxf(m, x[k]);
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    const float K = __fmul_rn(m, c2);
    int arg = INT_MAX;
#pragma unroll
    for (int k = 15; k >= 0; --k)
      if (x[k] == m) arg = cbase + k;
    arg = min(arg, __shfl_xor(arg, 1));
    arg = min(arg, __shfl_xor(arg, 2));
    arg = min(arg, __shfl_xor(arg, 4));
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) sum += exp2_hw(fmaf(x[k], c2, -K));
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    if ((q & 7) == 0 && row < p.M && mini < p.NMINI) {
      const size_t o = (size_t)row * p.NMS + mini;
      p.mmax[o] = m;
      p.msum[o] = sum;
      p.marg[o] = arg;
    }
  }
}

// Wave (row m = b R + rr, round t): mini-chunk records -> chunk records and sub-chunk sums
// at verification row b RR + rr, for sub-chunks 64 t .. 64 t + 63.  Lane l takes
// sub-chunk 64 t + l (its 8 records are 32 aligned bytes per array); the 16 lanes of a
// 16-lane group are the 16 sub-chunks of one chunk.
__global__ __launch_bounds__(256) void lmh_merge_kernel(const LmhLaunch p) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= p.M) return;
  const int b = m / p.R, rr = m - b * p.R;
  const size_t rowid = (size_t)b * p.RR + rr;
  const bool proposal = rr >= p.N - 1;
  const float c2 = p.c2;
  constexpr int MPS = VSUB / BN;  // mini-chunks per sub-chunk
  static_assert(MPS == 8, "two 16-byte loads per array and lane");
  const int j = 64 * blockIdx.y + lane;
  const bool valid = j < p.NSUB;
  const int jc = valid ? j : 0;
  const size_t o = (size_t)m * p.NMS + (size_t)MPS * jc;  // 32-byte aligned (NMS % 8 == 0)
  float mt[MPS], stt[MPS];
  int at[MPS];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p.mmax + o + 4 * h);
    const f32x4 b4 = *reinterpret_cast<const f32x4*>(p.msum + o + 4 * h);
    const u32x4 c = *reinterpret_cast<const u32x4*>(p.marg + o + 4 * h);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mt[4 * h + e] = a[e];
      stt[4 * h + e] = b4[e];
      at[4 * h + e] = (int)c[e];
    }
  }
  // records past the row's last mini-chunk are padding (never written): masked here
#pragma unroll
  for (int t = 0; t < MPS; ++t)
    if (!valid || MPS * j + t >= p.NMINI) {
      mt[t] = -__builtin_inff();
      stt[t] = 0.f;
      at[t] = INT_MAX;
    }
  float sm = -__builtin_inff();
  int sa = INT_MAX;
#pragma unroll
  for (int t = 0; t < MPS; ++t)
    if (mt[t] > sm) {  // strictly greater: ties keep the lower column
      sm = mt[t];
      sa = at[t];
    }
  float M = sm;
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) M = fmaxf(M, __shfl_xor(M, d));
  int A = (sm == M) ? sa : INT_MAX;
#pragma unroll
  for (int d = 8; d >= 1; d >>= 1) A = min(A, __shfl_xor(A, d));
  const float Kc = __fmul_rn(M, c2);
  double acc = 0.0;
#pragma unroll
  for (int t = 0; t < MPS; ++t)
    if (mt[t] > -__builtin_inff())
      acc += (double)stt[t] * exp2((double)__fmul_rn(mt[t], c2) - (double)Kc);
  if (valid) {
    p.csub[rowid * p.NSUB + j] = (float)acc;
    if ((lane & 15) == 0) {
      const int c = j / VCHUNK_SUBS;
      p.cmax[rowid * p.SV + c] = M;
      p.cref[rowid * p.SV + c] = Kc;
      p.cidx[rowid * p.SV + c] = proposal ? A : INT_MAX;
    }
  }
}

}  // namespace

hipError_t launch_lm_head(const LmhLaunch& p, hipStream_t s) {
  const int mt = (p.M + TBM - 1) / TBM;
  lmh_kernel<<<tile_grid(mt, (p.NMINI + 1) / 2), THREADS, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_lm_head_merge(const LmhLaunch& p, hipStream_t s) {
  lmh_merge_kernel<<<dim3((p.M + 3) / 4, (p.NSUB + 63) / 64), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace isd
