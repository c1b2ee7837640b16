// The rate at which the chip reads the paged KV cache of an attention step: the reference
// the attention kernel's own rate is measured against.  It reads exactly the cached tiles
// an attention step reads -- pages 0 .. ceil(L_b / 16) - 1 of every request b and KV head,
// K and V (the paged KV cache of 「首次超越 AR 模型」 "實際部署：SGLang 整合") -- once each,
// and folds them into an XOR checksum; nothing of the method is computed.
//
// The (request, head, page) tiles form one flat list in the attention's item order, and
// wave g of a grid of G waves takes tiles g, g + G, g + 2G, ...: every wave holds the same
// number of tiles, so no balancing loss enters the rate.  One workgroup of 8 waves per CU,
// as the attention kernel runs, with two tiles of loads in flight per wave (one, two or
// four read at the same rate) and the next two tiles' page ids loaded ahead of them.
#include <atomic>

#include "device.h"
#include "launch.h"

namespace isd {
namespace {

constexpr int PAGE = ATTN_PAGE;
constexpr int WAVES = 8;
constexpr int NT = 2;  // tiles of loads in flight per wave

__device__ __forceinline__ uint32_t fold(u32x4 a) { return a[0] ^ a[1] ^ a[2] ^ a[3]; }

template <int D>
__global__ __launch_bounds__(64 * WAVES) void kv_sweep_kernel(const KvSweepLaunch c) {
  constexpr int LOADS = PAGE * D * 2 / 16 / 64;  // 16-byte loads per lane for one K (or V) tile
  constexpr size_t TILE_U4 = (size_t)PAGE * D * 2 / 16;
  __shared__ int pre[ATTN_MAX_B + 1];  // exclusive prefix of Hkv * pages(b)

  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (c.B + 63) / 64;
    const int b0 = min(c.B, lane * per), b1 = min(c.B, b0 + per);
    auto tiles_of = [&](int b) -> int {
      const int L = min(max(c.ctx_lens[b], 0), c.max_ctx_len);
      return c.Hkv * ((L + PAGE - 1) / PAGE);
    };
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += tiles_of(b);
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o);
      if (lane >= o) incl += t;
    }
    int run = incl - sum;
    for (int b = b0; b < b1; ++b) {
      pre[b] = run;
      run += tiles_of(b);
    }
    if (lane == 63) pre[c.B] = incl;
  }
  __syncthreads();

  const int total = pre[c.B];
  const int lane = threadIdx.x & 63;
  const int g = blockIdx.x * WAVES + (threadIdx.x >> 6), G = gridDim.x * WAVES;
  const u32x4* __restrict__ k = static_cast<const u32x4*>(c.k_cache);
  const u32x4* __restrict__ v = static_cast<const u32x4*>(c.v_cache);
  if (total <= 0) return;  // no cached tile (uniform across the workgroup)
  uint32_t x = 0;
  // The page ids of a batch's tiles are loaded one batch ahead, so the tiles' own loads
  // never wait on a page-table round trip (the attention kernel, too, loads the page ids
  // of a piece's pages ahead of them).
  int b = 0;  // request of the look-ahead tiles: they ascend, so b only moves on
  int idn[NT], hn[NT];
  auto look = [&](int i0n) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int i = min(i0n + G * t, total - 1);  // past the end: the last tile again, not folded
      while (pre[b + 1] <= i) ++b;
      const int n = (pre[b + 1] - pre[b]) / c.Hkv;  // pages of request b (>= 1: it holds tile i)
      const int rr = i - pre[b], h = rr / n, j = rr - h * n;
      idn[t] = c.page_table[(size_t)b * c.max_pages + j];
      hn[t] = h;
    }
  };
  look(g);
  for (int i0 = g; i0 < total; i0 += G * NT) {
    int id[NT], hh[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      id[t] = min(max(idn[t], 0), c.num_pages - 1);
      hh[t] = hn[t];
    }
    look(i0 + G * NT);
    u32x4 r[NT][2 * LOADS];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const size_t o = ((size_t)id[t] * c.Hkv + hh[t]) * TILE_U4;
#pragma unroll
      for (int q = 0; q < LOADS; ++q) {  // non-temporal, as the attention step reads them
        r[t][q] = __builtin_nontemporal_load(k + o + q * 64 + lane);
        r[t][LOADS + q] = __builtin_nontemporal_load(v + o + q * 64 + lane);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (i0 + G * t < total)
#pragma unroll
        for (int q = 0; q < 2 * LOADS; ++q) x ^= fold(r[t][q]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  if (lane == 0 && x != 0) atomicXor(c.checksum, x);
}

}  // namespace

hipError_t launch_kv_sweep(const KvSweepLaunch& c, hipStream_t s) {
  // one workgroup per CU; the CU count is queried once per device
  static std::atomic<int> cus_of_device[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cus = (dev >= 0 && dev < 64) ? cus_of_device[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cus = max(1, cus);
    if (dev >= 0 && dev < 64) cus_of_device[dev].store(cus, std::memory_order_relaxed);
  }
  if (c.D == 128) kv_sweep_kernel<128><<<cus, 64 * WAVES, 0, s>>>(c);
  else kv_sweep_kernel<64><<<cus, 64 * WAVES, 0, s>>>(c);
  return hipGetLastError();
}

}  // namespace isd
