// Conversion between the logical paged-cache layout [num_pages][Hkv][16][D] (one row of D
// values per token slot) and the tile layout isd_attention_step reads (include/isd.h):
//   K  [num_pages][Hkv][D/8][16][8]       -- 8-dim blocks of the 16 slots, the A operand of
//                                            S^T = K Q^T loaded 1 KB per wave
//   V  [num_pages][Hkv][D/16][4][16][4]   -- 4-slot groups of 16 dims, the A operand of
//                                            O^T = V^T P^T loaded 512 B per wave
// Both directions are plain permutations (bit copies): one thread per 16 bytes of K (8
// consecutive dims of a slot, 16-byte loads and stores for bf16) and per 4 slots x 1 dim
// of V (a gather of 4 values 1 row apart into 4 consecutive elements).
#include "device.h"
#include "launch.h"

namespace isd {
namespace {

constexpr int PAGE = ATTN_PAGE;

// K: unit (p, h, d8, t) = dims 8 d8 .. 8 d8 + 7 of slot t; logical offset of the unit
// ((p Hkv + h) 16 + t) D + 8 d8, tile offset ((p Hkv + h) D/8 + d8) 128 + 8 t.
template <typename T, bool TO_TILES>
__global__ __launch_bounds__(256) void k_pages_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                      long long units, int D) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= units) return;
  const int D8 = D / 8;
  const int t = (int)(i % PAGE);
  const long long r = i / PAGE;          // (p Hkv + h) D8 + d8
  const int d8 = (int)(r % D8);
  const long long ph = r / D8;           // p Hkv + h
  const size_t logical = ((size_t)ph * PAGE + t) * D + 8 * d8;
  const size_t tiled = ((size_t)ph * D8 + d8) * 128 + 8 * t;
  const size_t from = TO_TILES ? logical : tiled, to = TO_TILES ? tiled : logical;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[to + e] = src[from + e];
}

// V: unit (p, h, n, grp, d16) = slots 4 grp .. 4 grp + 3 of dim 16 n + d16; tile offset
// ((p Hkv + h) D/16 + n) 256 + grp 64 + d16 4 (4 consecutive), logical offset
// ((p Hkv + h) 16 + 4 grp + tt) D + 16 n + d16 for tt = 0..3.
template <typename T, bool TO_TILES>
__global__ __launch_bounds__(256) void v_pages_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                      long long units, int D) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= units) return;
  const int D16 = D / 16;
  const int d16 = (int)(i % 16);
  const int grp = (int)((i / 16) % 4);
  const long long r = i / 64;            // (p Hkv + h) D16 + n
  const int n = (int)(r % D16);
  const long long ph = r / D16;
  const size_t tiled = ((size_t)ph * D16 + n) * 256 + grp * 64 + d16 * 4;
  const size_t logical = ((size_t)ph * PAGE + 4 * grp) * D + 16 * n + d16;
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    if (TO_TILES) dst[tiled + tt] = src[logical + (size_t)tt * D];
    else dst[logical + (size_t)tt * D] = src[tiled + tt];
  }
}

template <typename T, bool TO_TILES>
hipError_t launch_typed(const void* ksrc, const void* vsrc, void* kdst, void* vdst, int num_pages, int Hkv, int D,
                        hipStream_t s) {
  const long long elems = (long long)num_pages * Hkv * PAGE * D;
  const long long ku = elems / 8, vu = elems / 4;
  k_pages_kernel<T, TO_TILES><<<(unsigned)((ku + 255) / 256), 256, 0, s>>>(
      static_cast<const T*>(ksrc), static_cast<T*>(kdst), ku, D);
  v_pages_kernel<T, TO_TILES><<<(unsigned)((vu + 255) / 256), 256, 0, s>>>(
      static_cast<const T*>(vsrc), static_cast<T*>(vdst), vu, D);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_pages(const KvPagesLaunch& c, hipStream_t s) {
  if (c.dtype == 1)
    return c.to_tiles ? launch_typed<uint16_t, true>(c.k_src, c.v_src, c.k_dst, c.v_dst, c.num_pages, c.Hkv, c.D, s)
                      : launch_typed<uint16_t, false>(c.k_src, c.v_src, c.k_dst, c.v_dst, c.num_pages, c.Hkv, c.D, s);
  return c.to_tiles ? launch_typed<float, true>(c.k_src, c.v_src, c.k_dst, c.v_dst, c.num_pages, c.Hkv, c.D, s)
                    : launch_typed<float, false>(c.k_src, c.v_src, c.k_dst, c.v_dst, c.num_pages, c.Hkv, c.D, s);
}

}  // namespace isd
