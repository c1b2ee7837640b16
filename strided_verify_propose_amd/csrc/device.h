// Device helpers for the gfx950 kernels: vector types, bf16 conversion, wave64
// reductions and scans, MFMA wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace isd {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t b = __float_as_uint(f);
  return (b + 0x7fffu + ((b >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 2^x on the hardware transcendental unit (v_exp_f32).  -inf -> 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats -> packed bf16 pair (low, high), round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// max / sum over lanes l, l^16, l^32, l^48 (the four 16-lane rows) with the gfx950 row swaps.
__device__ __forceinline__ float row4_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------- wave64 reductions
// Butterfly over the 64 lanes without LDS: DPP quad permutes (lane ^ 1, lane ^ 2), row half
// mirror and row mirror (eight and sixteen lanes), then the gfx950 row swaps across
// 16-lane rows and 32-lane halves.  Every step combines a lane with a partner holding the
// complementary lanes, and partners compute op(a, b) and op(b, a), so with a commutative op
// every lane ends with the same value.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2, 3, 0, 1]
constexpr int DPP_HALF_MIRROR = 0x141;
constexpr int DPP_MIRROR = 0x140;

template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_mov<DPP_QUAD_XOR1>(v));
  v = op(v, dpp_mov<DPP_QUAD_XOR2>(v));
  v = op(v, dpp_mov<DPP_HALF_MIRROR>(v));
  v = op(v, dpp_mov<DPP_MIRROR>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(b[0], b[1]);
}
template <int CTRL>
__device__ __forceinline__ double dpp_mov_d(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = dpp_mov<CTRL>((uint32_t)u), hi = dpp_mov<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_mov_d<DPP_QUAD_XOR1>(v);
  v += dpp_mov_d<DPP_QUAD_XOR2>(v);
  v += dpp_mov_d<DPP_HALF_MIRROR>(v);
  v += dpp_mov_d<DPP_MIRROR>(v);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const uint64_t u = __double_as_longlong(v);
    const auto lo = half ? __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false)
                         : __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    const auto hi = half ? __builtin_amdgcn_permlane32_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false)
                         : __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
    v = __longlong_as_double((long long)(((uint64_t)hi[0] << 32) | lo[0])) +
        __longlong_as_double((long long)(((uint64_t)hi[1] << 32) | lo[1]));
  }
  return v;
}
// Sum over each 16-lane row (every lane of the row gets it).
__device__ __forceinline__ float row16_sum(float v) {
  v += __uint_as_float(dpp_mov<DPP_QUAD_XOR1>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<DPP_QUAD_XOR2>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<DPP_HALF_MIRROR>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<DPP_MIRROR>(__float_as_uint(v)));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ int wave_min_i(int v) {
  return (int)wave_reduce_u32((uint32_t)v, [](uint32_t a, uint32_t b) { return (uint32_t)min((int)a, (int)b); });
}
// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each 16-lane row with DPP
// row shifts (lanes shifted in from before the row read 0), then each row adds the totals
// of the rows before it, read from lanes 15, 31 and 47.
__device__ __forceinline__ double wave_incl_scan_d(double v, int lane) {
  v += dpp_mov_d<0x111>(v);  // row_shr:1
  v += dpp_mov_d<0x112>(v);  // row_shr:2
  v += dpp_mov_d<0x114>(v);  // row_shr:4
  v += dpp_mov_d<0x118>(v);  // row_shr:8
  const uint64_t u = __double_as_longlong(v);
  double tot[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)u, 16 * r + 15);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 16 * r + 15);
    tot[r] = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  }
  const int row = lane >> 4;
  double before = 0.0;  // sum of the earlier rows' totals, in row order
  if (row >= 1) before = tot[0];
  if (row >= 2) before += tot[1];
  if (row >= 3) before += tot[2];
  return v + before;
}

// ---------------------------------------------------------------- MFMA (CDNA4)
// D(16x16) += A(16x32) * B(32x16); lane l holds A[l%16][8*(l/16)+0..7],
// B[8*(l/16)+0..7][l%16]; D[4*(l/16)+i][l%16] in element i.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// D(16x16) += A(16x16) * B(16x16); lane l holds A[l%16][4*(l/16)+0..3],
// B[4*(l/16)+0..3][l%16]; D[4*(l/16)+i][l%16] in element i.
__device__ __forceinline__ f32x4 mfma16x16x16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ T ldg(const T* p) { return *p; }

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for every
// outstanding global load and store of the waves, which drains any load pipeline that
// runs across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace isd
