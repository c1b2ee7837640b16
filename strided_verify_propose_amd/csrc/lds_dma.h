// Global -> LDS loads for the large-tile MFMA kernels (LM head, split-K projection).
//
// Fragment: 16 rows x 32 bf16 of a K-contiguous operand (1 KB), loaded by one wave with
// global_load_lds_dwordx4: lane l's 16 bytes land at LDS slot l of the fragment.  For a
// row-major operand, four consecutive lanes read one row's 64 contiguous bytes: lane l takes
// row l / 4 and 16-byte chunk (l % 4) ^ (row / 4), so chunk c of row r sits at slot
// 4 r + (c ^ (r / 4)) -- where the MFMA lane holding (r, c) of v_mfma_f32_16x16x32_bf16 reads
// it, the xor keeping every 16-lane read on distinct banks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace isd {

// s_waitcnt with only the vector-memory count bounded (gfx9 encoding: vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void load_frag(const uint16_t* src, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// Row and 16-byte chunk that lane l loads of a row-major fragment.
__device__ __forceinline__ int frag_row(int lane) { return lane >> 2; }
__device__ __forceinline__ int frag_chunk(int lane) { return (lane & 3) ^ (lane >> 4); }

// LDS slot from which MFMA lane `lane` reads its operand of a row-major fragment.
__device__ __forceinline__ int frag_read_slot(int lane) {
  const int l16 = lane & 15;
  return 4 * l16 + ((lane >> 4) ^ (l16 >> 2));
}

// Barrier after this wave's loads of the next stage have landed (at most N of its vector
// loads still outstanding): the bare s_barrier does not wait for the younger loads still in
// flight, which a workgroup barrier would, and the fence orders the LDS reads after it.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  wait_vmcnt<N>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace isd
