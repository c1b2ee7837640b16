// Workgroup -> output tile mapping shared by the projection kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace isd {

constexpr int XCDS = 8;  // workgroups are dispatched to the XCDs round-robin by id

// Linear workgroup id -> (m tile, n tile): XCD x (= id % 8) takes the column blocks
// x, x + 8, ... with all their row tiles, so the tiles that share a weight-column block
// run on one XCD and reuse it from that XCD's L2.  Returns false for padding ids.
__device__ __forceinline__ bool tile_of(int id, int mt, int nt, int& m, int& n) {
  const int x = id % XCDS, k = id / XCDS;
  n = x + XCDS * (k / mt);
  m = k % mt;
  return n < nt;
}

// Grid size for mt x nt tiles under tile_of.
inline int tile_grid(int mt, int nt) { return XCDS * ((nt + XCDS - 1) / XCDS) * mt; }

}  // namespace isd
