// Workgroup -> output tile mapping shared by the projection kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace isd {

constexpr int XCDS = 8;  // workgroups are dispatched to the XCDs round-robin by id

// Linear workgroup id -> (m tile, n tile).  The mt x nt tiles are numbered column block by
// column block (t = n mt + m) and XCD x (= id % 8) takes the contiguous run
// [x per, (x+1) per), per = ceil(mt nt / 8): no XCD holds more than per tiles, so none
// runs a second round while others idle, and the row tiles of a weight-column block run
// on one XCD, or two, and reuse it from that XCD's L2.  Returns false for padding ids.
__device__ __forceinline__ bool tile_of(int id, int mt, int nt, int& m, int& n) {
  const int T = mt * nt, per = (T + XCDS - 1) / XCDS;
  const int x = id % XCDS, k = id / XCDS;
  const int t = x * per + k;
  if (k >= per || t >= T) return false;
  n = t / mt;
  m = t - n * mt;
  return true;
}

// Grid size for mt x nt tiles under tile_of.
inline int tile_grid(int mt, int nt) { return XCDS * ((mt * nt + XCDS - 1) / XCDS); }

}  // namespace isd
