// Host-side 3D Hilbert token order ([chapterpal] method paragraph and
// recommendations: space-filling Hilbert-curve reordering of visual tokens).
//
// Curve: J. Skilling, "Programming the Hilbert curve", AIP Conf. Proc. 707 (2004),
// FORWARD direction (cell -> index) in "transpose" form: per level, from the
// coarsest, the low bits of the first coordinate are reflected or exchanged with
// another coordinate's, then the coordinates are Gray-encoded; the index is the
// coordinates' bits interleaved from the most significant level down, first
// coordinate first.  Cells of a T x Hg x W grid are placed at the origin of the
// smallest 2^m cube holding it and sorted by index.
#include <stdint.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "sparge_internal.hpp"

namespace sparge {
namespace {

uint64_t hilbert_index3(uint32_t c0, uint32_t c1, uint32_t c2, int m) {
  uint32_t X[3] = {c0, c1, c2};
  if (m > 0) {
    const uint32_t top = 1u << (m - 1);
    for (uint32_t q = top; q > 1; q >>= 1) {
      const uint32_t low = q - 1;
      for (int d = 0; d < 3; ++d) {
        if (X[d] & q) {
          X[0] ^= low;                      // reflect
        } else {
          const uint32_t diff = (X[0] ^ X[d]) & low;
          X[0] ^= diff;                     // exchange low bits of axes 0 and d
          X[d] ^= diff;
        }
      }
    }
    X[1] ^= X[0];
    X[2] ^= X[1];
    uint32_t flip = 0;
    for (uint32_t q = top; q > 1; q >>= 1)
      if (X[2] & q) flip ^= q - 1;
    for (int d = 0; d < 3; ++d) X[d] ^= flip;
  }
  uint64_t key = 0;
  for (int b = m - 1; b >= 0; --b)
    for (int d = 0; d < 3; ++d) key = (key << 1) | ((X[d] >> b) & 1u);
  return key;
}

}  // namespace

void hilbert_perm3d_host(int T, int Hg, int W, int32_t* perm) {
  int m = 0;
  const int side = std::max(T, std::max(Hg, W));
  while ((1 << m) < side) ++m;
  std::vector<std::pair<uint64_t, int32_t>> cells;
  cells.reserve((size_t)T * Hg * W);
  for (int t = 0; t < T; ++t)
    for (int y = 0; y < Hg; ++y)
      for (int x = 0; x < W; ++x)
        cells.emplace_back(hilbert_index3((uint32_t)t, (uint32_t)y, (uint32_t)x, m),
                           (int32_t)(((int64_t)t * Hg + y) * W + x));
  std::sort(cells.begin(), cells.end());
  for (size_t p = 0; p < cells.size(); ++p) perm[p] = cells[p].second;
}

}  // namespace sparge
