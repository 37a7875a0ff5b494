// Device helpers shared by the block-mask and group-mask kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geom.h"

namespace bsa {

// order-preserving map of a double to uint64 (larger value -> larger key);
// -0.0 and +0.0 are equal values and must share one key
__device__ __forceinline__ uint64_t order_key(double z) {
  const uint64_t b = z == 0.0 ? 0ull : (uint64_t)__double_as_longlong(z);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Sliding-tile window (NABLA page, Metodologia item 3): block ids are tiles
// (t, y, x) of Hp x Wp patches per frame; ids i and j are within the window when
// every coordinate differs by at most the given extent.
__device__ __forceinline__ bool in_window(const Geom& g, int i, int j, int win_t, int win_h, int win_w) {
  const int HW = g.Hp * g.Wp;
  const int ti = i / HW, yi = (i / g.Wp) % g.Hp, xi = i % g.Wp;
  const int tj = j / HW, yj = (j / g.Wp) % g.Hp, xj = j % g.Wp;
  return abs(ti - tj) <= win_t && abs(yi - yj) <= win_h && abs(xi - xj) <= win_w;
}

}  // namespace bsa
