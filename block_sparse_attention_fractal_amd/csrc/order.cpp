// Token orders for the block partition, computed on the host (plain C++).
//
//   fractal    -- NABLA page (gist.science/es/paper/2507.13546), Metodologia
//                 item 1: frames outermost, P x P patches row-major, tokens
//                 row-major inside a patch;
//   tile-major -- TRA page ("Atencion de Radio de Tokens",
//                 gist.science/es/paper/2608.02504), "El Pipeline de
//                 TRA", item 3, bullet "Disposicion Tile-Major": tiles of
//                 tt x P x P tokens (tt = N / P^2 frames), tiles row-major in
//                 (t, y, x), tokens row-major inside a tile;
//   Hilbert    -- DFSAttn page (gist.science/es/paper/2605.23445), section 1:
//                 tokens in increasing index along the 3D Hilbert curve of the
//                 smallest 2^b cube that holds the grid, axes (t, y, x).
// The Hilbert index follows J. Skilling's transpose method ("Programming the
// Hilbert curve", AIP Conf. Proc. 707, 2004): per level from the top, the low
// bits are reflected or exchanged to undo the curve's orientation, the result is
// Gray-encoded, and the index is the bits of the three axes interleaved.
#include <algorithm>
#include <cstdint>
#include <string>
#include <utility>
#include <vector>

#include "order.h"

namespace bsa {

static uint64_t hilbert_index(uint32_t t, uint32_t y, uint32_t x, int bits) {
  uint32_t X[3] = {t, y, x};
  const uint32_t M = 1u << (bits - 1);
  for (uint32_t Q = M; Q > 1; Q >>= 1) {
    const uint32_t P = Q - 1;
    for (int i = 0; i < 3; ++i) {
      if (X[i] & Q) {
        X[0] ^= P;
      } else {
        const uint32_t s = (X[0] ^ X[i]) & P;
        X[0] ^= s;
        X[i] ^= s;
      }
    }
  }
  for (int i = 1; i < 3; ++i) X[i] ^= X[i - 1];
  uint32_t tg = 0;
  for (uint32_t Q = M; Q > 1; Q >>= 1)
    if (X[2] & Q) tg ^= Q - 1;
  for (int i = 0; i < 3; ++i) X[i] ^= tg;
  uint64_t h = 0;
  for (int b = bits - 1; b >= 0; --b)
    for (int i = 0; i < 3; ++i) h = (h << 1) | ((X[i] >> b) & 1u);
  return h;
}

int order_table(const Geom& g, int order, int32_t* table, std::string* msg) {
  const int T = g.T, H = g.H, W = g.W, P = g.P, N = g.N;
  const int64_t L = (int64_t)T * H * W;
  if (order == BSA_ORDER_FRACTAL || order == BSA_ORDER_TILE_MAJOR) {
    const int tt = order == BSA_ORDER_FRACTAL ? 1 : N / (P * P);
    if (order == BSA_ORDER_TILE_MAJOR && (N % (P * P) != 0 || T % tt != 0)) {
      *msg = "tile-major order needs N % (P*P) == 0 and T % (N/(P*P)) == 0";
      return BSA_ERR_SHAPE;
    }
    int64_t f = 0;
    for (int ct = 0; ct < T / tt; ++ct)
      for (int cy = 0; cy < H / P; ++cy)
        for (int cx = 0; cx < W / P; ++cx)
          for (int a = 0; a < tt; ++a)
            for (int y = 0; y < P; ++y)
              for (int x = 0; x < P; ++x)
                table[f++] = (int32_t)(((int64_t)(ct * tt + a) * H + cy * P + y) * W + cx * P + x);
    return f == L ? BSA_OK : BSA_ERR_SHAPE;
  }
  if (order == BSA_ORDER_HILBERT) {
    int bits = 1;
    while ((1 << bits) < std::max(T, std::max(H, W))) ++bits;
    std::vector<std::pair<uint64_t, int32_t>> key((size_t)L);
    int64_t n = 0;
    for (int t = 0; t < T; ++t)
      for (int y = 0; y < H; ++y)
        for (int x = 0; x < W; ++x, ++n) key[(size_t)n] = {hilbert_index(t, y, x, bits), (int32_t)n};
    std::sort(key.begin(), key.end());
    for (int64_t f = 0; f < L; ++f) table[f] = key[(size_t)f].second;
    return BSA_OK;
  }
  *msg = "order must be BSA_ORDER_FRACTAL, BSA_ORDER_TILE_MAJOR or BSA_ORDER_HILBERT";
  return BSA_ERR_INVALID_ARG;
}

}  // namespace bsa
