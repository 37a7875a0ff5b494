// Problem geometry shared by the host library and the kernels.
//
// Token layout follows the fractal flattening of the NABLA page
// (gist.science/es/paper/2507.13546, Metodologia item 1): frames outermost,
// P x P patches row-major inside a frame, tokens row-major inside a patch.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define BSA_HD __host__ __device__ __forceinline__
#else
#define BSA_HD inline
#endif

namespace bsa {

struct Geom {
  int32_t B, nh, T, H, W, D, P, N;
  int32_t L;        // T*H*W tokens per head
  int32_t S;        // L / N blocks per head
  int32_t Hp, Wp;   // patches per frame along h and w
  int32_t layout;   // 0 = original (t,h,w) order, 1 = fractal order
  int32_t dtype;    // 0 = f32, 1 = bf16
  int64_t rows;     // B*nh*S CSR rows
};

// Original row-major index of the token at fractal position f (any P).
BSA_HD int32_t fractal_to_original(const Geom& g, int32_t f) {
  const int32_t pp = g.P * g.P;
  const int32_t blk = f / pp, m = f - blk * pp;
  const int32_t px = blk % g.Wp;
  const int32_t rest = blk / g.Wp;
  const int32_t py = rest % g.Hp;
  const int32_t t = rest / g.Hp;
  const int32_t y = m / g.P, x = m - y * g.P;
  return (t * g.H + py * g.P + y) * g.W + px * g.P + x;
}

// Row (token index inside a head's [L, D] slab, in the tensor's own layout) of
// token m of block i.  With layout 0 a block is one P x P patch (N == P*P).
BSA_HD int32_t block_token_row(const Geom& g, int32_t i, int32_t m) {
  return g.layout == 1 ? i * g.N + m : fractal_to_original(g, i * g.N + m);
}

}  // namespace bsa
