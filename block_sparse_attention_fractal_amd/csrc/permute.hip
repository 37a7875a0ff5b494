// Fractal flattening (NABLA page, gist.science/es/paper/2507.13546,
// Metodologia item 1) as data movement, and the V layout used by the
// attention kernel.
//
// Both kernels are HBM-bound copies: every thread moves 16-byte chunks, and
// consecutive threads touch consecutive chunks of a row, so reads and writes
// are coalesced in runs of at least P rows on the original-order side.
#include "kernels.h"

namespace bsa {

// y[bh][f] = x[bh][orig(f)] (forward) or y[bh][orig(f)] = x[bh][f] (inverse).
__global__ void __launch_bounds__(256) permute_kernel(const uint4* __restrict__ x, uint4* __restrict__ y, Geom g,
                                                      int inverse, int cpr, int64_t total_chunks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total_chunks; c += stride) {
    const int64_t row = c / cpr;
    const int32_t part = (int32_t)(c - row * cpr);
    const int64_t bh = row / g.L;
    const int32_t f = (int32_t)(row - bh * g.L);
    const int64_t orow = bh * g.L + fractal_to_original(g, f);
    if (!inverse)
      y[row * cpr + part] = x[orow * cpr + part];
    else
      y[orow * cpr + part] = x[row * cpr + part];
  }
}

hipError_t launch_permute(const Geom& g, const void* x, void* y, int inverse, hipStream_t s) {
  const int elt = g.dtype == 1 ? 2 : 4;
  const int cpr = g.D * elt / 16;
  const int64_t total = (int64_t)g.B * g.nh * g.L * cpr;
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 65536 * 8 ? want : 65536 * 8);
  permute_kernel<<<grid, 256, 0, s>>>((const uint4*)x, (uint4*)y, g, inverse, cpr, total);
  return hipGetLastError();
}

// Any other token order, from a device table: y[bh, f] = x[bh, table[f]] (or the
// reverse scatter).  Entries are clamped into [0, L), so a malformed table
// copies wrong rows but never leaves the tensors.
__global__ void __launch_bounds__(256) permute_table_kernel(const uint4* __restrict__ x, uint4* __restrict__ y,
                                                            const int32_t* __restrict__ table, Geom g, int inverse,
                                                            int cpr, int64_t total_chunks) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total_chunks; c += stride) {
    const int64_t row = c / cpr;
    const int32_t part = (int32_t)(c - row * cpr);
    const int64_t bh = row / g.L;
    const int32_t f = (int32_t)(row - bh * g.L);
    const int64_t orow = bh * g.L + min(max(table[f], 0), g.L - 1);
    if (!inverse)
      y[row * cpr + part] = x[orow * cpr + part];
    else
      y[orow * cpr + part] = x[row * cpr + part];
  }
}

hipError_t launch_permute_table(const Geom& g, const int32_t* table, const void* x, void* y, int inverse,
                                hipStream_t s) {
  const int elt = g.dtype == 1 ? 2 : 4;
  const int cpr = g.D * elt / 16;
  const int64_t total = (int64_t)g.B * g.nh * g.L * cpr;
  const int64_t want = (total + 255) / 256;
  const int grid = (int)(want < 65536 * 8 ? want : 65536 * 8);
  permute_table_kernel<<<grid, 256, 0, s>>>((const uint4*)x, (uint4*)y, table, g, inverse, cpr, total);
  return hipGetLastError();
}

// Vt[bh][j][d][p] = V[bh][token(j, key(p))][d] with D = 128 or 64, 64 keys per block.
// Inside every group of 16 keys, stored position p holds key perm(p) with
// perm = 0,1,2,3, 8,9,10,11, 4,5,6,7, 12,13,14,15: the key order in which the
// softmax probabilities come out of the 32x32 MFMA accumulator, so the PV
// product can read its V operand as one 16-byte LDS load per lane.
__device__ __forceinline__ int vt_key_of_pos(int p) {
  const int w = p & 15;
  const int q = (w & 3) | ((w & 4) << 1) | ((w & 8) >> 1);
  return (p & ~15) | q;
}

template <int D>
__global__ void __launch_bounds__(256) prep_vt_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vt, Geom g) {
  constexpr int CH = D / 8;             // 16-byte chunks per token row
  __shared__ uint16_t tile[64][D + 8];  // +8 halves: rows 2D + 16 bytes apart, spreads banks on the column reads
  const int64_t blk = blockIdx.x;       // bh*S + j
  const int64_t bh = blk / g.S;
  const int32_t j = (int32_t)(blk - bh * g.S);
  const uint16_t* vb = v + (size_t)bh * g.L * D;
  const int tid = threadIdx.x;
  // 64 rows x CH chunks of 16 B; 256 threads -> D / 32 chunks each
#pragma unroll
  for (int it = 0; it < D / 32; ++it) {
    const int c = tid + it * 256;
    const int row = c / CH, part = c % CH;
    const uint4 val = *(const uint4*)(vb + (size_t)block_token_row(g, j, row) * D + part * 8);
    *(uint4*)(&tile[row][part * 8]) = val;
  }
  __syncthreads();
  // output: D d-rows x 64 keys = D rows x 8 chunks of 8 halves
  uint16_t* ob = vt + (size_t)blk * D * 64;
#pragma unroll
  for (int it = 0; it < D / 32; ++it) {
    const int c = tid + it * 256;
    const int d = c >> 3, part = c & 7;
    uint16_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = tile[vt_key_of_pos(part * 8 + e)][d];
    uint4 out;
    out.x = h[0] | ((uint32_t)h[1] << 16);
    out.y = h[2] | ((uint32_t)h[3] << 16);
    out.z = h[4] | ((uint32_t)h[5] << 16);
    out.w = h[6] | ((uint32_t)h[7] << 16);
    *(uint4*)(ob + (size_t)d * 64 + part * 8) = out;
  }
}

hipError_t launch_prep_vt(const Geom& g, const void* v, void* vt, hipStream_t s) {
  const int64_t blocks = (int64_t)g.B * g.nh * g.S;
  if (g.D == 64)
    prep_vt_kernel<64><<<(unsigned)blocks, 256, 0, s>>>((const uint16_t*)v, (uint16_t*)vt, g);
  else
    prep_vt_kernel<128><<<(unsigned)blocks, 256, 0, s>>>((const uint16_t*)v, (uint16_t*)vt, g);
  return hipGetLastError();
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s) {
  zero_i32_kernel<<<(n + 63) / 64, 64, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace bsa
