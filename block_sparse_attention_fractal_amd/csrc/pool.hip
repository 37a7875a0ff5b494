// Block average pooling of Q and K (NABLA page, gist.science/es/paper/2507.13546,
// Metodologia item 2, bullet "Submuestreo"): the mean of the N = 64 fractal-order
// tokens of every block.
//
// HBM-bound: each workgroup streams one 64-token block of Q or K exactly once
// (16-byte coalesced loads; in original order a block is 8 runs of 8 rows) and
// writes D float64 means.  Sums are accumulated in float64: for bf16 inputs
// every partial sum is exact, so the result does not depend on summation order.
#include "kernels.h"

namespace bsa {

template <typename T>
__device__ __forceinline__ void add_chunk(double* acc, const uint4& c);

template <>
__device__ __forceinline__ void add_chunk<uint16_t>(double* acc, const uint4& c) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += (double)__uint_as_float(w[e] << 16);
    acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void add_chunk<float>(double* acc, const uint4& c) {
  acc[0] += (double)__uint_as_float(c.x);
  acc[1] += (double)__uint_as_float(c.y);
  acc[2] += (double)__uint_as_float(c.z);
  acc[3] += (double)__uint_as_float(c.w);
}

// grid.x = rows (bh*S + i); one 256-thread workgroup pools block i of both Q
// and K, so every thread has 2*RPT independent 16-byte loads in flight.
template <typename T, int D>
__global__ void __launch_bounds__(256) pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   double* __restrict__ qp, double* __restrict__ kp, Geom g) {
  constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int CPR = D / EPC;             // chunks per row
  constexpr int RG = 256 / CPR;            // row groups
  constexpr int RPT = 64 / RG;             // rows per thread
  __shared__ double part[2][RG][D + 1];
  const int64_t r = blockIdx.x;
  const int64_t bh = r / g.S;
  const int32_t i = (int32_t)(r - bh * g.S);
  const int tid = threadIdx.x;
  const int c = tid % CPR, rg = tid / CPR;
  uint4 bq[RPT], bk[RPT];
#pragma unroll
  for (int it = 0; it < RPT; ++it) {
    const size_t off = ((size_t)bh * g.L + block_token_row(g, i, rg + it * RG)) * D + c * EPC;
    bq[it] = *(const uint4*)(q + off);
    bk[it] = *(const uint4*)(k + off);
  }
  double aq[EPC], ak[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) aq[e] = ak[e] = 0.0;
#pragma unroll
  for (int it = 0; it < RPT; ++it) {
    add_chunk<T>(aq, bq[it]);
    add_chunk<T>(ak, bk[it]);
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    part[0][rg][c * EPC + e] = aq[e];
    part[1][rg][c * EPC + e] = ak[e];
  }
  __syncthreads();
  for (int x = tid; x < 2 * D; x += 256) {
    const int t = x / D, d = x - t * D;
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < RG; ++j) s += part[t][j][d];
    (t == 0 ? qp : kp)[(size_t)r * D + d] = s * (1.0 / 64.0);
  }
}

hipError_t launch_pool(const Geom& g, const void* q, const void* k, double* qp, double* kp, hipStream_t s) {
  dim3 grid((unsigned)g.rows);
  if (g.dtype == 1 && g.D == 64)
    pool_kernel<uint16_t, 64><<<grid, 256, 0, s>>>((const uint16_t*)q, (const uint16_t*)k, qp, kp, g);
  else if (g.dtype == 1)
    pool_kernel<uint16_t, 128><<<grid, 256, 0, s>>>((const uint16_t*)q, (const uint16_t*)k, qp, kp, g);
  else if (g.D == 64)
    pool_kernel<float, 64><<<grid, 256, 0, s>>>((const float*)q, (const float*)k, qp, kp, g);
  else
    pool_kernel<float, 128><<<grid, 256, 0, s>>>((const float*)q, (const float*)k, qp, kp, g);
  return hipGetLastError();
}

}  // namespace bsa
