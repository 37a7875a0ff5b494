// Adaptive block mask (NABLA page, gist.science/es/paper/2507.13546,
// Metodologia item 2, bullets "Atencion Reducida" and "Umbralizacion CDF", and
// item 3, the union with a static sliding-tile window), emitted as CSR.
//
// Numerics: the cut must agree with a float64 evaluation except where the
// cumulative mass sits within 1e-4 of 1 - thr.  Block logits reach |z| ~ 10^3
// for strongly local heads, where float32 cannot even represent the 1e-4-level
// differences that decide the ordering, so logits, exponentials, the sort keys
// and the prefix sums are all float64.  MI355X issues float64 FMAs at the same
// rate as unpacked float32 FMAs, so this costs no throughput.
#include <float.h>

#include "kernels.h"

namespace bsa {

// ---------------------------------------------------------------------------
// Block logits: z[bh][i][j] = (qp_i . kp_j) / sqrt(D), float64 GEMM per head.
// 128 x 128 output tile per 256-thread workgroup, 8 x 8 per thread, k chunks
// of 16 staged in LDS k-major.  Each thread owns rows/cols 32c + 2t + {0,1}
// (c = 0..3), so its LDS operand reads are 16-byte loads at a 16-byte lane
// stride (no bank conflicts).
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) block_logits_kernel(const double* __restrict__ qp, const double* __restrict__ kp,
                                                           double* __restrict__ z, Geom g, double inv_sqrt_d) {
  constexpr int TM = 128, KC = 16;
  __shared__ __attribute__((aligned(16))) double As[KC][TM];
  __shared__ __attribute__((aligned(16))) double Bs[KC][TM];
  const int S = g.S;
  const int64_t bh = blockIdx.z;
  const int i0 = blockIdx.y * TM, j0 = blockIdx.x * TM;
  const double* qh = qp + (size_t)bh * S * D;
  const double* kh = kp + (size_t)bh * S * D;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
  // loader: row lr = tid >> 1, k half lk = (tid & 1) * 8
  const int lr = tid >> 1, lk = (tid & 1) * 8;
  for (int k0 = 0; k0 < D; k0 += KC) {
    {
      const int gi = i0 + lr, gj = j0 + lr;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        As[lk + e][lr] = gi < S ? qh[(size_t)gi * D + k0 + lk + e] : 0.0;
        Bs[lk + e][lr] = gj < S ? kh[(size_t)gj * D + k0 + lk + e] : 0.0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      double a[8], b[8];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double2 av = *(const double2*)&As[kk][32 * c + 2 * ty];
        const double2 bv = *(const double2*)&Bs[kk][32 * c + 2 * tx];
        a[2 * c] = av.x; a[2 * c + 1] = av.y;
        b[2 * c] = bv.x; b[2 * c + 1] = bv.y;
      }
#pragma unroll
      for (int x = 0; x < 8; ++x)
#pragma unroll
        for (int y = 0; y < 8; ++y) acc[x][y] = __fma_rn(a[x], b[y], acc[x][y]);
    }
    __syncthreads();
  }
  double* zh = z + (size_t)bh * S * S;
#pragma unroll
  for (int x = 0; x < 8; ++x) {
    const int gi = i0 + 32 * (x >> 1) + 2 * ty + (x & 1);
    if (gi >= S) continue;
#pragma unroll
    for (int y = 0; y < 8; ++y) {
      const int gj = j0 + 32 * (y >> 1) + 2 * tx + (y & 1);
      if (gj < S) zh[(size_t)gi * S + gj] = acc[x][y] * inv_sqrt_d;
    }
  }
}

hipError_t launch_block_logits(const Geom& g, const double* qp, const double* kp, double* z, hipStream_t s) {
  const int t = (g.S + 127) / 128;
  dim3 grid(t, t, (unsigned)(g.B * g.nh));
  const double inv = 1.0 / sqrt((double)g.D);
  if (g.D == 64)
    block_logits_kernel<64><<<grid, 256, 0, s>>>(qp, kp, z, g, inv);
  else
    block_logits_kernel<128><<<grid, 256, 0, s>>>(qp, kp, z, g, inv);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Workgroup reductions (256 threads, fixed tree order => deterministic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_reduce_max(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = fmax(red[tid], red[tid + s]);
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

__device__ __forceinline__ double block_reduce_sum(double v, double* red) {
  const int tid = threadIdx.x;
  red[tid] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) red[tid] = red[tid] + red[tid + s];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// exclusive scan of one value per thread (Hillis-Steele over 256 slots)
template <typename V>
__device__ __forceinline__ V block_exclusive_scan(V v, V* buf, V* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const V add = tid >= off ? buf[tid - off] : V(0);
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const V incl = buf[tid];
  *total = buf[255];
  __syncthreads();
  return incl - v;
}

// Row softmax of the block logits (inspection entry point only).
__global__ void __launch_bounds__(256) block_softmax_kernel(const double* __restrict__ z, double* __restrict__ p, Geom g) {
  __shared__ double red[256];
  const int64_t r = blockIdx.x;
  const double* zr = z + r * g.S;
  double* pr = p + r * g.S;
  double m = -DBL_MAX;
  for (int j = threadIdx.x; j < g.S; j += 256) m = fmax(m, zr[j]);
  m = block_reduce_max(m, red);
  double s = 0.0;
  for (int j = threadIdx.x; j < g.S; j += 256) s += exp(zr[j] - m);
  s = block_reduce_sum(s, red);
  for (int j = threadIdx.x; j < g.S; j += 256) pr[j] = exp(zr[j] - m) / s;
}

hipError_t launch_block_softmax(const Geom& g, const double* z, double* probs, hipStream_t s) {
  block_softmax_kernel<<<(unsigned)g.rows, 256, 0, s>>>(z, probs, g);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// CDF cut of one row per workgroup.
//   p_j = exp(z_j - max) / sum; order blocks by (p desc, j asc); c_k = exclusive
//   prefix of that order; keep position k iff k == 0 or c_k < 1 - thr; thr == 0
//   keeps all.  Only "candidates" with z_j >= max - lambda enter the sort: each
//   other block has p_j < exp(-lambda), and lambda (set by the host to
//   40 + ln S - ln thr) makes their total mass < 1e-17 * thr, so the cut can
//   never reach them and their omission cannot change the kept set.
// ---------------------------------------------------------------------------
constexpr int kMaxS = 4096;

__device__ __forceinline__ bool before(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__global__ void __launch_bounds__(256) select_kernel(const double* __restrict__ z, Geom g, double thr, double lambda,
                                                     int win_t, int win_h, int win_w, uint32_t* __restrict__ bitmap,
                                                     int32_t* __restrict__ counts, int words) {
  __shared__ double key[kMaxS];
  __shared__ int idx[kMaxS];
  __shared__ double red[256];
  __shared__ int ired[256];
  __shared__ uint32_t bm[kMaxS / 32];
  const int tid = threadIdx.x;
  const int S = g.S;
  const int64_t r = blockIdx.x;
  const int i = (int)(r % S);
  const double* zr = z + r * S;

  for (int w = tid; w < words; w += 256) bm[w] = 0u;

  if (thr == 0.0) {
    __syncthreads();
    for (int j = tid; j < S; j += 256) atomicOr(&bm[j >> 5], 1u << (j & 31));
  } else {
    double m = -DBL_MAX;
    for (int j = tid; j < S; j += 256) m = fmax(m, zr[j]);
    m = block_reduce_max(m, red);
    double s = 0.0;
    int nc = 0;
    for (int j = tid; j < S; j += 256) {
      const double zj = zr[j];
      s += exp(zj - m);
      nc += (zj - m >= -lambda);
    }
    const double sum = block_reduce_sum(s, red);
    int ntot;
    int off = block_exclusive_scan<int>(nc, ired, &ntot);
    for (int j = tid; j < S; j += 256) {
      const double zj = zr[j];
      if (zj - m >= -lambda) {
        key[off] = exp(zj - m);
        idx[off] = j;
        ++off;
      }
    }
    int n2 = 2;
    while (n2 < ntot) n2 <<= 1;
    for (int k = ntot + tid; k < n2; k += 256) {
      key[k] = -1.0;
      idx[k] = 0x7fffffff;
    }
    __syncthreads();
    // bitonic sort, final order: "before" first
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (n2 >> 1); t += 256) {
          const int lo = 2 * stride * (t / stride) + (t % stride);
          const int hi = lo + stride;
          const double klo = key[lo], khi = key[hi];
          const int ilo = idx[lo], ihi = idx[hi];
          const bool up = (lo & size) == 0;
          const bool sw = up ? before(khi, ihi, klo, ilo) : before(klo, ilo, khi, ihi);
          if (sw) {
            key[lo] = khi; key[hi] = klo;
            idx[lo] = ihi; idx[hi] = ilo;
          }
        }
        __syncthreads();
      }
    }
    // exclusive prefix of p = key / sum over the sorted candidates
    const int ept = (ntot + 255) / 256;           // contiguous elements per thread
    const int k0 = tid * ept;
    const int k1 = min(k0 + ept, ntot);
    double loc = 0.0;
    for (int k = k0; k < k1; ++k) loc += key[k] / sum;
    double tot;
    double c = block_exclusive_scan<double>(loc, red, &tot);
    const double target = 1.0 - thr;
    for (int k = k0; k < k1; ++k) {
      if (k == 0 || c < target) atomicOr(&bm[idx[k] >> 5], 1u << (idx[k] & 31));
      c += key[k] / sum;
    }
  }
  if (win_t >= 0) {
    const int HW = g.Hp * g.Wp;
    const int ti = i / HW, yi = (i / g.Wp) % g.Hp, xi = i % g.Wp;
    for (int j = tid; j < S; j += 256) {
      const int tj = j / HW, yj = (j / g.Wp) % g.Hp, xj = j % g.Wp;
      if (abs(ti - tj) <= win_t && abs(yi - yj) <= win_h && abs(xi - xj) <= win_w)
        atomicOr(&bm[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
  int pc = 0;
  for (int w = tid; w < words; w += 256) {
    const uint32_t v = bm[w];
    bitmap[r * words + w] = v;
    pc += __popc(v);
  }
  int total;
  block_exclusive_scan<int>(pc, ired, &total);
  if (tid == 0) counts[r] = total;
}

hipError_t launch_select(const Geom& g, const double* z, double thr, double lambda, int win_t, int win_h, int win_w,
                         uint32_t* bitmap, int32_t* counts, int words, hipStream_t s) {
  select_kernel<<<(unsigned)g.rows, 256, 0, s>>>(z, g, thr, lambda, win_t, win_h, win_w, bitmap, counts, words);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// row_ptr = exclusive scan of counts (one 1024-thread workgroup).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024) scan_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ row_ptr,
                                                    int32_t* __restrict__ nnz, int64_t rows) {
  __shared__ int32_t buf[1024];
  const int tid = threadIdx.x;
  const int64_t per = (rows + 1023) / 1024;
  const int64_t a = tid * per;
  const int64_t b = a + per < rows ? a + per : rows;
  int32_t loc = 0;
  for (int64_t k = a; k < b; ++k) loc += counts[k];
  buf[tid] = loc;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  int32_t run = buf[tid] - loc;
  for (int64_t k = a; k < b; ++k) {
    row_ptr[k] = run;
    run += counts[k];
  }
  if (tid == 1023) {
    row_ptr[rows] = buf[1023];
    if (nnz) *nnz = buf[1023];
  }
}

hipError_t launch_scan(const Geom& g, const int32_t* counts, int32_t* row_ptr, int32_t* nnz, hipStream_t s) {
  scan_kernel<<<1, 1024, 0, s>>>(counts, row_ptr, nnz, g.rows);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bitmap -> ascending column list; one wavefront per row.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) compact_kernel(const uint32_t* __restrict__ bitmap, int words,
                                                      const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                                      int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const uint32_t* bm = bitmap + r * words;
  int32_t base = row_ptr[r];
  for (int w0 = 0; w0 < words; w0 += 64) {
    const int w = w0 + lane;
    const uint32_t v = w < words ? bm[w] : 0u;
    const int pc = __popc(v);
    int incl = pc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int pos = base + incl - pc;
    uint32_t bits = v;
    while (bits) {
      const int b = __ffs(bits) - 1;
      col_idx[pos++] = w * 32 + b;
      bits &= bits - 1;
    }
    base += __shfl(incl, 63, 64);
  }
}

hipError_t launch_compact(const Geom& g, const uint32_t* bitmap, int words, const int32_t* row_ptr, int32_t* col_idx,
                          hipStream_t s) {
  compact_kernel<<<(unsigned)((g.rows + 3) / 4), 256, 0, s>>>(bitmap, words, row_ptr, col_idx, g.rows);
  return hipGetLastError();
}

}  // namespace bsa
