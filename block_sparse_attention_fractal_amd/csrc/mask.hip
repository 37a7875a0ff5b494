// Adaptive block mask (NABLA page, gist.science/es/paper/2507.13546,
// Metodologia item 2, bullets "Atencion Reducida" and "Umbralizacion CDF", and
// item 3, the union with a static sliding-tile window), emitted as CSR.
//
// Numerics: the cut must agree with a float64 evaluation except where the
// cumulative mass sits within 1e-4 of 1 - thr.  Block logits reach |z| ~ 10^3
// for strongly local heads, where float32 cannot even represent the 1e-4-level
// differences that decide the ORDER of the blocks, so pooled means, logits and
// the selection keys are float64 (MI355X issues float64 FMAs at the same rate
// as unpacked float32 FMAs).  The masses compared with 1 - thr only need an
// absolute accuracy well below the band, so they come from float32
// exponentials summed exactly in fixed point.
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
// CDF cut of one row per workgroup, by radix selection instead of a sort.
//
//   p_j = exp(z_j - max) / sum; order blocks by (p desc, j asc); c_k = exclusive
//   prefix mass of that order; keep position k iff k == 0 or c_k < 1 - thr;
//   thr == 0 keeps all.
//
// The order is decided on the float64 logits (p is monotone in z), so it is as
// exact as the logits.  Only the MASSES enter the comparison with 1 - thr, and
// for those float32 exponentials (relative error ~1e-6) are far inside the 1e-4
// band; they are accumulated as exact unsigned fixed-point integers (2^-50
// units), so every partial sum is independent of summation order and the cut is
// bitwise deterministic.
//
// Selection: the kept set is {key > K*} plus the block(s) with key K*, where K*
// is the key of the block at which the cumulative mass first reaches 1 - thr.
// K* is found MSB-first, 8 key bits per pass: a 256-bin histogram of (count,
// mass) of the blocks still sharing the decided prefix, a suffix scan over the
// bins, and the bin where the mass crosses the target.  Passes stop when that
// bin holds a single block; equal keys (exact ties) are resolved by index.
// Blocks with z < max - lambda are never candidates: lambda (set by the host to
// 40 + ln S - ln thr) bounds their total mass below 1e-17 * thr, so the cut can
// never reach them.
// ---------------------------------------------------------------------------
constexpr int kMaxS = 4096;
constexpr int kPerThread = kMaxS / 256;

// order-preserving map of a double to uint64 (larger value -> larger key);
// -0.0 and +0.0 are equal values and must share one key
__device__ __forceinline__ uint64_t order_key(double z) {
  const uint64_t b = z == 0.0 ? 0ull : (uint64_t)__double_as_longlong(z);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_down_u64(uint64_t v, int d) {
  const uint32_t lo = __shfl_down((uint32_t)v, d, 64), hi = __shfl_down((uint32_t)(v >> 32), d, 64);
  return ((uint64_t)hi << 32) | lo;
}

// 256-thread reductions: butterfly inside each wave, then the four wave results
// in a fixed order (deterministic, one barrier).
template <typename V, typename Op>
__device__ __forceinline__ V wg_reduce(V v, V* slot4, Op op) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    if constexpr (sizeof(V) == 8) {
      uint64_t u;
      __builtin_memcpy(&u, &v, 8);
      u = shfl_xor_u64(u, m);
      V o;
      __builtin_memcpy(&o, &u, 8);
      v = op(v, o);
    } else {
      v = op(v, __shfl_xor(v, m, 64));
    }
  }
  __syncthreads();
  if ((threadIdx.x & 63) == 0) slot4[threadIdx.x >> 6] = v;
  __syncthreads();
  return op(op(slot4[0], slot4[1]), op(slot4[2], slot4[3]));
}

__global__ void __launch_bounds__(256) select_kernel(const double* __restrict__ z, Geom g, double thr, double lambda,
                                                     int win_t, int win_h, int win_w, uint32_t* __restrict__ bitmap,
                                                     int32_t* __restrict__ counts, int words) {
  __shared__ uint64_t umass[256];
  __shared__ uint32_t ucount[256];
  __shared__ uint32_t bm[kMaxS / 32];
  __shared__ uint32_t tie[kMaxS / 32];
  __shared__ double dslot[4];
  __shared__ uint64_t uslot[4];
  __shared__ uint64_t s_prefix, s_above;
  __shared__ uint32_t s_cnt;
  const int tid = threadIdx.x, lane = tid & 63;
  const int S = g.S;
  const int64_t r = blockIdx.x;
  const int i = (int)(r % S);
  const double* zr = z + r * S;

  for (int w = tid; w < kMaxS / 32; w += 256) bm[w] = 0u;

  if (thr == 0.0) {
    __syncthreads();
    for (int j = tid; j < S; j += 256) atomicOr(&bm[j >> 5], 1u << (j & 31));
  } else {
    double zv[kPerThread];
    double m = -DBL_MAX;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int j = tid + 256 * k;
      zv[k] = j < S ? zr[j] : -DBL_MAX;
      m = fmax(m, zv[k]);
    }
    m = wg_reduce(m, dslot, [](double a, double b) { return fmax(a, b); });
    // candidates: fixed-point masses (2^-50 units, S * 2^50 < 2^63) and order keys
    uint64_t key[kPerThread], w[kPerThread];
    uint64_t wsum = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const double d = zv[k] - m;
      const bool cand = (tid + 256 * k < S) && d >= -lambda;
      const float e = cand ? __builtin_amdgcn_exp2f((float)d * 1.44269504088896341f) : 0.f;
      w[k] = cand ? (uint64_t)((double)e * 1125899906842624.0) : 0ull;
      key[k] = cand ? order_key(zv[k]) : 0ull;
      wsum += w[k];
    }
    const uint64_t total = wg_reduce(wsum, uslot, [](uint64_t a, uint64_t b) { return a + b; });
    const double target = (1.0 - thr) * (double)total;        // keep while exclusive prefix < target
    // Pass 0: 256 uniform buckets of d = z - max over [dmin, 0].  The bucket index
    // is a monotone function of z, so it refines the order without breaking it,
    // and it spreads even near-uniform rows thinly over the bins (few LDS atomic
    // collisions).  Later passes use the exact key, inside the crossing bucket only.
    double dmin = 0.0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
      if (w[k] != 0ull) dmin = fmin(dmin, zv[k] - m);
    dmin = wg_reduce(dmin, dslot, [](double a, double b) { return fmin(a, b); });
    const double bscale = dmin < 0.0 ? 255.999 / (-dmin) : 0.0;
    int bucket[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) bucket[k] = (int)((zv[k] - m - dmin) * bscale);
    ucount[tid] = 0u;
    umass[tid] = 0ull;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
      if (w[k] != 0ull) {
        atomicAdd(&ucount[bucket[k]], 1u);
        atomicAdd((unsigned long long*)&umass[bucket[k]], (unsigned long long)w[k]);
      }
    __syncthreads();
    auto crossing_bin = [&](uint64_t above_in, uint64_t prefix_in, int shift_in) {
      // lane l owns bins 4l..4l+3; suffix sums over bins (bin 255 = largest keys)
      uint64_t mb[4];
      uint32_t cb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) { mb[x] = umass[4 * lane + x]; cb[x] = ucount[4 * lane + x]; }
      const uint64_t lane_tot = mb[0] + mb[1] + mb[2] + mb[3];
      uint64_t suf = lane_tot;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint64_t o = shfl_down_u64(suf, d);
        if (lane + d < 64) suf += o;
      }
      uint64_t run = suf - lane_tot;
#pragma unroll
      for (int x = 3; x >= 0; --x) {
        const uint64_t excl = run;
        run += mb[x];
        if (cb[x] != 0u && (double)(above_in + excl) < target && target <= (double)(above_in + run)) {
          s_prefix = prefix_in | ((uint64_t)(4 * lane + x) << shift_in);
          s_above = above_in + excl;
          s_cnt = cb[x];
        }
      }
    };
    if (tid == 0) { s_prefix = 0; s_above = 0; s_cnt = 0; }   // unreachable target: keep every candidate
    __syncthreads();
    if (tid < 64) crossing_bin(0, 0, 0);
    __syncthreads();
    const int b0 = (int)s_prefix;
    uint64_t above = s_above;
    uint32_t cnt_bin = s_cnt;
    // exact passes over the keys of the crossing bucket
    uint64_t kmax = 0, kmin = ~0ull;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const bool in = w[k] != 0ull && bucket[k] == b0;
      if (!in) w[k] = w[k] != 0ull && bucket[k] > b0 ? w[k] : 0ull;  // keep "above" blocks, drop the rest
      if (in) {
        kmax = key[k] > kmax ? key[k] : kmax;
        kmin = key[k] < kmin ? key[k] : kmin;
      }
    }
    kmax = wg_reduce(kmax, uslot, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
    kmin = wg_reduce(kmin, uslot, [](uint64_t a, uint64_t b) { return a < b ? a : b; });
    const uint64_t diff = kmax ^ kmin;
    int shift = diff == 0 ? 0 : ((63 - __clzll(diff)) & ~7);
    uint64_t prefix = shift >= 56 ? 0ull : (kmax & (~0ull << (shift + 8)));
    if (cnt_bin > 1u) {
      if (tid == 0) { s_prefix = prefix; s_cnt = 0; }
      for (;;) {
        ucount[tid] = 0u;
        umass[tid] = 0ull;
        __syncthreads();
        const uint64_t hi_mask = shift >= 56 ? 0ull : (~0ull << (shift + 8));
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
          if (w[k] != 0ull && bucket[k] == b0 && (key[k] & hi_mask) == prefix) {
            const int d = (int)((key[k] >> shift) & 255);
            atomicAdd(&ucount[d], 1u);
            atomicAdd((unsigned long long*)&umass[d], (unsigned long long)w[k]);
          }
        }
        __syncthreads();
        if (tid < 64) crossing_bin(above, prefix, shift);
        __syncthreads();
        prefix = s_prefix;
        above = s_above;
        cnt_bin = s_cnt;
        if (cnt_bin <= 1u || shift == 0) break;
        shift -= 8;
      }
    } else {
      prefix = cnt_bin == 0u ? 0ull : kmax;   // one block in the crossing bucket: its key; none: keep all
      shift = 0;
    }
    // keep: keys above the final bin, and the final bin itself when it holds one block
    const uint64_t lo_key = prefix;
    const uint64_t hi_key = shift == 0 ? prefix : (prefix | ((1ull << shift) - 1));
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      if (w[k] == 0ull) continue;
      const int j = tid + 256 * k;
      if (bucket[k] > b0 || key[k] > hi_key || (cnt_bin <= 1u && key[k] >= lo_key))
        atomicOr(&bm[j >> 5], 1u << (j & 31));
    }
    if (cnt_bin > 1u) {
      // exact ties at K* = prefix: keep the lowest-index ones until the mass reaches the target
      for (int x = tid; x < kMaxS / 32; x += 256) tie[x] = 0u;
      __syncthreads();
      uint64_t wt = 0;
#pragma unroll
      for (int k = 0; k < kPerThread; ++k)
        if (w[k] != 0ull && bucket[k] == b0 && key[k] == prefix) {
          atomicOr(&tie[(tid + 256 * k) >> 5], 1u << ((tid + 256 * k) & 31));
          wt = w[k];
        }
      if (wt != 0ull) umass[0] = wt;            // all ties share one mass
      __syncthreads();
      if (tid == 0) {
        const uint64_t wtie = umass[0];
        uint64_t acc = above;
        for (int x = 0; x < (S + 31) / 32; ++x) {
          uint32_t bits = tie[x];
          while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1;
            if ((double)acc < target) {
              bm[x] |= 1u << b;
              acc += wtie;
            }
          }
        }
      }
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
  uint32_t pc = 0;
  for (int w2 = tid; w2 < words; w2 += 256) {
    const uint32_t v = bm[w2];
    bitmap[r * words + w2] = v;
    pc += __popc(v);
  }
  pc = wg_reduce(pc, ucount, [](uint32_t a, uint32_t b) { return a + b; });
  if (tid == 0) counts[r] = (int32_t)pc;
}

hipError_t launch_select(const Geom& g, const double* z, double thr, double lambda, int win_t, int win_h, int win_w,
                         uint32_t* bitmap, int32_t* counts, int words, hipStream_t s) {
  select_kernel<<<(unsigned)g.rows, 256, 0, s>>>(z, g, thr, lambda, win_t, win_h, win_w, bitmap, counts, words);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// row_ptr = exclusive scan of counts, in two launches: per-chunk totals, then
// every chunk scans its own counts after summing the totals of the chunks
// before it (at most rows/1024 of them).
// ---------------------------------------------------------------------------
constexpr int kScanChunk = 1024;

__device__ __forceinline__ int32_t wave_incl_scan(int32_t v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// 1024-thread exclusive scan of one value per thread; returns (exclusive, total)
__device__ __forceinline__ int32_t wg1024_excl_scan(int32_t v, int32_t* wsum, int32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int32_t incl = wave_incl_scan(v, lane);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int32_t x = lane < 16 ? wsum[lane] : 0;
    const int32_t xi = wave_incl_scan(x, lane);
    if (lane < 16) wsum[lane] = xi - x;
    if (lane == 15) wsum[16] = xi;
  }
  __syncthreads();
  *total = wsum[16];
  return wsum[w] + incl - v;
}

__global__ void __launch_bounds__(1024) chunk_sum_kernel(const int32_t* __restrict__ counts, int32_t* __restrict__ sums,
                                                         int64_t rows) {
  __shared__ int32_t wsum[17];
  const int64_t r = (int64_t)blockIdx.x * kScanChunk + threadIdx.x;
  int32_t tot;
  wg1024_excl_scan(r < rows ? counts[r] : 0, wsum, &tot);
  if (threadIdx.x == 0) sums[blockIdx.x] = tot;
}

__global__ void __launch_bounds__(1024) chunk_scan_kernel(const int32_t* __restrict__ counts,
                                                          const int32_t* __restrict__ sums, int32_t* __restrict__ row_ptr,
                                                          int32_t* __restrict__ nnz, int64_t rows, int nchunks) {
  __shared__ int32_t wsum[17];
  __shared__ int32_t s_base;
  const int tid = threadIdx.x;
  // offset of this chunk: sum of the chunk totals before it (fixed order)
  if (tid < 64) {
    int32_t acc = 0;
    for (int c = tid; c < (int)blockIdx.x; c += 64) acc += sums[c];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (tid == 0) s_base = acc;
  }
  __syncthreads();
  const int64_t r = (int64_t)blockIdx.x * kScanChunk + tid;
  const int32_t v = r < rows ? counts[r] : 0;
  int32_t tot;
  const int32_t ex = wg1024_excl_scan(v, wsum, &tot) + s_base;
  if (r < rows) row_ptr[r] = ex;
  if (blockIdx.x == (unsigned)(nchunks - 1) && tid == 0) {
    row_ptr[rows] = s_base + tot;
    if (nnz) *nnz = s_base + tot;
  }
}

hipError_t launch_scan(const Geom& g, const int32_t* counts, int32_t* row_ptr, int32_t* chunk_sums, int32_t* nnz,
                       hipStream_t s) {
  const int nchunks = (int)((g.rows + kScanChunk - 1) / kScanChunk);
  chunk_sum_kernel<<<nchunks, kScanChunk, 0, s>>>(counts, chunk_sums, g.rows);
  chunk_scan_kernel<<<nchunks, kScanChunk, 0, s>>>(counts, chunk_sums, row_ptr, nnz, g.rows, nchunks);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bitmap -> ascending column list; one wavefront per row.  Each lane tests one
// block id per step and a ballot turns the bits into coalesced output slots.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) compact_kernel(const uint32_t* __restrict__ bitmap, int words,
                                                      const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                                      int64_t rows, int S) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const uint32_t* bm = bitmap + r * words;
  int32_t base = row_ptr[r];
  for (int j0 = 0; j0 < S; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t wv = bm[min(j >> 5, words - 1)];
    const bool on = j < S && ((wv >> (j & 31)) & 1u);
    const uint64_t mask = __ballot(on);
    if (on) col_idx[base + __popcll(mask & ((1ull << lane) - 1))] = j;
    base += __popcll(mask);
  }
}

hipError_t launch_compact(const Geom& g, const uint32_t* bitmap, int words, const int32_t* row_ptr, int32_t* col_idx,
                          hipStream_t s) {
  compact_kernel<<<(unsigned)((g.rows + 3) / 4), 256, 0, s>>>(bitmap, words, row_ptr, col_idx, g.rows, g.S);
  return hipGetLastError();
}

}  // namespace bsa
