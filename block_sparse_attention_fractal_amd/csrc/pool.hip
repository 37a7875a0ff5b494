// Block average pooling of Q and K (NABLA page, gist.science/es/paper/2507.13546,
// Metodologia item 2, bullet "Submuestreo"): the mean of the N = 64 fractal-order
// tokens of every block.
//
// HBM-bound: a wavefront streams 64-token blocks of Q or K exactly once with
// 16-byte loads (LPR lanes cover a token row, so one load instruction covers
// RPI = 64 / LPR rows; in original order a block is 8 runs of 8 rows) and sums
// in float64 straight from the loaded registers, the next block's loads in
// flight meanwhile.  For bf16 inputs every partial
// sum is exact, so neither the order of the per-lane sums nor that of the
// cross-lane combine changes the result.
//
// With kScreen the same pass also writes the screen operands of the CDF cut
// (see mask_screen.hip): the channel mean mu, the centred vector c = x - mu
// scaled by 2^ex into [2^13, 2^14) and split into fp16 hi + lo, and (query
// blocks) an upper bound of |c|; key blocks also fold their mean and |c| into
// per-head maxima / minima.
#include "kernels.h"
#include "mask_util.h"

namespace bsa {

constexpr int kPoolBlocks = 2;          // consecutive blocks per wavefront (150 VGPRs, three waves per SIMD)

// grid = (ceil(S / (4 kPoolBlocks)), B * heads, 2 or 1): z = 0 pools Q, z = 1 pools K;
// wave w of workgroup x takes blocks (4x + w) kPoolBlocks + b of head y, with the
// loads of block b + 1 in flight while block b is summed and written.
template <typename T, int D, bool kScreen>
__global__ void __launch_bounds__(256) pool_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                   double* __restrict__ qp, double* __restrict__ kp, ScreenOps ops,
                                                   Geom g) {
  constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
  constexpr int LPR = D / EPC;             // lanes per token row
  constexpr int RPI = 64 / LPR;            // rows per load instruction
  constexpr int NL = 64 / RPI;             // loads per lane
  constexpr int EPR = EPC / RPI;           // means each lane writes
  static_assert(EPR >= 1 && RPI >= 2, "tile shape");
  __shared__ uint64_t red[3][4];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // scalar: block coordinates on the SALU
  const int64_t bh = blockIdx.y;
  const bool keys = blockIdx.z == 1;
  const int i0 = (blockIdx.x * 4 + wave) * kPoolBlocks;
  const int c = lane % LPR, rg = lane / LPR;
  const T* base = (keys ? k : q) + (size_t)bh * g.L * D + c * EPC;
  // row offset of token m inside a block (m = rg + u * RPI); the original layout
  // has P = 8 (P * P = N = 64), a block being 8 runs of 8 rows
  int off[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int m = rg + u * RPI;
    off[u] = (g.layout == 1 ? m : (m >> 3) * g.W + (m & 7)) * D;
  }
  // first token row of each of this wave's blocks: one division chain for the first,
  // then patch steps (x, then y, then frame) for the others
  int brow[kPoolBlocks];
  {
    int px = i0 % g.Wp, py = (i0 / g.Wp) % g.Hp, t = i0 / (g.Wp * g.Hp);
#pragma unroll
    for (int b = 0; b < kPoolBlocks; ++b) {
      brow[b] = g.layout == 1 ? (i0 + b) * 64 : (t * g.H + py * 8) * g.W + px * 8;
      if (++px == g.Wp) {
        px = 0;
        if (++py == g.Hp) {
          py = 0;
          ++t;
        }
      }
    }
  }
  auto load = [&](int b, uint4* buf) {
    const T* src = base + (size_t)brow[b] * D;
#pragma unroll
    for (int u = 0; u < NL; ++u) buf[u] = *(const uint4*)(src + off[u]);
  };
  uint64_t st_max = 0ull, st_min = ~0ull, st_n = 0ull;   // this wave's key-block statistics
  auto process = [&](int i, const uint4* buf) {
    const int64_t r = bh * g.S + i;
    double acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
#pragma unroll
    for (int u = 0; u < NL; ++u) add_chunk<T>(acc, buf[u]);
    // combine the RPI row groups (lanes equal in the low log2(LPR) bits)
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      if constexpr (LPR <= 8) acc[e] += __shfl_xor(acc[e], 8, 64);
      if constexpr (LPR <= 16) acc[e] += xor16(acc[e], lane);
      acc[e] += xor32(acc[e], lane);
      acc[e] *= (1.0 / 64.0);
    }
    // row group 0 writes the means (every row group holds them)
    if (rg == 0) {
      double2* dst = (double2*)((keys ? kp : qp) + (size_t)r * D + c * EPC);
#pragma unroll
      for (int x = 0; x < EPC / 2; ++x) dst[x] = make_double2(acc[2 * x], acc[2 * x + 1]);
    }
    if constexpr (kScreen) {
      double s = 0.0;
#pragma unroll
      for (int e = 0; e < EPC; ++e) s += acc[e];
      const double mu = group_reduce<LPR>(s, lane, [](double a, double b) { return a + b; }) * (1.0 / D);
      double amax = 0.0, n2 = 0.0;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        acc[e] -= mu;
        amax = fmax(amax, fabs(acc[e]));
        n2 = fma(acc[e], acc[e], n2);
      }
      amax = group_reduce<LPR>(amax, lane, [](double a, double b) { return fmax(a, b); });
      n2 = group_reduce<LPR>(n2, lane, [](double a, double b) { return a + b; });
      const int ex = amax > 0.0 ? 13 - ilogb(amax) : 0;   // scaled magnitudes in [2^13, 2^14)
      // row group 0 writes the hi halves, row group 1 the lo halves
      if (rg < 2) {
        _Float16 h[EPC];
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          // double -> float -> fp16 on the hardware converts (the opaque copy keeps
          // the compiler from fusing them into a software double -> fp16 rounding)
          const double x = ldexp(acc[e], ex);
          float xf = (float)x;
          asm volatile("" : "+v"(xf));
          const _Float16 hi = (_Float16)xf;
          float rf = (float)(x - (double)hi);
          asm volatile("" : "+v"(rf));
          h[e] = rg == 0 ? hi : (_Float16)rf;
        }
        _Float16* dst;
        if (keys) {
          // key blocks in MFMA operand order: 16-block tiles, per 32-channel step s and
          // half (hi, lo) 1 KB holding, at lane slot 16 (channel / 8 % 4) + block % 16,
          // the 8 channels that lane of v_mfma_f32_16x16x32_f16 takes
          const int ch0 = c * EPC, cc = ch0 >> 3, s = cc >> 2, kg = cc & 3;
          const int64_t tile = bh * ((g.S + 15) / 16) + (i >> 4);
          dst = ops.ks + ((tile * (D / 32) + s) * 2 + rg) * 512 + (16 * kg + (i & 15)) * 8 + (ch0 & 7);
        } else {
          dst = ops.qs + (size_t)r * 2 * D + rg * D + c * EPC;
        }
        if constexpr (EPC == 8) {
          *(uint4*)dst = *(const uint4*)h;
        } else {
          *(uint2*)dst = *(const uint2*)h;
        }
      }
      const double nrm = sqrt(n2) * (1.0 + 0x1p-50);    // rounded up: an upper bound of |c|
      if (lane == 0) {
        if (keys) {
          ops.krec[r] = make_double2(mu, (double)ex);
        } else {
          ops.qmu[r] = mu;
          ops.qe[r] = ex;
          ops.qn[r] = nrm;
        }
      }
      const uint64_t km = order_key(mu), kn = order_key(nrm);
      st_max = km > st_max ? km : st_max;
      st_min = km < st_min ? km : st_min;
      st_n = kn > st_n ? kn : st_n;
    }
  };
  if (i0 < g.S) {
    // two register buffers; the scheduling barriers keep every load of the next
    // block issued before the sums of the current one
    uint4 ba[NL], bb[NL];
    load(0, ba);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < kPoolBlocks; b += 2) {
      const bool has1 = b + 1 < kPoolBlocks && i0 + b + 1 < g.S, has2 = b + 2 < kPoolBlocks && i0 + b + 2 < g.S;
      if (has1) load(b + 1, bb);
      __builtin_amdgcn_sched_barrier(0);
      process(i0 + b, ba);
      __builtin_amdgcn_sched_barrier(0);
      if (!has1) break;
      if (has2) load(b + 2, ba);
      __builtin_amdgcn_sched_barrier(0);
      process(i0 + b + 1, bb);
      __builtin_amdgcn_sched_barrier(0);
      if (!has2) break;
    }
  }
  if constexpr (kScreen) {
    if (!keys) return;                   // whole workgroup: z is uniform
    if (lane == 0) {
      red[0][wave] = st_max;
      red[1][wave] = st_min;
      red[2][wave] = st_n;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint64_t a = red[0][0], b = red[1][0], n = red[2][0];
      for (int w = 1; w < 4; ++w) {
        a = red[0][w] > a ? red[0][w] : a;
        b = red[1][w] < b ? red[1][w] : b;
        n = red[2][w] > n ? red[2][w] : n;
      }
      unsigned long long* hs = (unsigned long long*)(ops.hstat + 3 * bh);
      atomicMax(&hs[0], (unsigned long long)a);
      atomicMin(&hs[1], (unsigned long long)b);
      atomicMax(&hs[2], (unsigned long long)n);
    }
  }
}

template <bool kScreen>
static hipError_t launch_pool_impl(const Geom& g, const void* q, const void* k, double* qp, double* kp,
                                   const ScreenOps& ops, hipStream_t s, bool queries_only = false) {
  dim3 grid((unsigned)((g.S + 4 * kPoolBlocks - 1) / (4 * kPoolBlocks)), (unsigned)((int64_t)g.B * g.nh),
            queries_only ? 1u : 2u);
  if (g.dtype == 1 && g.D == 64)
    pool_kernel<uint16_t, 64, kScreen><<<grid, 256, 0, s>>>((const uint16_t*)q, (const uint16_t*)k, qp, kp, ops, g);
  else if (g.dtype == 1)
    pool_kernel<uint16_t, 128, kScreen><<<grid, 256, 0, s>>>((const uint16_t*)q, (const uint16_t*)k, qp, kp, ops, g);
  else if (g.D == 64)
    pool_kernel<float, 64, kScreen><<<grid, 256, 0, s>>>((const float*)q, (const float*)k, qp, kp, ops, g);
  else
    pool_kernel<float, 128, kScreen><<<grid, 256, 0, s>>>((const float*)q, (const float*)k, qp, kp, ops, g);
  return hipGetLastError();
}

hipError_t launch_pool(const Geom& g, const void* q, const void* k, double* qp, double* kp, hipStream_t s) {
  return launch_pool_impl<false>(g, q, k, qp, kp, ScreenOps{}, s);
}

hipError_t launch_pool_screen(const Geom& g, const void* q, const void* k, double* qp, double* kp,
                              const ScreenOps& ops, hipStream_t s) {
  return launch_pool_impl<true>(g, q, k, qp, kp, ops, s);
}

hipError_t launch_pool_queries_screen(const Geom& g, const void* q, double* qp, const ScreenOps& ops, hipStream_t s) {
  return launch_pool_impl<true>(g, q, q, qp, nullptr, ops, s, true);
}

}  // namespace bsa
