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
#include "mask_util.h"

namespace bsa {

// ---------------------------------------------------------------------------
// Block logits: z[bh][i][j] = (qp_i . kp_j) / sqrt(D), float64 GEMM per head on
// the float64 matrix cores (v_mfma_f64_16x16x4f64: A[i][k] in lane 16k + i,
// B[k][j] in lane 16k + j, C[i][j] in lane 16(i % 4) + j, register i / 4).
// 128 x 128 output tile per 256-thread workgroup, each wave a 64 x 64 quarter
// (4 x 4 MFMA tiles); k chunks of 16 staged in LDS k-major (so the 16 lanes of a
// fragment read 128 contiguous bytes), double-buffered: the next chunk is read
// into registers while the current one is multiplied.
// Sk key columns per head and heads h0 .. h0 + gridDim.z - 1 (z holds only those
// heads' rows).
// ---------------------------------------------------------------------------
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ void __launch_bounds__(256, 2) block_logits_kernel(const double* __restrict__ qp, const double* __restrict__ kp,
                                                           double* __restrict__ z, int Sq, int Sk, int64_t h0,
                                                           double inv_sqrt_d) {
  constexpr int TM = 128, KC = 16;
  __shared__ __attribute__((aligned(16))) double As[2][KC][TM];
  __shared__ __attribute__((aligned(16))) double Bs[2][KC][TM];
  const int64_t bh = h0 + blockIdx.z;
  const int i0 = blockIdx.y * TM, j0 = blockIdx.x * TM;
  const double* qh = qp + (size_t)bh * Sq * D;
  const double* kh = kp + (size_t)bh * Sk * D;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = (wave >> 1) * 64, wc = (wave & 1) * 64;   // this wave's quarter of the tile
  const int fi = lane & 15, fk = lane >> 4;                 // fragment row/col and k of this lane
  f64x4 acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = (f64x4){0.0, 0.0, 0.0, 0.0};
  // loader: row lr = tid >> 1, k half lk = (tid & 1) * 8; the next chunk is read
  // into registers while the current one is multiplied out of the other buffer
  const int lr = tid >> 1, lk = (tid & 1) * 8;
  const int gi = i0 + lr, gj = j0 + lr;
  const double* qrow = qh + (size_t)min(gi, Sq - 1) * D + lk;
  const double* krow = kh + (size_t)min(gj, Sk - 1) * D + lk;
  double ra[8], rb[8];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ra[e] = gi < Sq ? qrow[k0 + e] : 0.0;
      rb[e] = gj < Sk ? krow[k0 + e] : 0.0;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      As[buf][lk + e][lr] = ra[e];
      Bs[buf][lk + e][lr] = rb[e];
    }
  };
  fetch(0);
  stash(0);
  __syncthreads();
#pragma unroll 1
  for (int c = 0; c < D / KC; ++c) {
    const int buf = c & 1;
    if (c + 1 < D / KC) fetch((c + 1) * KC);
#pragma unroll
    for (int kk = 0; kk < KC; kk += 4) {
      double a[4], b[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) a[m] = As[buf][kk + fk][wr + 16 * m + fi];
#pragma unroll
      for (int n = 0; n < 4; ++n) b[n] = Bs[buf][kk + fk][wc + 16 * n + fi];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], b[n], acc[m][n], 0, 0, 0);
    }
    if (c + 1 < D / KC) stash(buf ^ 1);
    __syncthreads();
  }
  double* zh = z + (size_t)blockIdx.z * Sq * Sk;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gi = i0 + wr + 16 * m + 4 * r + fk;
      if (gi >= Sq) continue;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int gj = j0 + wc + 16 * n + fi;
        if (gj < Sk) zh[(size_t)gi * Sk + gj] = acc[m][n][r] * inv_sqrt_d;
      }
    }
}

static hipError_t launch_logits(const Geom& g, const double* qp, const double* kp, double* z, int Sk, int64_t h0,
                                int64_t nheads, hipStream_t s) {
  dim3 grid((Sk + 127) / 128, (g.S + 127) / 128, (unsigned)nheads);
  const double inv = 1.0 / sqrt((double)g.D);
  if (g.D == 64)
    block_logits_kernel<64><<<grid, 256, 0, s>>>(qp, kp, z, g.S, Sk, h0, inv);
  else
    block_logits_kernel<128><<<grid, 256, 0, s>>>(qp, kp, z, g.S, Sk, h0, inv);
  return hipGetLastError();
}

hipError_t launch_block_logits(const Geom& g, const double* qp, const double* kp, double* z, hipStream_t s) {
  return launch_logits(g, qp, kp, z, g.S, 0, (int64_t)g.B * g.nh, s);
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
// CDF cut, one wavefront per row (four rows per 256-thread workgroup, no
// workgroup barriers), by radix selection instead of a sort.
//
//   p_j = exp(z_j - max) / sum; order blocks by (p desc, j asc); c_k = exclusive
//   prefix mass of that order; keep position k iff k == 0 or c_k < 1 - thr;
//   thr == 0 keeps all.
//
// The order is decided on the float64 logits (p is monotone in z), so it is as
// exact as the logits.  Only the MASSES enter the comparison with 1 - thr, and
// for those float32 exponentials (relative error ~1e-6) are far inside the 1e-4
// band; they are accumulated as unsigned fixed-point integers in units of 2^-30
// of the row maximum (every partial sum exact, so the cut does not depend on
// summation order and is bitwise deterministic; the rounding of all masses
// together moves a prefix by less than S * 2^-30 < 4e-6).
//
// Selection: the kept set is every block ordered before the block at which the
// cumulative mass first reaches 1 - thr, and that block.  It is found in three
// steps, each exact with respect to the order above:
//   1. a 24-bit key t = (z - max - dmin) * (2^24 - 1) / (-dmin) in float32
//      (dmin = smallest candidate offset) -- a monotone function of z, so it
//      refines the order without breaking it, and it spreads even near-uniform
//      rows over the bins -- is radix-selected MSB-first, 8 bits and one
//      (count, mass) histogram per pass, until the crossing bin holds at most 64
//      blocks; blocks in higher bins are kept, blocks in lower bins dropped;
//   2. the crossing bin's blocks are compacted one per lane, their exact float64
//      logits gathered, and each lane sums the mass of the bin's blocks ordered
//      before its own (larger logit, or equal logit and smaller id): the exact
//      exclusive prefix;
//   3. only if more than 64 blocks share one 24-bit key (logits equal to ~1e-7
//      relative): MSB-first passes over the exact order-preserving key of the
//      logit, then exact ties by block id.
// Blocks whose mass is below 2^-30 of the maximum, or with z < max - lambda
// (lambda = 40 + ln S - ln thr, set by the host), are never candidates: the cut
// cannot reach them unless thr < 4e-6, and then they lie inside the band.
// ---------------------------------------------------------------------------
constexpr int kMaxS = 4096;

// The cut of row r from its float64 logits zr[0 .. S) (global memory or LDS),
// by one wavefront; umass / ucount / bm: that wavefront's LDS scratch.
template <int NS>
__device__ __forceinline__ void select_row(const double* zr, int64_t r, const Geom& g, double thr, double lambda,
                                           int win_t, int win_h, int win_w, uint64_t* umass, uint32_t* ucount,
                                           uint32_t* bm, uint32_t* __restrict__ bitmap, int32_t* __restrict__ counts,
                                           int words) {
  const int lane = threadIdx.x & 63;
  const int S = g.S;
  const int i = (int)(r % S);
  auto u64max = [](uint64_t a, uint64_t b) { return a > b ? a : b; };
  auto u64min = [](uint64_t a, uint64_t b) { return a < b ? a : b; };
  auto u64add = [](uint64_t a, uint64_t b) { return a + b; };
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
  auto set_bit = [&](int j) { atomicOr(&bm[j >> 5], 1u << (j & 31)); };
  // the lane index through an opaque copy: block ids l + 64 k are then recomputed
  // where used instead of being kept live in NS registers for the whole kernel
  auto lane_id = [&]() {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };

  if (thr == 0.0) {
    for (int x = lane; x < words; x += 64) {
      const int left = S - 32 * x;
      bm[x] = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
    }
  } else {
    for (int x = lane; x < words; x += 64) bm[x] = 0u;
    // slot k of lane l is block l + 64 k: mass in 2^-30 units of the row maximum
    // (0 = not a candidate) and the 24-bit monotone key
    uint32_t w[NS], t[NS];
    uint64_t total;
    {
      double zv[NS];
      double m = -DBL_MAX;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int j = lane + 64 * k;
        const double v = zr[min(j, S - 1)];   // unconditional, so all loads are in flight at once
        zv[k] = j < S ? v : -DBL_MAX;
        m = fmax(m, zv[k]);
      }
      m = wave_reduce(m, lane, [](double a, double b) { return fmax(a, b); });
      float df[NS];
      uint64_t wsum = 0;
      float dmin = 0.f;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const double d = zv[k] - m;
        const bool cand = (lane + 64 * k < S) && d >= -lambda;
        df[k] = (float)d;
        const float e = cand ? __builtin_amdgcn_exp2f(df[k] * 1.44269504088896341f) : 0.f;
        w[k] = (uint32_t)(e * 1073741824.0f);   // e <= 1, so at most 2^30; e * 2^30 is exact
        wsum += w[k];
        if (w[k] != 0u) dmin = fminf(dmin, df[k]);
      }
      total = wave_reduce(wsum, lane, u64add);
      dmin = wave_reduce(dmin, lane, [](float a, float b) { return fminf(a, b); });
      const float tscale = dmin < 0.f ? 16777215.0f / (-dmin) : 0.f;
#pragma unroll
      for (int k = 0; k < NS; ++k) t[k] = w[k] != 0u ? (uint32_t)fminf((df[k] - dmin) * tscale, 16777215.0f) : 0u;
    }
    const double target = (1.0 - thr) * (double)total;        // keep while exclusive prefix < target

    // Histogram of (count, mass) of the blocks with bin(k) >= 0, then the bin in
    // which the cumulative mass from the top (bin 255 first) reaches the target.
    // Returns false when no bin does (the target lies beyond every candidate).
    auto crossing = [&](auto bin, uint64_t above_in, int& b_out, uint64_t& above_out, uint32_t& cnt_out) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        ucount[4 * lane + x] = 0u;
        umass[4 * lane + x] = 0ull;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int b = w[k] != 0u ? bin(k) : -1;
        if (b >= 0) {
          atomicAdd(&ucount[b], 1u);
          atomicAdd((unsigned long long*)&umass[b], (unsigned long long)w[k]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      uint64_t mb[4];
      uint32_t cb[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        mb[x] = umass[4 * lane + x];
        cb[x] = ucount[4 * lane + x];
      }
      const uint64_t lane_tot = mb[0] + mb[1] + mb[2] + mb[3];
      uint64_t suf = lane_tot;                 // inclusive suffix sum over lanes
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t lo = __shfl_down((uint32_t)suf, d, 64), hi = __shfl_down((uint32_t)(suf >> 32), d, 64);
        if (lane + d < 64) suf += ((uint64_t)hi << 32) | lo;
      }
      uint64_t run = suf - lane_tot;
      int found = -1;
      uint64_t f_above = 0;
      uint32_t f_cnt = 0;
#pragma unroll
      for (int x = 3; x >= 0; --x) {
        const uint64_t excl = run;
        run += mb[x];
        if (cb[x] != 0u && (double)(above_in + excl) < target && target <= (double)(above_in + run)) {
          found = 4 * lane + x;
          f_above = above_in + excl;
          f_cnt = cb[x];
        }
      }
      __builtin_amdgcn_wave_barrier();         // the arrays are reused right after
      const uint64_t ball = __ballot(found >= 0);
      if (ball == 0ull) return false;
      const int src = __ffsll((unsigned long long)ball) - 1;
      b_out = __builtin_amdgcn_readlane(found, src);
      cnt_out = (uint32_t)__builtin_amdgcn_readlane((int)f_cnt, src);
      above_out = readlane_u64(f_above, src);
      return true;
    };

    // step 1: radix selection on the 24-bit key
    uint32_t tpre = 0;                         // decided high bits of the crossing key
    int tsh = 24;                              // bits below the decided prefix
    uint64_t above = 0;
    uint32_t cnt = 0;
    bool reach = true;
    while (tsh > 0) {
      const int sh = tsh - 8;
      const uint32_t pf = tpre;
      int b;
      uint64_t ab;
      uint32_t cb;
      if (!crossing([&](int k) { return (t[k] >> tsh) == pf ? (int)((t[k] >> sh) & 255u) : -1; }, above, b, ab, cb)) {
        reach = false;                         // only possible on the first pass
        break;
      }
      tpre = (pf << 8) | (uint32_t)b;
      tsh = sh;
      above = ab;
      cnt = cb;
      if (cnt <= 64u) break;
    }
    if (!reach) {                              // every candidate is kept
      const int ln = lane_id();
#pragma unroll
      for (int k = 0; k < NS; ++k)
        if (w[k] != 0u) set_bit(ln + 64 * k);
    } else {
      auto in_bin = [&](int k) { return w[k] != 0u && (t[k] >> tsh) == tpre; };
      {
        const int ln = lane_id();
#pragma unroll
        for (int k = 0; k < NS; ++k)
          if (w[k] != 0u && (t[k] >> tsh) > tpre) set_bit(ln + 64 * k);
      }
      if (cnt <= 64u) {
        // step 2: one block of the crossing bin per lane, exact logits gathered
        uint32_t* cj = ucount;
        uint32_t* cw = ucount + 64;
        uint32_t base = 0;
        const int ln = lane_id();
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          const bool in = in_bin(k);
          const uint64_t ball = __ballot(in);
          if (in) {
            const uint32_t rank = base + (uint32_t)__popcll(ball & lt_mask);
            cj[rank] = (uint32_t)(ln + 64 * k);
            cw[rank] = w[k];
          }
          base += (uint32_t)__popcll(ball);
        }
        __builtin_amdgcn_wave_barrier();
        const bool have = (uint32_t)lane < cnt;
        const uint32_t my_j = have ? cj[lane] : 0u;
        const uint32_t my_w = have ? cw[lane] : 0u;
        const uint64_t my_key = have ? order_key(zr[my_j]) : 0ull;
        uint64_t before = 0;
        for (uint32_t y = 0; y < cnt; ++y) {
          const uint64_t ky = readlane_u64(my_key, (int)y);
          const uint32_t jy = (uint32_t)__builtin_amdgcn_readlane((int)my_j, (int)y);
          const uint32_t wy = (uint32_t)__builtin_amdgcn_readlane((int)my_w, (int)y);
          if (ky > my_key || (ky == my_key && jy < my_j)) before += wy;
        }
        if (have && (double)(above + before) < target) set_bit((int)my_j);
      } else {
        // step 3 (more than 64 blocks share one 24-bit key): exact keys, re-read
        // from the logits where needed (rare, so registers are not spent on them)
        auto key_of = [&](int k) {
          const double* zl = zr;
          asm volatile("" : "+s"(zl));        // re-issue the load at each use
          return order_key(zl[lane + 64 * k]);
        };
        uint64_t kmax = 0, kmin = ~0ull;
        for (int k = 0; k < NS; ++k)
          if (in_bin(k)) {
            const uint64_t key = key_of(k);
            kmax = u64max(kmax, key);
            kmin = u64min(kmin, key);
          }
        kmax = wave_reduce(kmax, lane, u64max);
        kmin = wave_reduce(kmin, lane, u64min);
        const uint64_t diff = kmax ^ kmin;
        int shift = diff == 0 ? 0 : ((63 - __clzll(diff)) & ~7);
        uint64_t prefix = shift >= 56 ? 0ull : (kmax & (~0ull << (shift + 8)));
        for (;;) {
          const uint64_t hi_mask = shift >= 56 ? 0ull : (~0ull << (shift + 8));
          const int sh = shift;
          const uint64_t pf = prefix;
          int b;
          uint64_t ab;
          uint32_t cb;
          // the crossing block lies in this bin and shares the decided prefix, so
          // a bin is always found
          crossing(
              [&](int k) {
                if (!in_bin(k)) return -1;
                const uint64_t key = key_of(k);
                return (key & hi_mask) == pf ? (int)((key >> sh) & 255u) : -1;
              },
              above, b, ab, cb);
          prefix |= (uint64_t)b << shift;
          above = ab;
          cnt = cb;
          if (cnt <= 1u || shift == 0) break;
          shift -= 8;
        }
        const uint64_t hi_key = shift == 0 ? prefix : (prefix | ((1ull << shift) - 1));
        uint64_t tie_bits = 0;                 // bit k: slot k of this lane ties at the cut
        uint32_t wt = 0;
        for (int k = 0; k < NS; ++k)
          if (in_bin(k)) {
            const uint64_t key = key_of(k);
            if (key > hi_key || (cnt <= 1u && key >= prefix)) set_bit(lane + 64 * k);
            if (cnt > 1u && key == prefix) {
              tie_bits |= 1ull << k;
              wt = w[k];
            }
          }
        if (cnt > 1u) {
          // exact ties at the cut: the lowest block ids, until the mass reaches the
          // target; slots then lanes run in block-id order, and ties share one mass
          wt = wave_reduce(wt, lane, [](uint32_t a, uint32_t b2) { return a > b2 ? a : b2; });
          uint64_t acc = above;
          for (int k = 0; k < NS; ++k) {
            const uint64_t tb = __ballot((tie_bits >> k) & 1ull);
            if (((tie_bits >> k) & 1ull) && (double)(acc + (uint64_t)__popcll(tb & lt_mask) * wt) < target)
              set_bit(lane + 64 * k);
            acc += (uint64_t)__popcll(tb) * wt;
          }
        }
      }
    }
  }
  if (win_t >= 0) for_each_window_block(g, i, win_t, win_h, win_w, lane, 64, set_bit);
  __builtin_amdgcn_wave_barrier();
  uint32_t pc = 0;
  for (int x = lane; x < words; x += 64) {
    const uint32_t v = bm[x];
    bitmap[r * words + x] = v;
    pc += __popc(v);
  }
  pc = wave_reduce(pc, lane, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 0) counts[r] = (int32_t)pc;
}

template <int NS>
__global__ void __launch_bounds__(256) select_kernel(const double* __restrict__ z, Geom g, double thr, double lambda,
                                                     int win_t, int win_h, int win_w, uint32_t* __restrict__ bitmap,
                                                     int32_t* __restrict__ counts, int words) {
  __shared__ uint64_t umass_all[4][256];
  __shared__ uint32_t ucount_all[4][256];
  __shared__ uint32_t bm_all[4][kMaxS / 32];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  if (r >= g.rows) return;                     // whole wavefront; nothing below waits on other waves
  select_row<NS>(z + r * g.S, r, g, thr, lambda, win_t, win_h, win_w, umass_all[wv], ucount_all[wv], bm_all[wv],
                 bitmap, counts, words);
}

// Rows the screened cut left undecided (see mask_screen.hip): their float64 logits
// are computed into LDS and cut by select_row.  A persistent grid walks the list
// the screened cut filled (its length is read on the device).
template <int NS>
__global__ void __launch_bounds__(256) fallback_select_kernel(const double* __restrict__ qp,
                                                              const double* __restrict__ kp, Geom g, double thr,
                                                              double lambda, int win_t, int win_h, int win_w,
                                                              uint32_t* __restrict__ bitmap,
                                                              int32_t* __restrict__ counts, int words,
                                                              const int32_t* __restrict__ flag_list,
                                                              const int32_t* __restrict__ nflag, double inv_sqrt_d) {
  __shared__ double zrow[kMaxS];
  __shared__ uint64_t umass[256];
  __shared__ uint32_t ucount[256];
  __shared__ uint32_t bm[kMaxS / 32];
  const int n = *nflag;
  for (int x = blockIdx.x; x < n; x += gridDim.x) {
    const int64_t r = flag_list[x];
    const int64_t bh = r / g.S;
    const double* qrow = qp + (size_t)r * g.D;
    __syncthreads();                     // the previous row's cut has finished with zrow
    for (int j = threadIdx.x; j < g.S; j += 256) {
      const double* krow = kp + (size_t)(bh * g.S + j) * g.D;
      double z = 0.0;
      for (int d = 0; d < g.D; ++d) z = fma(qrow[d], krow[d], z);
      zrow[j] = z * inv_sqrt_d;
    }
    __syncthreads();
    if (threadIdx.x < 64)
      select_row<NS>(zrow, r, g, thr, lambda, win_t, win_h, win_w, umass, ucount, bm, bitmap, counts, words);
  }
}

hipError_t launch_fallback_select(const Geom& g, const double* qp, const double* kp, double thr, double lambda,
                                  int win_t, int win_h, int win_w, uint32_t* bitmap, int32_t* counts, int words,
                                  const int32_t* flag_list, const int32_t* nflag, hipStream_t s) {
  const double inv = 1.0 / sqrt((double)g.D);
  const unsigned grid = 512;
#define BSA_FALLBACK(NS_)                                                                                      \
  fallback_select_kernel<NS_><<<grid, 256, 0, s>>>(qp, kp, g, thr, lambda, win_t, win_h, win_w, bitmap, counts, \
                                                   words, flag_list, nflag, inv)
  if (g.S <= 128) BSA_FALLBACK(2);
  else if (g.S <= 512) BSA_FALLBACK(8);
  else if (g.S <= 1024) BSA_FALLBACK(16);
  else if (g.S <= 2048) BSA_FALLBACK(32);
  else BSA_FALLBACK(64);
#undef BSA_FALLBACK
  return hipGetLastError();
}

hipError_t launch_select(const Geom& g, const double* z, double thr, double lambda, int win_t, int win_h, int win_w,
                         uint32_t* bitmap, int32_t* counts, int words, hipStream_t s) {
  const unsigned grid = (unsigned)((g.rows + 3) / 4);
#define BSA_SELECT(NS_) \
  select_kernel<NS_><<<grid, 256, 0, s>>>(z, g, thr, lambda, win_t, win_h, win_w, bitmap, counts, words)
  if (g.S <= 128) BSA_SELECT(2);
  else if (g.S <= 512) BSA_SELECT(8);
  else if (g.S <= 1024) BSA_SELECT(16);
  else if (g.S <= 2048) BSA_SELECT(32);
  else BSA_SELECT(64);
#undef BSA_SELECT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// SIP: sampling with inclusion-probability weights (AB-Attention page, "Los tres
// recursos de AB-Attention", second resource), one wavefront per row.
//
//   p_j  = exp(z_j - max) / sum                       (the reduced map, float64)
//   pi_top = 1 for the row's top block (largest p, lowest id on ties), and for
//   the others pi_j = min(1, c p_j),  sum_j pi_j = k  (k = the row's CDF-cut count)
//   take j iff u_rj < pi_j,  u_rj from Philox4x64-10 at counter (r, floor(j/4), 0, 0),
//   key (seed, 0): u = (word_(j mod 4) >> 11) * 2^-53 (one generator block serves
//   four consecutive blocks of the row)
//
// c is found by capping: c = (k - t) / (mass of the uncapped blocks), then every
// uncapped block with c p_j >= 1 is capped (pi = 1) and c recomputed, until none
// is; c only grows along the way, so the capped blocks are exactly those with
// c p_j >= 1 for the final c.  The row's (max, sum, c) are kept so that the
// compaction recomputes pi of every taken block bit for bit and writes its
// logit shift log(1 / pi); the top block's id is kept with them.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_prob(double z, double m, double sum) { return exp(z - m) / sum; }
__device__ __forceinline__ double incl_prob(double p, double c) { return p > 0.0 ? fmin(1.0, c * p) : 0.0; }

// Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw: "Parallel random numbers:
// as easy as 1, 2, 3", SC 2011): the four words of the block at counter
// (c0, c1, 0, 0), key (k0, 0).
__device__ __forceinline__ void philox4x64(uint64_t c0, uint64_t c1, uint64_t k0, uint64_t (&w)[4]) {
  uint64_t x0 = c0, x1 = c1, x2 = 0, x3 = 0, key0 = k0, key1 = 0;
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    const uint64_t hi0 = __umul64hi(x0, 0xD2E7470EE14C6C93ull), lo0 = x0 * 0xD2E7470EE14C6C93ull;
    const uint64_t hi1 = __umul64hi(x2, 0xCA5A826395121157ull), lo1 = x2 * 0xCA5A826395121157ull;
    x0 = hi1 ^ x1 ^ key0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ key1;
    x3 = lo0;
    key0 += 0x9E3779B97F4A7C15ull;
    key1 += 0xBB67AE8584CAA73Bull;
  }
  w[0] = x0;
  w[1] = x1;
  w[2] = x2;
  w[3] = x3;
}

template <int NS>
__global__ void __launch_bounds__(256) sip_kernel(const double* __restrict__ z, Geom g, double thr, uint64_t seed,
                                                  int win_t, int win_h, int win_w, uint32_t* __restrict__ bitmap,
                                                  int32_t* __restrict__ counts, double* __restrict__ rowstat,
                                                  int words) {
  __shared__ uint32_t bm_all[4][kMaxS / 32];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int64_t r = (int64_t)blockIdx.x * 4 + wv;
  if (r >= g.rows) return;                     // whole wavefront; nothing below waits on other waves
  uint32_t* bm = bm_all[wv];
  const int S = g.S;
  const int i = (int)(r % S);
  const double* zr = z + r * S;
  auto set_bit = [&](int j) { atomicOr(&bm[j >> 5], 1u << (j & 31)); };
  auto dsum = [&](double v) { return wave_reduce(v, lane, [](double a, double b) { return a + b; }); };
  auto isum = [&](int v) {
    return (int)wave_reduce((uint32_t)v, lane, [](uint32_t a, uint32_t b) { return a + b; });
  };
  const int budget = counts[r];                // the CDF cut's count for this row

  double m = 0.0, sum = 1.0, c = HUGE_VAL;
  int top = -1;
  if (thr == 0.0) {
    for (int x = lane; x < words; x += 64) {
      const int left = S - 32 * x;
      bm[x] = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
    }
  } else {
    for (int x = lane; x < words; x += 64) bm[x] = 0u;
    // slot k of this lane holds block jk(k): lane groups of four consecutive blocks,
    // so that one generator block serves a lane's four draws
    auto jk = [&](int k) { return 4 * (lane + 64 * (k >> 2)) + (k & 3); };
    double p[NS];
    m = -DBL_MAX;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const int j = jk(k);
      const double v = zr[min(j, S - 1)];
      p[k] = j < S ? v : -DBL_MAX;
      m = fmax(m, p[k]);
    }
    m = wave_reduce(m, lane, [](double a, double b) { return fmax(a, b); });
    double part = 0.0;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      p[k] = jk(k) < S ? exp(p[k] - m) : 0.0;
      part += p[k];
    }
    sum = dsum(part);
    int pos = 0;
    double pmax = 0.0;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      p[k] = p[k] / sum;                       // = block_prob(z_j, m, sum), the same operations
      pos += p[k] > 0.0;
      pmax = fmax(pmax, p[k]);
    }
    pos = isum(pos);
    pmax = wave_reduce(pmax, lane, [](double a, double b) { return fmax(a, b); });
    // the row's top block (largest probability, lowest id on ties) is always taken
    int tj = S;
#pragma unroll
    for (int k = 0; k < NS; ++k)
      if (p[k] == pmax) tj = min(tj, jk(k));
    top = (int)wave_reduce((uint32_t)tj, lane, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    // the others share budget - 1: min(1, c p_j), capped blocks found by iteration
    const int kk = budget - 1;
    if (kk <= 0) {
      c = 0.0;
    } else if (kk < pos - 1) {
      uint64_t capped = 0;                     // bit k: slot k of this lane is capped (or the top block)
#pragma unroll
      for (int k = 0; k < NS; ++k)
        if (jk(k) == top) capped |= 1ull << k;
      int t = 0;
      for (int it = 0; it <= S; ++it) {        // every pass caps at least one block
        double rest = 0.0;
#pragma unroll
        for (int k = 0; k < NS; ++k)
          if (!((capped >> k) & 1ull)) rest += p[k];
        c = (double)(kk - t) / dsum(rest);
        int fresh = 0;
#pragma unroll
        for (int k = 0; k < NS; ++k)
          if (!((capped >> k) & 1ull) && p[k] > 0.0 && c * p[k] >= 1.0) {
            capped |= 1ull << k;
            ++fresh;
          }
        fresh = isum(fresh);
        if (fresh == 0) break;
        t += fresh;
        // the budget is spent on capped blocks only when every other block has
        // zero mass; keep the last c (> 0), for which the capped blocks give pi = 1
        if (t >= kk) break;
      }
    }                                          // else c stays +inf: every positive block is taken
#pragma unroll
    for (int kq = 0; kq < NS / 4; ++kq) {
      // u in [0, 1): pi >= 1 is always taken and pi == 0 never, so the generator
      // runs only where one of the four blocks needs a draw
      const int q = lane + 64 * kq;            // blocks 4q .. 4q+3, generator counter (r, q)
      double pi[4];
      bool draw = false;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int j = 4 * q + w;
        pi[w] = j >= S ? 0.0 : (j == top ? 1.0 : incl_prob(p[4 * kq + w], c));
        if (pi[w] >= 1.0) set_bit(j);
        draw |= pi[w] > 0.0 && pi[w] < 1.0;
      }
      if (draw) {
        uint64_t u64[4];
        philox4x64((uint64_t)r, (uint64_t)q, seed, u64);
#pragma unroll
        for (int w = 0; w < 4; ++w)
          if (pi[w] > 0.0 && pi[w] < 1.0 && (double)(u64[w] >> 11) * 0x1p-53 < pi[w]) set_bit(4 * q + w);
      }
    }
  }
  if (win_t >= 0) for_each_window_block(g, i, win_t, win_h, win_w, lane, 64, set_bit);
  __builtin_amdgcn_wave_barrier();
  uint32_t pc = 0;
  for (int x = lane; x < words; x += 64) {
    const uint32_t v = bm[x];
    bitmap[r * words + x] = v;
    pc += __popc(v);
  }
  pc = wave_reduce(pc, lane, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 0) {
    counts[r] = (int32_t)pc;
    rowstat[4 * r + 0] = m;
    rowstat[4 * r + 1] = sum;
    rowstat[4 * r + 2] = c;
    rowstat[4 * r + 3] = (double)top;
  }
}

hipError_t launch_sip(const Geom& g, const double* z, double thr, uint64_t seed, int win_t, int win_h, int win_w,
                      uint32_t* bitmap, int32_t* counts, double* rowstat, int words, hipStream_t s) {
  const unsigned grid = (unsigned)((g.rows + 3) / 4);
#define BSA_SIP(NS_) \
  sip_kernel<NS_><<<grid, 256, 0, s>>>(z, g, thr, seed, win_t, win_h, win_w, bitmap, counts, rowstat, words)
  if (g.S <= 256) BSA_SIP(4);
  else if (g.S <= 512) BSA_SIP(8);
  else if (g.S <= 1024) BSA_SIP(16);
  else if (g.S <= 2048) BSA_SIP(32);
  else BSA_SIP(64);
#undef BSA_SIP
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
// Bitmap -> ascending column list; one wavefront per row, 64 bitmap words
// (2048 columns) per step: popcounts and an exclusive scan across the lanes give
// each word's output offset; a sparse step lets each lane write its own word's
// column ids, a dense one walks the columns in order, 64 per ballot.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) compact_kernel(const uint32_t* __restrict__ bitmap, int words,
                                                      const int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx,
                                                      int64_t rows, int S) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const uint32_t* bm = bitmap + r * words;
  int32_t base = row_ptr[r];
  for (int x0 = 0; x0 < words; x0 += 64) {
    const int x = x0 + lane;
    uint32_t wbits = x < words ? bm[x] : 0u;
    if (32 * x + 32 > S) wbits &= x * 32 >= S ? 0u : ((1u << (S - 32 * x)) - 1u);   // columns >= S
    const int pc = __popc(wbits);
    int incl = pc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int total = __shfl(incl, 63, 64);
    if (total > 256) {
      // dense step: columns in order, 64 per ballot, so the stores are coalesced
      const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      int32_t b2 = base;
      for (int c = 0; c < 32; ++c) {
        const uint32_t wv = (uint32_t)__shfl((int)wbits, 2 * c + (lane >> 5), 64);   // word of column 64c + lane
        const bool on = (wv >> (lane & 31)) & 1u;
        const uint64_t msk = __ballot(on);
        if (on) col_idx[b2 + __popcll(msk & lt)] = 32 * x0 + 64 * c + lane;
        b2 += __popcll(msk);
      }
    } else {
      // sparse step: each lane writes its own word's columns
      int32_t* out = col_idx + base + (incl - pc);
      while (wbits) {
        const int b = __ffs(wbits) - 1;
        *out++ = 32 * x + b;
        wbits &= wbits - 1u;
      }
    }
    base += total;
  }
}

hipError_t launch_compact(const Geom& g, const uint32_t* bitmap, int words, const int32_t* row_ptr, int32_t* col_idx,
                          hipStream_t s) {
  compact_kernel<<<(unsigned)((g.rows + 3) / 4), 256, 0, s>>>(bitmap, words, row_ptr, col_idx, g.rows, g.S);
  return hipGetLastError();
}

// The same compaction for a SIP mask, which also writes each entry's logit shift
// log(1 / pi) from the row's (max, sum, c); window blocks, the top block and
// thr == 0 rows carry shift 0.
__global__ void __launch_bounds__(256) compact_sip_kernel(const uint32_t* __restrict__ bitmap, int words,
                                                          const int32_t* __restrict__ row_ptr,
                                                          int32_t* __restrict__ col_idx, float* __restrict__ shift,
                                                          const double* __restrict__ z,
                                                          const double* __restrict__ rowstat, Geom g, double thr,
                                                          int win_t, int win_h, int win_w) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= g.rows) return;
  const int S = g.S;
  const int i = (int)(r % S);
  const uint32_t* bm = bitmap + r * words;
  const double m = rowstat[4 * r], sum = rowstat[4 * r + 1], c = rowstat[4 * r + 2];
  const int top = (int)rowstat[4 * r + 3];
  // -log(min(1, c * exp(z - m) / sum)) = max(0, log(sum) - log(c) - (z - m)): one log pair
  // per row instead of an exp and a log per entry (c = inf gives 0: every block certain)
  const double lsc = log(sum) - log(c);
  int32_t base = row_ptr[r];
  for (int j0 = 0; j0 < S; j0 += 64) {
    const int j = j0 + lane;
    const uint32_t wv = bm[min(j >> 5, words - 1)];
    const bool on = j < S && ((wv >> (j & 31)) & 1u);
    const uint64_t mask = __ballot(on);
    if (on) {
      const int32_t slot = base + __popcll(mask & ((1ull << lane) - 1));
      col_idx[slot] = j;
      float sh = 0.f;
      if (thr != 0.0 && j != top && !(win_t >= 0 && in_window(g, i, j, win_t, win_h, win_w)))
        sh = (float)fmax(0.0, lsc - (z[r * S + j] - m));
      shift[slot] = sh;
    }
    base += __popcll(mask);
  }
}

hipError_t launch_compact_sip(const Geom& g, const uint32_t* bitmap, int words, const int32_t* row_ptr,
                              int32_t* col_idx, float* shift, const double* z, const double* rowstat, double thr,
                              int win_t, int win_h, int win_w, hipStream_t s) {
  compact_sip_kernel<<<(unsigned)((g.rows + 3) / 4), 256, 0, s>>>(bitmap, words, row_ptr, col_idx, shift, z, rowstat,
                                                                  g, thr, win_t, win_h, win_w);
  return hipGetLastError();
}

}  // namespace bsa
