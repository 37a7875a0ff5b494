// Key-group mask, the float64 path (AB-Attention page, news.hamidun.com/es/news/14960,
// "Los tres recursos de AB-Attention", third resource: 4-token key/value blocks),
// cut with the NABLA reduced map and CDF cut taken at group granularity (NABLA
// page, gist.science/es/paper/2507.13546, Metodologia item 2, "Atencion Reducida"
// and "Umbralizacion CDF"; item 3 for the window union).
//
// The rows the screened cut (group_screen.hip) cannot decide are cut here from
// float64 logits: group_fallback_kernel walks the list of such rows with a
// persistent grid, computes each row's L/4 logits qp_i . kg_j / sqrt(D) (kg_j the
// float64 mean of group j's 4 keys) into its own float64 scratch row, and cuts it with select_row: the float32 offsets
// z - max in LDS (4 B per entry), the masses float32 exponentials in fixed point
// (2^-30 of the row max) summed exactly, the 24-bit monotone key radix-selected
// 8 bits per pass until the crossing bin holds <= 256 entries, which are then
// ranked exactly on their float64 logits (ties by index); more than 256 entries
// with one 24-bit key fall back to passes over the exact 64-bit order keys, then
// index order.
#include <float.h>

#include "kernels.h"
#include "mask_util.h"
#include "validate.h"

namespace bsa {
namespace gmask {

constexpr int kMaxSG = 32768;     // groups per head the LDS row buffer holds
constexpr int kNT = 1024;         // threads per row: the LDS row buffer allows one workgroup
constexpr int kNW = kNT / 64;     // per CU, so the row gets 16 waves to hide its loads
constexpr int kFallbackWGs = kGroupFallbackRows;   // persistent grid, one float64 scratch row each

struct SelectSmem {
  float dv[kMaxSG];                   // (float)(z - max) of candidates, -inf otherwise
  uint32_t bm[kMaxSG / 32];           // kept bits of the row
  uint32_t hc[256];                   // radix bins: counts
  unsigned long long hm[256];         //             masses
  uint32_t cj[256], cw[256];          // crossing entries: index, mass
  unsigned long long ck[256];         //                   exact order key
  unsigned long long red_u[kNW];
  double red_d[kNW];
  float red_f[kNW];
  unsigned long long scan[kNW];
  int found_bin;
  uint32_t found_cnt, ncross;
  unsigned long long found_above;
};

__device__ __forceinline__ unsigned long long shfl_up_u64(unsigned long long v, int d) {
  const uint32_t lo = __shfl_up((uint32_t)v, d, 64), hi = __shfl_up((uint32_t)(v >> 32), d, 64);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int d) {
  const uint32_t lo = __shfl_xor((uint32_t)v, d, 64), hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
  return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int d) {
  return __longlong_as_double((long long)shfl_xor_u64((unsigned long long)__double_as_longlong(v), d));
}

// The cut of row r from its float64 logits zr (global memory, L/4 entries); m_part:
// this thread's share of the row max.  Called by all kNT threads of the workgroup.
__device__ __forceinline__ void select_row(const double* __restrict__ zr, double m_part, int64_t r, int SG,
                                           const Geom& g, double thr, double lambda, int win_t, int win_h,
                                           int win_w, uint32_t* __restrict__ bitmap, int32_t* __restrict__ counts,
                                           int words, SelectSmem& sm) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int i = (int)(r % g.S);
  const int gpb = g.N / 4;
  for (int x = tid; x < words; x += kNT) sm.bm[x] = 0u;

  // workgroup reductions (fixed tree order, deterministic)
  auto sum_u64 = [&](unsigned long long v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v += shfl_xor_u64(v, d);
    if (lane == 0) sm.red_u[wv] = v;
    __syncthreads();
    unsigned long long t = 0;
    for (int x = 0; x < kNW; ++x) t += sm.red_u[x];
    __syncthreads();
    return t;
  };
  auto max_u64 = [&](unsigned long long v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) { const unsigned long long o = shfl_xor_u64(v, d); v = o > v ? o : v; }
    if (lane == 0) sm.red_u[wv] = v;
    __syncthreads();
    unsigned long long t = sm.red_u[0];
    for (int x = 1; x < kNW; ++x) t = sm.red_u[x] > t ? sm.red_u[x] : t;
    __syncthreads();
    return t;
  };
  auto min_u64 = [&](unsigned long long v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) { const unsigned long long o = shfl_xor_u64(v, d); v = o < v ? o : v; }
    if (lane == 0) sm.red_u[wv] = v;
    __syncthreads();
    unsigned long long t = sm.red_u[0];
    for (int x = 1; x < kNW; ++x) t = sm.red_u[x] < t ? sm.red_u[x] : t;
    __syncthreads();
    return t;
  };
  auto max_f64 = [&](double v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v = fmax(v, shfl_xor_f64(v, d));
    if (lane == 0) sm.red_d[wv] = v;
    __syncthreads();
    double t = sm.red_d[0];
    for (int x = 1; x < kNW; ++x) t = fmax(t, sm.red_d[x]);
    __syncthreads();
    return t;
  };
  auto min_f32 = [&](float v) {
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) v = fminf(v, __shfl_xor(v, d, 64));
    if (lane == 0) sm.red_f[wv] = v;
    __syncthreads();
    float t = sm.red_f[0];
    for (int x = 1; x < kNW; ++x) t = fminf(t, sm.red_f[x]);
    __syncthreads();
    return t;
  };
  // inclusive prefix sum of one value per thread, thread order
  auto incl_scan_u64 = [&](unsigned long long v) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const unsigned long long o = shfl_up_u64(v, d);
      if (lane >= d) v += o;
    }
    if (lane == 63) sm.scan[wv] = v;
    __syncthreads();
    unsigned long long base = 0;
    for (int x = 0; x < wv; ++x) base += sm.scan[x];
    __syncthreads();
    return base + v;
  };
  auto set_bit = [&](int j) { atomicOr(&sm.bm[j >> 5], 1u << (j & 31)); };

  if (thr == 0.0) {
    for (int x = tid; x < words; x += kNT) {
      const int left = SG - 32 * x;
      sm.bm[x] = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
    }
  } else {
    // one pass over the logits: candidates, masses, offsets into LDS (four loads
    // in flight per thread)
    const double m = max_f64(m_part);
    unsigned long long wsum = 0;
    float dmin = 0.f;
    for (int j0 = tid; j0 < SG; j0 += 4 * kNT) {
      double v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = zr[min(j0 + u * kNT, SG - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u * kNT;
        if (j >= SG) continue;
        const double d = v[u] - m;
        const float df = (float)d;
        const float e = d >= -lambda ? __builtin_amdgcn_exp2f(df * 1.44269504088896341f) : 0.f;
        const uint32_t w = (uint32_t)(e * 1073741824.0f);   // e <= 1: at most 2^30, exact
        sm.dv[j] = w != 0u ? df : -INFINITY;
        wsum += w;
        if (w != 0u) dmin = fminf(dmin, df);
      }
    }
    const unsigned long long total = sum_u64(wsum);     // (its barriers also publish dv)
    dmin = min_f32(dmin);
    const float tscale = dmin < 0.f ? 16777215.0f / (-dmin) : 0.f;
    const double target = (1.0 - thr) * (double)total;   // keep while exclusive prefix < target
    // 24-bit key of a candidate offset, and its mass, recomputed exactly as above
    auto key_of = [&](float df) { return (uint32_t)fminf((df - dmin) * tscale, 16777215.0f); };
    auto mass_of = [&](float df) {
      return (uint32_t)(__builtin_amdgcn_exp2f(df * 1.44269504088896341f) * 1073741824.0f);
    };
    // one radix pass: (count, mass) histogram of bin(j) >= 0, then the bin in
    // which the cumulative mass from the top (bin 255 first) reaches the target
    auto crossing = [&](auto bin, unsigned long long above_in, int& b_out, unsigned long long& above_out,
                        uint32_t& cnt_out) {
      if (tid < 256) {
        sm.hc[tid] = 0u;
        sm.hm[tid] = 0ull;
      }
      if (tid == 0) sm.found_bin = -1;
      __syncthreads();
      for (int j = tid; j < SG; j += kNT) {
        const float df = sm.dv[j];
        if (df == -INFINITY) continue;
        const int b = bin(j, df);
        if (b >= 0) {
          atomicAdd(&sm.hc[b], 1u);
          atomicAdd(&sm.hm[b], (unsigned long long)mass_of(df));
        }
      }
      __syncthreads();
      const int b = 255 - min(tid, 255);                 // threads 0..255: bins from the top
      const unsigned long long mb = tid < 256 ? sm.hm[b] : 0ull;
      const unsigned long long incl = incl_scan_u64(mb);
      const unsigned long long excl = incl - mb;
      if (tid < 256 && sm.hc[b] != 0u && (double)(above_in + excl) < target &&
          target <= (double)(above_in + incl)) {
        sm.found_bin = b;
        sm.found_above = above_in + excl;
        sm.found_cnt = sm.hc[b];
      }
      __syncthreads();
      b_out = sm.found_bin;
      above_out = sm.found_above;
      cnt_out = sm.found_cnt;
      __syncthreads();                                   // bins and results are reused next pass
      return b_out >= 0;
    };

    uint32_t tpre = 0;
    int tsh = 24;
    unsigned long long above = 0;
    uint32_t cnt = 0;
    bool reach = true;
    while (tsh > 0) {
      const int sh = tsh - 8;
      const uint32_t pf = tpre;
      const int tshc = tsh;
      int b;
      unsigned long long ab;
      uint32_t cb;
      if (!crossing(
              [&](int, float df) {
                const uint32_t t = key_of(df);
                return (t >> tshc) == pf ? (int)((t >> sh) & 255u) : -1;
              },
              above, b, ab, cb)) {
        reach = false;                                   // only possible on the first pass
        break;
      }
      tpre = (pf << 8) | (uint32_t)b;
      tsh = sh;
      above = ab;
      cnt = cb;
      if (cnt <= 256u) break;
    }
    auto in_bin = [&](float df) { return df != -INFINITY && (key_of(df) >> tsh) == tpre; };
    if (!reach) {                                        // every candidate is kept
      for (int j = tid; j < SG; j += kNT)
        if (sm.dv[j] != -INFINITY) set_bit(j);
    } else {
      for (int j = tid; j < SG; j += kNT) {
        const float df = sm.dv[j];
        if (df != -INFINITY && (key_of(df) >> tsh) > tpre) set_bit(j);
      }
      if (cnt <= 256u) {
        // the crossing bin's entries, ranked exactly on their float64 logits
        if (tid == 0) sm.ncross = 0u;
        __syncthreads();
        for (int j = tid; j < SG; j += kNT) {
          const float df = sm.dv[j];
          if (in_bin(df)) {
            const uint32_t x = atomicAdd(&sm.ncross, 1u);
            sm.cj[x] = (uint32_t)j;
            sm.cw[x] = mass_of(df);
            sm.ck[x] = order_key(zr[j]);
          }
        }
        __syncthreads();
        const uint32_t n = sm.ncross;
        if ((uint32_t)tid < n) {
          const uint32_t my_j = sm.cj[tid];
          const unsigned long long my_k = sm.ck[tid];
          unsigned long long before = 0;
          for (uint32_t y = 0; y < n; ++y) {
            const unsigned long long ky = sm.ck[y];
            if (ky > my_k || (ky == my_k && sm.cj[y] < my_j)) before += sm.cw[y];
          }
          if ((double)(above + before) < target) set_bit((int)my_j);
        }
      } else {
        // more than 256 entries share one 24-bit key: exact 64-bit keys, then ties
        unsigned long long kmax = 0, kmin = ~0ull;
        for (int j = tid; j < SG; j += kNT) {
          if (in_bin(sm.dv[j])) {
            const unsigned long long key = order_key(zr[j]);
            kmax = key > kmax ? key : kmax;
            kmin = key < kmin ? key : kmin;
          }
        }
        kmax = max_u64(kmax);
        kmin = min_u64(kmin);
        const unsigned long long diff = kmax ^ kmin;
        int shift = diff == 0 ? 0 : ((63 - __clzll(diff)) & ~7);
        unsigned long long prefix = shift >= 56 ? 0ull : (kmax & (~0ull << (shift + 8)));
        for (;;) {
          const unsigned long long hi_mask = shift >= 56 ? 0ull : (~0ull << (shift + 8));
          const int sh = shift;
          const unsigned long long pf = prefix;
          int b;
          unsigned long long ab;
          uint32_t cb;
          // the crossing entry lies in this bin and shares the decided prefix,
          // so a bin is always found
          crossing(
              [&](int j, float df) {
                if (!in_bin(df)) return -1;
                const unsigned long long key = order_key(zr[j]);
                return (key & hi_mask) == pf ? (int)((key >> sh) & 255u) : -1;
              },
              above, b, ab, cb);
          prefix |= (unsigned long long)b << shift;
          above = ab;
          cnt = cb;
          if (cnt <= 1u || shift == 0) break;
          shift -= 8;
        }
        const unsigned long long hi_key = shift == 0 ? prefix : (prefix | ((1ull << shift) - 1));
        uint32_t wt = 0;
        for (int j = tid; j < SG; j += kNT) {
          const float df = sm.dv[j];
          if (in_bin(df)) {
            const unsigned long long key = order_key(zr[j]);
            if (key > hi_key || (cnt <= 1u && key >= prefix)) set_bit(j);
            if (cnt > 1u && key == prefix) wt = mass_of(df);
          }
        }
        if (cnt > 1u) {
          // exact ties at the cut: lowest indices first while the mass stays below
          // the target; all tied entries have the same logit, hence the same mass
          wt = (uint32_t)max_u64(wt);
          unsigned long long acc = above;
          for (int base = 0; base < SG; base += kNT) {
            const int j = base + tid;
            const bool tie = j < SG && in_bin(sm.dv[j]) && order_key(zr[j]) == prefix;
            const unsigned long long incl = incl_scan_u64(tie ? 1ull : 0ull);
            if (tie && (double)(acc + (incl - 1) * wt) < target) set_bit(j);
            acc += sum_u64(tie ? 1ull : 0ull) * wt;
          }
        }
      }
    }
  }
  __syncthreads();
  if (win_t >= 0)   // every group of every window block (gpb groups per block)
    for (int x = 0; x < gpb; ++x)
      for_each_window_block(g, i, win_t, win_h, win_w, tid, kNT, [&](int jb) { set_bit(jb * gpb + x); });
  __syncthreads();
  unsigned long long pc = 0;
  for (int x = tid; x < words; x += kNT) {
    const uint32_t v = sm.bm[x];
    bitmap[r * words + x] = v;
    pc += __popc(v);
  }
  pc = sum_u64(pc);
  if (tid == 0) counts[r] = (int32_t)pc;
}

// Rows left by the screened cut: a persistent grid of kFallbackWGs workgroups, each
// with its own float64 scratch row (zscr: kFallbackWGs * L/4 doubles); the group
// means are formed from the 4 keys of each group (exact, as in the oracle).
template <typename T>
__global__ void __launch_bounds__(kNT) group_fallback_kernel(const double* __restrict__ qp, const T* __restrict__ k,
                                                             double* __restrict__ zscr, Geom g, double thr,
                                                             double lambda, int win_t, int win_h, int win_w,
                                                             uint32_t* __restrict__ bitmap,
                                                             int32_t* __restrict__ counts, int words,
                                                             const int32_t* __restrict__ flag_list,
                                                             const int32_t* __restrict__ nflag, double inv_sqrt_d) {
  __shared__ SelectSmem sm;
  __shared__ double qrow[128];
  const int SG = g.L / 4;
  double* zr = zscr + (size_t)blockIdx.x * SG;
  const int n = *nflag;
  for (int x = blockIdx.x; x < n; x += gridDim.x) {
    const int64_t r = flag_list[x];
    const int64_t bh = r / g.S;
    __syncthreads();                     // the previous row is done with qrow, zr and sm
    if ((int)threadIdx.x < g.D) qrow[threadIdx.x] = qp[(size_t)r * g.D + threadIdx.x];
    __syncthreads();
    double m = -DBL_MAX;
    for (int j = threadIdx.x; j < SG; j += kNT) {
      double z = 0.0;
      for (int c0 = 0; c0 < g.D; c0 += 8) {
        double mk[8];
        group_mean<T, 8>(k, g, bh, j, c0, mk);
#pragma unroll
        for (int e = 0; e < 8; ++e) z = fma(qrow[c0 + e], mk[e], z);
      }
      z *= inv_sqrt_d;
      zr[j] = z;
      m = fmax(m, z);
    }
    // (the row max's barriers make zr visible to the whole workgroup)
    select_row(zr, m, r, SG, g, thr, lambda, win_t, win_h, win_w, bitmap, counts, words, sm);
  }
}

}  // namespace gmask

hipError_t launch_group_fallback(const Geom& g, const double* qp, const void* k, double* zscr, double thr,
                                 double lambda, int win_t, int win_h, int win_w, uint32_t* bitmap, int32_t* counts,
                                 int words, const int32_t* flag_list, const int32_t* nflag, hipStream_t s) {
  const double inv = 1.0 / sqrt((double)g.D);
  if (g.dtype == 1)
    gmask::group_fallback_kernel<uint16_t><<<gmask::kFallbackWGs, gmask::kNT, 0, s>>>(
        qp, (const uint16_t*)k, zscr, g, thr, lambda, win_t, win_h, win_w, bitmap, counts, words, flag_list, nflag, inv);
  else
    gmask::group_fallback_kernel<float><<<gmask::kFallbackWGs, gmask::kNT, 0, s>>>(
        qp, (const float*)k, zscr, g, thr, lambda, win_t, win_h, win_w, bitmap, counts, words, flag_list, nflag, inv);
  return hipGetLastError();
}

int group_select_max_groups() { return gmask::kMaxSG; }

}  // namespace bsa
