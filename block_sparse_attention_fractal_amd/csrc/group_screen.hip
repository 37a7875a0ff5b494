// Screened key-group map and CDF cut (AB-Attention page, news.hamidun.com/es/news/14960,
// "Los tres recursos de AB-Attention", third resource: 4-token key/value blocks; the
// map and the cut are those of the NABLA page, gist.science/es/paper/2507.13546,
// Metodologia item 2, "Atencion Reducida" and "Umbralizacion CDF"; item 3 for the
// window union).
//
// A row of the group map has L/4 entries (31 680 at 33 x 48 x 80 tokens), 16 times
// the block map's, and one head's map is S x L/4; in float64 the GEMM alone needs
// about 10 ms of the float64 matrix-core peak at that size.  The block map's screen
// (mask_screen.hip) is taken over with the same identity
//
//   qp_i . kg_j = D mu_i nu_j + c_i . e_j      (mu, nu: channel means; c, e centred)
//
// the rank-one part in float64, the centred part on the fp16 matrix cores with both
// operands split into hi + lo (each vector scaled by a power of two into
// [2^13, 2^14)).  The products hi*hi of the first and of the second half of the
// channels and the cross products hi*lo + lo*hi go to three float32 accumulators:
// with at most 64 additions per accumulator (D = 128) the float32 sums are within
// 2^-17 of the sum of |products|, the split and the dropped lo*lo term add
// 3 * 2^-22, so every screened logit of row i is within
//   eps_i = 1.125 * 2^-17 |c_i| max_j |e_j| / sqrt(D)
// of the exact one (four times tighter than the single-accumulator bound of the
// block screen: the group means average 4 tokens instead of 64, so their centred
// norms are about 4 times larger).
//
//   * pool_groups_screen_kernel: float64 means of the 4 keys of every group (kept
//     for the exact recomputation) and their screen operands, in MFMA tile order;
//   * group_logits_screen_kernel: the screened map of a chunk of heads as float32
//     offsets z - ub_i (ub_i an upper bound of the row's largest logit), written
//     to HBM (4 bytes per entry instead of 8);
//   * group_screen_select_kernel: one 1024-thread workgroup per row, each thread
//     holding 32 consecutive entries in registers (so its bits are one bitmap
//     word).  The cut is the block screen's: masses in fixed point from the
//     screened offsets, a 24-bit key radix-selected 8 bits per pass with one
//     histogram per wavefront, the crossing bin widened by the error margin; the
//     entries above it are kept, those inside it (at most 64) are handed with the
//     mass above them to group_rank_kernel.  Rows whose margin the screen cannot
//     guarantee, or with more than 64 entries inside it, are listed for the exact
//     float64 path (group_mask.hip);
//   * group_rank_kernel: the handed-over entries get their exact float64 logits
//     and are ranked exactly, one wavefront per row with many rows in flight (so
//     the loads of the group means do not stall a whole workgroup).
#include <float.h>

#include <algorithm>

#include "kernels.h"
#include "mask_util.h"

namespace bsa {
namespace gscr {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr double kScreenErr = 0x1.2p-17;   // relative error of the screened centred dot product
constexpr float kTrust = 4e-5f;            // largest offset error (logit units) a screened row may carry
constexpr int kNT = 1024;                  // select: threads per row
constexpr int kNW = kNT / 64;
constexpr int kPer = 32;                   // entries per thread: 32768 groups per head at most
constexpr int kMaxCand = 64;               // exactly ranked entries per row
constexpr int kRowsWG = 128;               // map: query blocks per workgroup (32 per wave)
constexpr int kStep = 64;                  // map: key groups per LDS stage (4 tiles of 16)

// ---------------------------------------------------------------------------
// Group means and screen operands.  grid = (ceil(L/4 / (4 GPW)), B * heads),
// 256 threads; LPG lanes per group (a 16-byte chunk of each of its 4 token rows
// per lane), GPW groups per wave.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) pool_groups_screen_kernel(const T* __restrict__ k, double* __restrict__ kg,
                                                                 ScreenOps ops, Geom g) {
  constexpr int EPC = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int LPG = D / EPC;               // lanes per group
  constexpr int GPW = 64 / LPG;              // groups per wave
  __shared__ uint64_t red[3][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t bh = blockIdx.y;
  const int SG = g.L / 4, ntg = (SG + 15) / 16, gpb = g.N / 4;
  const int gid = (blockIdx.x * 4 + wave) * GPW + lane / LPG;
  const int c = lane % LPG;
  const bool ok = gid < SG;
  const int gq = min(gid, SG - 1);
  const int blk = gq / gpb, m0 = (gq % gpb) * 4;
  uint4 raw[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    raw[t] = *(const uint4*)(k + ((size_t)bh * g.L + block_token_row(g, blk, m0 + t)) * D + c * EPC);
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
#pragma unroll
  for (int t = 0; t < 4; ++t) add_chunk<T>(acc, raw[t]);
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] *= 0.25;          // sums of 4 inputs are exact in float64
  if (ok) {
    double2* dst = (double2*)(kg + ((size_t)bh * SG + gid) * D + c * EPC);
#pragma unroll
    for (int x = 0; x < EPC / 2; ++x) dst[x] = make_double2(acc[2 * x], acc[2 * x + 1]);
  }
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < EPC; ++e) s += acc[e];
  const double mu = group_reduce<LPG>(s, lane, [](double a, double b) { return a + b; }) * (1.0 / D);
  double amax = 0.0, n2 = 0.0;
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    acc[e] -= mu;
    amax = fmax(amax, fabs(acc[e]));
    n2 = fma(acc[e], acc[e], n2);
  }
  amax = group_reduce<LPG>(amax, lane, [](double a, double b) { return fmax(a, b); });
  n2 = group_reduce<LPG>(n2, lane, [](double a, double b) { return a + b; });
  const int ex = amax > 0.0 ? 13 - ilogb(amax) : 0;     // scaled magnitudes in [2^13, 2^14)
  if (ok) {
    _Float16 hv[EPC], lv[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      // double -> float -> fp16 on the hardware converts (the opaque copies keep the
      // compiler from fusing them into a software double -> fp16 rounding)
      const double x = ldexp(acc[e], ex);
      float xf = (float)x;
      asm volatile("" : "+v"(xf));
      const _Float16 hi = (_Float16)xf;
      float rf = (float)(x - (double)hi);
      asm volatile("" : "+v"(rf));
      hv[e] = hi;
      lv[e] = (_Float16)rf;
    }
    // 16-group tiles, per 32-channel step s and half (hi, lo) 1 KB holding, at lane
    // slot 16 (channel / 8 % 4) + group % 16, the 8 channels that lane of
    // v_mfma_f32_16x16x32_f16 takes
    const int ch0 = c * EPC, cc = ch0 >> 3, st = cc >> 2, kq = cc & 3;
    _Float16* dst = ops.ks + (((size_t)(bh * ntg + gid / 16) * (D / 32) + st) * 2) * 512 +
                    (16 * kq + (gid & 15)) * 8 + (ch0 & 7);
    if constexpr (EPC == 8) {
      *(uint4*)dst = *(const uint4*)hv;
      *(uint4*)(dst + 512) = *(const uint4*)lv;
    } else {
      *(uint2*)dst = *(const uint2*)hv;
      *(uint2*)(dst + 512) = *(const uint2*)lv;
    }
  }
  const double nrm = sqrt(n2) * (1.0 + 0x1p-50);          // rounded up: an upper bound of |e|
  if (ok && c == 0) ops.krec[(size_t)bh * SG + gid] = make_double2(mu, (double)ex);
  uint64_t st_max = ok ? order_key(mu) : 0ull, st_min = ok ? order_key(mu) : ~0ull, st_n = ok ? order_key(nrm) : 0ull;
  st_max = wave_reduce(st_max, lane, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
  st_min = wave_reduce(st_min, lane, [](uint64_t a, uint64_t b) { return a < b ? a : b; });
  st_n = wave_reduce(st_n, lane, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
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

// the row constants of the screen: a = D mu_i, the upper bound ub_i of the row's
// logits and the error bound eps_i (identical expressions in both kernels)
struct RowScreen {
  double a, ub, eps;
};
__device__ __forceinline__ RowScreen row_screen(const ScreenOps& ops, int64_t r, int64_t bh, int D, double inv_sqrt_d) {
  const double a = (double)D * ops.qmu[r];
  const double bmax = key_to_double(ops.hstat[3 * bh]), bmin = key_to_double(ops.hstat[3 * bh + 1]);
  const double cmax = key_to_double(ops.hstat[3 * bh + 2]);
  const double nq = ops.qn[r];
  RowScreen rs;
  rs.a = a;
  rs.ub = (a * (a >= 0.0 ? bmax : bmin) + nq * cmax) * inv_sqrt_d;
  rs.eps = kScreenErr * nq * cmax * inv_sqrt_d;
  return rs;
}

// ---------------------------------------------------------------------------
// Screened map of heads h0 .. h0 + gridDim.z - 1: zt[(h - h0) S + i][j] =
// float(z~_ij - ub_i), row pitch `pitch` floats.  grid = (column slices,
// ceil(S / 128), heads), 256 threads.  Wave w holds the A operands (hi, lo) of
// query blocks i0 + 32 w .. + 31 in registers; the workgroup streams its slice
// of key groups through LDS 64 at a time (the next stage's 16-byte chunks in
// registers while the current one is multiplied).  MFMA layouts as in
// mask_screen.hip: A[i][k] in lane 16 (k / 8) + i, B[k][j] in lane 16 (k / 8) + j,
// C[i][j] in lane 16 (i / 4) + j, register i % 4.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256, 2) group_logits_screen_kernel(ScreenOps ops, float* __restrict__ zt, Geom g,
                                                                     int64_t h0, int steps_per_slice, int pitch,
                                                                     double inv_sqrt_d) {
  constexpr int KS = D / 32;                 // k-steps of 32 channels
  constexpr int kTileH = KS * 1024;          // halfs per 16-group tile (hi and lo)
  constexpr int kChunks = 4 * kTileH * 2 / (256 * 16);   // 16-byte chunks per thread per stage
  static_assert(kChunks * 256 * 16 == 4 * kTileH * 2, "stage shape");
  __shared__ __attribute__((aligned(16))) _Float16 bs[4 * kTileH];
  __shared__ double2 recs[kStep];            // (nu_j, exponent) of the stage's groups
  __shared__ double rc_a[kRowsWG], rc_ub[kRowsWG];
  __shared__ int rc_e[kRowsWG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = g.S, SG = g.L / 4, ntg = (SG + 15) / 16;
  const int64_t bh = h0 + blockIdx.z;
  const int i0 = blockIdx.y * kRowsWG;
  const int64_t rbase = bh * S;
  if (tid < kRowsWG) {
    const int i = i0 + tid;
    if (i < S) {
      const RowScreen rs = row_screen(ops, rbase + i, bh, D, inv_sqrt_d);
      rc_a[tid] = rs.a;
      rc_ub[tid] = rs.ub;
      rc_e[tid] = ops.qe[rbase + i];
    } else {
      rc_a[tid] = 0.0;
      rc_ub[tid] = 0.0;
      rc_e[tid] = 0;
    }
  }
  f16x8 ah[2][KS], al[2][KS];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int ia = min(i0 + 32 * wave + 16 * rt + (lane & 15), S - 1);
    const _Float16* src = ops.qs + (size_t)(rbase + ia) * 2 * D + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      ah[rt][s] = *(const f16x8*)(src + 32 * s);
      al[rt][s] = *(const f16x8*)(src + D + 32 * s);
    }
  }
  const int nsteps = (SG + kStep - 1) / kStep;
  const int st0 = blockIdx.x * steps_per_slice, st1 = min(st0 + steps_per_slice, nsteps);
  const _Float16* kh = ops.ks + (size_t)bh * ntg * kTileH;
  u32x4 stg[kChunks];
  double2 srec;
  auto fetch = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < kChunks; ++x) {
      const int idx = x * 256 + tid;                       // 16-byte chunk of the stage
      const int tin = idx / (kTileH / 8), off = idx % (kTileH / 8);
      const int t = min(4 * st + tin, ntg - 1);            // past the end: the last tile (unused)
      stg[x] = *(const u32x4*)(kh + (size_t)t * kTileH + off * 8);
    }
    if (tid < kStep) srec = ops.krec[(size_t)bh * SG + min(st * kStep + tid, SG - 1)];
  };
  if (st0 < st1) fetch(st0);
  __syncthreads();                                         // the row constants
  double ra[2][4], rub[2][4];
  int re[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int rho = 32 * wave + 16 * rt + 4 * (lane >> 4) + x;
      ra[rt][x] = rc_a[rho];
      rub[rt][x] = rc_ub[rho];
      re[rt][x] = rc_e[rho];
    }
  float* zh = zt + (size_t)blockIdx.z * S * (size_t)pitch;
  const int jl = lane & 15;
  for (int st = st0; st < st1; ++st) {
#pragma unroll
    for (int x = 0; x < kChunks; ++x) *(u32x4*)(bs + (x * 256 + tid) * 8) = stg[x];
    if (tid < kStep) recs[tid] = srec;
    __syncthreads();
    if (st + 1 < st1) fetch(st + 1);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j0 = (4 * st + u) * 16;
      if (j0 >= SG) break;
      const int j = j0 + jl;
      const double2 rec = recs[16 * u + jl];
      f16x8 bhi[KS], blo[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bhi[s] = *(const f16x8*)(bs + u * kTileH + s * 1024 + 8 * lane);
        blo[s] = *(const f16x8*)(bs + u * kTileH + s * 1024 + 512 + 8 * lane);
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0, px = p0;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (s < KS / 2)
            p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt][s], bhi[s], p0, 0, 0, 0);
          else
            p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt][s], bhi[s], p1, 0, 0, 0);
          px = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt][s], blo[s], px, 0, 0, 0);
          px = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[rt][s], bhi[s], px, 0, 0, 0);
        }
        if (j < SG) {
          const int ek = (int)rec.y;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int i = i0 + 32 * wave + 16 * rt + 4 * (lane >> 4) + x;
            if (i < S) {
              const double dot = ((double)p0[x] + (double)p1[x]) + (double)px[x];
              const double z = fma(ra[rt][x], rec.x, ldexp(dot, -(re[rt][x] + ek)));
              zh[(size_t)i * pitch + j] = (float)fma(z, inv_sqrt_d, -rub[rt][x]);
            }
          }
        }
      }
    }
    __syncthreads();                                       // the stage is consumed
  }
}

// ---------------------------------------------------------------------------
// The cut of rows row0 .. row0 + gridDim.x - 1 (zt: those rows, pitch floats
// apart).  Thread t holds entries 32 t .. 32 t + 31 of the row.
// ---------------------------------------------------------------------------
struct SelSmem {
  uint64_t hist[kNW][256];            // per wave: (count << 44) | mass, top bin first
  uint32_t bm[kNT];                   // the row's bitmap words
  uint32_t cj[kMaxCand], cw[kMaxCand];   // entries inside the margin: index, mass
  uint64_t red_u[kNW];
  float red_f[kNW];
  uint64_t scan[4];
  uint64_t found_above;
  int found_bin;
  uint32_t found_cnt, ncand;
};

__global__ void __launch_bounds__(kNT) group_screen_select_kernel(
    const float* __restrict__ zt, int pitch, ScreenOps ops, const double* __restrict__ qp,
    const double* __restrict__ kg, int64_t row0, Geom g, double thr, double lambda, int win_t, int win_h, int win_w,
    uint32_t* __restrict__ bitmap, int32_t* __restrict__ counts, int words, int32_t* __restrict__ flag_list,
    int32_t* __restrict__ nflag, int32_t* __restrict__ cn, double2* __restrict__ cab, uint2* __restrict__ cjw,
    double inv_sqrt_d) {
  __shared__ SelSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int SG = g.L / 4, gpb = g.N / 4;
  const int64_t r = row0 + blockIdx.x;
  const int64_t bh = r / g.S;
  const int i = (int)(r - bh * g.S);
  const int jb = kPer * tid;                               // this thread's first entry
  int nv = SG - jb;
  asm volatile("" : "+v"(nv));   // opaque: no per-entry lane masks hoisted and kept live
  constexpr uint64_t kMassMask = (1ull << 44) - 1;
  auto u64add = [](uint64_t a, uint64_t b) { return a + b; };
  auto bsum = [&](uint64_t v) {
    v = wave_reduce(v, lane, u64add);
    if (lane == 0) sm.red_u[wv] = v;
    __syncthreads();
    uint64_t t = 0;
    for (int x = 0; x < kNW; ++x) t += sm.red_u[x];
    __syncthreads();
    return t;
  };
  auto bmin_f = [&](float v) {
    v = wave_reduce(v, lane, [](float a, float b) { return fminf(a, b); });
    if (lane == 0) sm.red_f[wv] = v;
    __syncthreads();
    float t = sm.red_f[0];
    for (int x = 1; x < kNW; ++x) t = fminf(t, sm.red_f[x]);
    __syncthreads();
    return t;
  };
  auto bmax_f = [&](float v) {
    v = wave_reduce(v, lane, [](float a, float b) { return fmaxf(a, b); });
    if (lane == 0) sm.red_f[wv] = v;
    __syncthreads();
    float t = sm.red_f[0];
    for (int x = 1; x < kNW; ++x) t = fmaxf(t, sm.red_f[x]);
    __syncthreads();
    return t;
  };

  uint32_t bits = 0;                                       // bit k: entry jb + k is kept
  uint32_t nrank = 0;                                      // entries left to group_rank_kernel
  if (thr == 0.0) {
    bits = nv >= 32 ? 0xffffffffu : (nv > 0 ? (1u << nv) - 1u : 0u);
  } else {
    float v[kPer];
    if (nv > 0) {
      const float4* src = (const float4*)(zt + (size_t)blockIdx.x * pitch + jb);   // pitch: a multiple of 32
#pragma unroll
      for (int m = 0; m < kPer / 4; ++m) {
        const float4 x = src[m];
        v[4 * m] = x.x;
        v[4 * m + 1] = x.y;
        v[4 * m + 2] = x.z;
        v[4 * m + 3] = x.w;
      }
    }
    float mt = -FLT_MAX;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      v[k] = k < nv ? v[k] : -FLT_MAX;
      mt = fmaxf(mt, v[k]);
    }
    if (tid == 0) sm.ncand = 0u;
    mt = bmax_f(mt);
    // error of the offsets d = v - mt against the exact z - max: the screen (twice)
    // plus the float32 roundings of v and of d (|d| <= 30 ln 2 for an entry with mass)
    const double eps_i = row_screen(ops, r, bh, g.D, inv_sqrt_d).eps;
    const float eps_d = (float)(2.0 * eps_i) + 0x1p-23f * (fabsf(mt) + 22.f);
    if (!(eps_d <= kTrust)) {                              // uniform: the float64 path owns this row
      if (tid == 0) {
        flag_list[atomicAdd(nflag, 1)] = (int32_t)r;
        cn[r] = 0;
      }
      return;
    }
    uint32_t w[kPer], t[kPer];
    uint64_t wsum = 0;
    float dmin = 0.f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const float d = v[k] - mt;
      const float e = d >= (float)-lambda ? __builtin_amdgcn_exp2f(d * 1.44269504088896341f) : 0.f;
      w[k] = (uint32_t)(e * 1073741824.0f);                // e <= 1: at most 2^30, exact
      wsum += w[k];
      dmin = fminf(dmin, w[k] != 0u ? d : 0.f);
      v[k] = d;
    }
    const uint64_t total = bsum(wsum);
    dmin = bmin_f(dmin);
    const float tscale = dmin < 0.f ? 16777215.0f / (-dmin) : 0.f;
    // entries without mass get key 2^31: no radix prefix matches it, it is negative
    // as an int and above every margin unsigned
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      t[k] = w[k] != 0u ? (uint32_t)fminf((v[k] - dmin) * tscale, 16777215.0f) : 0x80000000u;
    const double target = (1.0 - thr) * (double)total;     // keep while the mass before < target

    // one radix pass: (count, mass) histogram of bin(k) >= 0 per wave, summed over
    // the waves by threads 0..255 (thread x: bin 255 - x), a prefix over the bins
    // from the top, and the bin in which the mass reaches the target
    auto crossing = [&](auto bin, uint64_t above_in, int& b_out, uint64_t& above_out, uint32_t& cnt_out)
                        __attribute__((always_inline)) {
      uint64_t* hw = sm.hist[wv];
      *(uint4*)(hw + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
      *(uint4*)(hw + 4 * lane + 2) = make_uint4(0u, 0u, 0u, 0u);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int b = bin(k);
        uint32_t wk = w[k];
        asm volatile("" : "+v"(wk));   // opaque: no 64-bit copies of the masses kept live across passes
        if (b >= 0) atomicAdd((unsigned long long*)&hw[255 - b], (1ull << 44) | (unsigned long long)wk);
      }
      __syncthreads();
      uint64_t mb = 0;
      uint32_t cb = 0;
      if (tid < 256) {
#pragma unroll
        for (int x = 0; x < kNW; ++x) {
          const uint64_t h = sm.hist[x][tid];
          mb += h & kMassMask;
          cb += (uint32_t)(h >> 44);
        }
      }
      uint64_t incl = wave_prefix_u64(mb, lane);
      if (tid == 0) sm.found_bin = -1;
      if (wv < 4 && lane == 63) sm.scan[wv] = incl;
      __syncthreads();
      if (tid < 256) {
        for (int x = 0; x < wv; ++x) incl += sm.scan[x];
        const uint64_t excl = incl - mb;
        if (cb != 0u && (double)(above_in + excl) < target && target <= (double)(above_in + incl)) {
          sm.found_bin = 255 - tid;
          sm.found_above = above_in + excl;
          sm.found_cnt = cb;
        }
      }
      __syncthreads();
      b_out = sm.found_bin;
      above_out = sm.found_above;
      cnt_out = sm.found_cnt;
      return b_out >= 0;
    };
    uint32_t tpre = 0;
    int tsh = 24;
    uint64_t above = 0;
    uint32_t cnt = 0;
    bool reach = true;
    while (tsh > 0) {
      const int sh = tsh - 8;
      const uint32_t pf = tpre;
      const int tshc = tsh;
      int b;
      uint64_t ab;
      uint32_t cb;
      if (!crossing([&](int k) { return (t[k] >> tshc) == pf ? (int)((t[k] >> sh) & 255u) : -1; }, above, b, ab,
                    cb)) {
        reach = false;                                     // only possible on the first pass
        break;
      }
      tpre = (pf << 8) | (uint32_t)b;
      tsh = sh;
      above = ab;
      cnt = cb;
      if (cnt <= 48u) break;
    }
    if (!reach) {
#pragma unroll
      for (int k = 0; k < kPer; ++k)
        if ((int)t[k] >= 0) bits |= 1u << k;
    } else {
      // the crossing bin widened by the error margin in key units; entries above it
      // are kept, those inside it ranked exactly, those below dropped
      const uint32_t mt_keys = (uint32_t)fminf(ceilf(2.f * eps_d * tscale), 16777215.0f) + 1u;
      const uint32_t lo_t = tpre << tsh, hi_t = lo_t + ((1u << tsh) - 1u);
      const uint32_t lo_m = lo_t > mt_keys ? lo_t - mt_keys : 0u;
      const uint32_t hi_m = hi_t + mt_keys;                // < 2^25: no wrap
      uint64_t sure = 0;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        if ((int)t[k] > (int)hi_m) {
          bits |= 1u << k;
          sure += w[k];
        } else if (t[k] >= lo_m && t[k] <= hi_m) {
          const uint32_t slot = atomicAdd(&sm.ncand, 1u);
          if (slot < (uint32_t)kMaxCand) {
            sm.cj[slot] = (uint32_t)(jb + k);
            sm.cw[slot] = w[k];
          }
        }
      }
      above = bsum(sure);                                  // (its barriers also publish the candidates)
      const uint32_t ncand = sm.ncand;
      if (ncand > (uint32_t)kMaxCand) {                    // uniform: the float64 path owns this row
        if (tid == 0) {
          flag_list[atomicAdd(nflag, 1)] = (int32_t)r;
          cn[r] = 0;
        }
        return;
      }
      // the entries inside the margin go to group_rank_kernel with the mass above
      // them and the target
      if ((uint32_t)tid < ncand) cjw[r * kMaxCand + tid] = make_uint2(sm.cj[tid], sm.cw[tid]);
      if (tid == 0) cab[r] = make_double2((double)above, target);
      nrank = ncand;
    }
  }
  // the bitmap row: this thread's word, then the window on top (every group of
  // every window block)
  if (tid == 0) cn[r] = (int32_t)nrank;
  sm.bm[tid] = bits;
  __syncthreads();
  if (win_t >= 0) {
    const int HW = g.Hp * g.Wp;
    for_each_window_run(g, i / HW, (i / g.Wp) % g.Hp, i % g.Wp, win_t, win_h, win_w, tid, kNT, [&](int a, int b) {
      const int ga = a * gpb, gb = (b + 1) * gpb - 1;
      for (int wd = ga >> 5; wd <= (gb >> 5); ++wd) {
        const int lo = max(ga - 32 * wd, 0), hi = min(gb - 32 * wd, 31);
        const uint32_t m = hi - lo == 31 ? 0xffffffffu : ((1u << (hi - lo + 1)) - 1u) << lo;
        atomicOr(&sm.bm[wd], m);
      }
    });
  }
  __syncthreads();
  uint64_t pc = 0;
  if (tid < words) {
    const uint32_t x = sm.bm[tid];
    bitmap[r * words + tid] = x;
    pc = (uint64_t)__popc(x);
  }
  pc = bsum(pc);
  if (tid == 0) counts[r] = (int32_t)pc;
}

// The entries a screened cut left inside its margin, ranked on their exact float64
// logits (logit descending, index ascending): one wavefront per row, eight lanes per
// entry (each D / 8 channels), eight entries per pass; the kept ones are added to
// the row's bits and count.
__global__ void __launch_bounds__(256) group_rank_kernel(const int32_t* __restrict__ cn, const double2* __restrict__ cab,
                                                         const uint2* __restrict__ cjw, const double* __restrict__ qp,
                                                         const double* __restrict__ kg, Geom g, int64_t rows,
                                                         uint32_t* __restrict__ bitmap, int32_t* __restrict__ counts,
                                                         int words, double inv_sqrt_d) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;                                   // whole wavefronts
  const uint32_t ncand = (uint32_t)cn[r];
  if (ncand == 0u) return;
  const int SG = g.L / 4, D = g.D, per = D / 8;
  const int64_t bh = r / g.S;
  const int sub = lane & 7, slot = lane >> 3;
  const bool have = (uint32_t)lane < ncand;
  const uint2 mine_jw = cjw[r * kMaxCand + min((uint32_t)lane, ncand - 1u)];
  const double* qrow = qp + (size_t)r * D + sub * per;
  double z = 0.0;
  for (int p = 0; p < (int)((ncand + 7u) / 8u); ++p) {
    const uint32_t cidx = min(8u * (uint32_t)p + (uint32_t)slot, ncand - 1u);
    const uint32_t cj = (uint32_t)__shfl((int)mine_jw.x, (int)cidx, 64);
    const double* krow = kg + ((size_t)bh * SG + cj) * D + sub * per;
    double part = 0.0;
    for (int e = 0; e < per; e += 2) {
      const double2 qv = *(const double2*)(qrow + e), kv = *(const double2*)(krow + e);
      part = fma(qv.x, kv.x, part);
      part = fma(qv.y, kv.y, part);
    }
    part = sum8(part);
    const double got = __shfl(part, 8 * (lane & 7), 64);   // entry 8 p + lane % 8 -> lane
    if ((lane >> 3) == p) z = got;
  }
  const uint32_t my_j = mine_jw.x, my_w = have ? mine_jw.y : 0u;
  const uint64_t my_key = have ? order_key(z * inv_sqrt_d) : 0ull;   // as the float64 path scales
  uint64_t before = 0;
  for (uint32_t y = 0; y < ncand; ++y) {
    const uint64_t ky = readlane_u64(my_key, (int)y);
    const uint32_t jy = (uint32_t)__builtin_amdgcn_readlane((int)my_j, (int)y);
    const uint32_t wy = (uint32_t)__builtin_amdgcn_readlane((int)my_w, (int)y);
    if (ky > my_key || (ky == my_key && jy < my_j)) before += wy;
  }
  const double2 at = cab[r];                               // (mass above the margin, target)
  if (have && at.x + (double)before < at.y) {
    const uint32_t bit = 1u << (my_j & 31);
    const uint32_t old = atomicOr(&bitmap[r * words + (my_j >> 5)], bit);
    if (!(old & bit)) atomicAdd(&counts[r], 1);            // not already kept by the window
  }
}

}  // namespace gscr

hipError_t launch_pool_groups_screen(const Geom& g, const void* k, double* kg, const ScreenOps& ops, hipStream_t s) {
  const int SG = g.L / 4;
  const unsigned heads = (unsigned)((int64_t)g.B * g.nh);
#define BSA_PGS(T_, D_)                                                                                   \
  do {                                                                                                    \
    constexpr int gpw = 64 / (D_ / (16 / (int)sizeof(T_)));                                               \
    gscr::pool_groups_screen_kernel<T_, D_><<<dim3((unsigned)((SG + 4 * gpw - 1) / (4 * gpw)), heads), 256, 0, \
                                              s>>>((const T_*)k, kg, ops, g);                              \
  } while (0)
  if (g.dtype == 1 && g.D == 64) BSA_PGS(uint16_t, 64);
  else if (g.dtype == 1) BSA_PGS(uint16_t, 128);
  else if (g.D == 64) BSA_PGS(float, 64);
  else BSA_PGS(float, 128);
#undef BSA_PGS
  return hipGetLastError();
}

hipError_t launch_group_logits_screen(const Geom& g, const ScreenOps& ops, float* zt, int64_t h0, int64_t nheads,
                                      int pitch, hipStream_t s) {
  const int SG = g.L / 4;
  const int nsteps = (SG + gscr::kStep - 1) / gscr::kStep;
  const int64_t rowblocks = (g.S + gscr::kRowsWG - 1) / gscr::kRowsWG;
  // about 2048 workgroups per launch (8 per CU), every slice a whole number of stages
  const int64_t want = std::max<int64_t>(1, (2048 + rowblocks * nheads - 1) / (rowblocks * nheads));
  const int slices = (int)std::min<int64_t>(want, nsteps);
  const int per = (nsteps + slices - 1) / slices;
  dim3 grid((unsigned)((nsteps + per - 1) / per), (unsigned)rowblocks, (unsigned)nheads);
  const double inv = 1.0 / sqrt((double)g.D);
  if (g.D == 64)
    gscr::group_logits_screen_kernel<64><<<grid, 256, 0, s>>>(ops, zt, g, h0, per, pitch, inv);
  else
    gscr::group_logits_screen_kernel<128><<<grid, 256, 0, s>>>(ops, zt, g, h0, per, pitch, inv);
  return hipGetLastError();
}

hipError_t launch_group_screen_select(const Geom& g, const float* zt, int pitch, const ScreenOps& ops,
                                      const double* qp, const double* kg, int64_t row0, int64_t nrows, double thr,
                                      double lambda, int win_t, int win_h, int win_w, uint32_t* bitmap,
                                      int32_t* counts, int words, int32_t* flag_list, int32_t* nflag,
                                      const GroupRankBufs& rb, hipStream_t s) {
  const double inv = 1.0 / sqrt((double)g.D);
  gscr::group_screen_select_kernel<<<(unsigned)nrows, gscr::kNT, 0, s>>>(zt, pitch, ops, qp, kg, row0, g, thr, lambda,
                                                                         win_t, win_h, win_w, bitmap, counts, words,
                                                                         flag_list, nflag, rb.cn, rb.cab, rb.cjw, inv);
  return hipGetLastError();
}

hipError_t launch_group_rank(const Geom& g, const GroupRankBufs& rb, const double* qp, const double* kg,
                             uint32_t* bitmap, int32_t* counts, int words, hipStream_t s) {
  const double inv = 1.0 / sqrt((double)g.D);
  gscr::group_rank_kernel<<<(unsigned)((g.rows + 3) / 4), 256, 0, s>>>(rb.cn, rb.cab, rb.cjw, qp, kg, g, g.rows, bitmap,
                                                                       counts, words, inv);
  return hipGetLastError();
}

}  // namespace bsa
