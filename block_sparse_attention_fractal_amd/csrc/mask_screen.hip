// Reduced map and CDF cut without materialising the map (NABLA page,
// gist.science/es/paper/2507.13546, Metodologia item 2, bullets "Atencion
// Reducida" and "Umbralizacion CDF", and item 3, the sliding-tile window).
//
// The cut needs the ORDER of the float64 block logits z_ij = qp_i . kp_j / sqrt(D)
// near the cut, and masses accurate well inside the 1e-4 band.  Instead of a
// float64 GEMM written to HBM, each workgroup screens the logits of 16 query
// blocks against all key blocks of their head on the fp16 matrix cores and keeps
// them in LDS:
//
//   qp_i . kp_j = D mu_i nu_j + c_i . e_j      (mu, nu: channel means; c, e: the
//                                               centred vectors, sum_d c = sum_d e = 0)
//
// The rank-one part is evaluated in float64; the centred part, which no longer
// carries a component common to all channels (the positional term of video
// latents), goes through the MFMA as c = c_hi + c_lo in fp16 (each vector scaled
// by a power of two into [2^13, 2^14)), three products per k-step accumulated in
// float32.  Its error is at most 2^-15 |c_i| |e_j| (split error 3 * 2^-22 plus
// 384 float32 additions), so every screened logit of row i is within
//   eps_i = 2^-15 |c_i| max_j |e_j| / sqrt(D)
// of the exact one.  Rows whose eps (plus the float32 rounding of the stored
// offsets) would move a mass by more than the band allows are handed to an exact
// float64 path (fallback_select_kernel); the others are cut here:
//   * the per-row selection of select_kernel (fixed-point masses, a 24-bit
//     monotone key radix-selected 8 bits per pass) runs on the screened offsets;
//   * the blocks whose key lies within the error margin of the crossing bin
//     (2 eps in logit units on either side) get their exact float64 logit
//     qp_i . kp_j, and are ranked exactly (logit descending, block id ascending);
//     the blocks above the margin are kept, those below dropped;
//   * more than 64 such blocks (logits equal to within ~eps) also go to the exact
//     path.
#include <float.h>

#include "kernels.h"
#include "mask_util.h"

namespace bsa {
namespace scr {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxS = 4096;
constexpr double kScreenErr = 0x1p-15;   // relative error of the screened centred dot product
constexpr float kTrust = 4e-5f;          // largest offset error (logit units) a screened row may carry

__device__ __forceinline__ double key_to_double(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)b);
}

// ---------------------------------------------------------------------------
// Screen operands of the pooled blocks: channel mean, power-of-two scale
// exponent, fp16 hi / lo of the scaled centred vector and (query blocks) its
// norm; per head the max / min key-block mean and the largest key-block norm
// (order-preserving 64-bit keys, one atomic per workgroup and statistic).
// grid = (ceil(S / 32), B * heads, 2): z = 0 query blocks, z = 1 key blocks;
// each wave takes 8 consecutive blocks of one head, one block per step.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_fp16(double x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)(float)x;
  lo = (_Float16)(float)(x - (double)hi);
}

template <int D>
__global__ void __launch_bounds__(256) screen_ops_kernel(const double* __restrict__ qp, const double* __restrict__ kp,
                                                         ScreenOps ops, Geom g) {
  constexpr int PL = D / 64;             // channels per lane
  __shared__ uint64_t red[3][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t bh = blockIdx.y;
  const bool keys = blockIdx.z == 1;
  const double* src = keys ? kp : qp;
  uint64_t kmax = 0ull, kmin = ~0ull, nmax = 0ull;   // head statistics of this wave's key blocks
  for (int b = 0; b < 8; ++b) {
    const int i = (blockIdx.x * 4 + wave) * 8 + b;
    if (i >= g.S) break;
    const int64_t r = bh * g.S + i;
    double v[PL];
#pragma unroll
    for (int x = 0; x < PL; ++x) v[x] = src[(size_t)r * D + lane + 64 * x];
    double sum = 0.0;
#pragma unroll
    for (int x = 0; x < PL; ++x) sum += v[x];
    const double mu = wave_reduce(sum, lane, [](double a, double c) { return a + c; }) * (1.0 / D);
    double amax = 0.0, n2 = 0.0;
#pragma unroll
    for (int x = 0; x < PL; ++x) {
      v[x] -= mu;
      amax = fmax(amax, fabs(v[x]));
      n2 = fma(v[x], v[x], n2);
    }
    amax = wave_reduce(amax, lane, [](double a, double c) { return fmax(a, c); });
    n2 = wave_reduce(n2, lane, [](double a, double c) { return a + c; });
    const int ex = amax > 0.0 ? 13 - ilogb(amax) : 0;   // scaled magnitudes in [2^13, 2^14)
    _Float16* dst = (keys ? ops.ks : ops.qs) + (size_t)r * 2 * D;
#pragma unroll
    for (int x = 0; x < PL; ++x) {
      _Float16 hi, lo;
      split_fp16(ldexp(v[x], ex), hi, lo);
      dst[lane + 64 * x] = hi;
      dst[D + lane + 64 * x] = lo;
    }
    const double nrm = sqrt(n2) * (1.0 + 0x1p-50);    // rounded up: an upper bound of |c|
    if (lane == 0) {
      if (keys) {
        ops.kmu[r] = mu;
        ops.ke[r] = ex;
      } else {
        ops.qmu[r] = mu;
        ops.qe[r] = ex;
        ops.qn[r] = nrm;
      }
    }
    const uint64_t km = order_key(mu);
    kmax = km > kmax ? km : kmax;
    kmin = km < kmin ? km : kmin;
    const uint64_t kn = order_key(nrm);
    nmax = kn > nmax ? kn : nmax;
  }
  if (!keys) return;                     // whole workgroup: z is uniform
  if (lane == 0) {
    red[0][wave] = kmax;
    red[1][wave] = kmin;
    red[2][wave] = nmax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t a = red[0][0], b = red[1][0], c = red[2][0];
    for (int w = 1; w < 4; ++w) {
      a = red[0][w] > a ? red[0][w] : a;
      b = red[1][w] < b ? red[1][w] : b;
      c = red[2][w] > c ? red[2][w] : c;
    }
    unsigned long long* hs = (unsigned long long*)(ops.hstat + 3 * bh);
    atomicMax(&hs[0], (unsigned long long)a);
    atomicMin(&hs[1], (unsigned long long)b);
    atomicMax(&hs[2], (unsigned long long)c);
  }
}

__global__ void __launch_bounds__(256) hstat_init_kernel(uint64_t* __restrict__ hstat, int32_t* __restrict__ nflag,
                                                        int64_t heads) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x < heads) {
    hstat[3 * x] = 0ull;                 // max of mu: below every key
    hstat[3 * x + 1] = ~0ull;            // min of mu: above every key
    hstat[3 * x + 2] = 0ull;             // max norm
  }
  if (x == 0) *nflag = 0;
}

// ---------------------------------------------------------------------------
// Screened map + cut.  grid = (ceil(S / ROWS), B * heads), 512 threads (8 waves,
// two per SIMD): the GEMM of the workgroup's ROWS query blocks against the S key
// blocks (16 x 16 tiles of v_mfma_f32_16x16x32_f16; A[i][k] in lane 16 (k / 8) + i,
// register k % 8, B[k][j] likewise with j, C[i][j] in lane 16 (i / 4) + j,
// register i % 4; wave w takes tiles w, w + 8, ...) writes the offsets
// zt_ij = z_ij - ub_i (float32, ub_i an upper bound of the row's largest logit,
// so the offsets of the heavy blocks are small numbers) to LDS; then each wave
// cuts its rows (ROWS / 8 of them).
// ---------------------------------------------------------------------------
constexpr int kWaves = 8;

template <int D, int NS, int ROWS>
__global__ void __launch_bounds__(512, 1) screen_select_kernel(ScreenOps ops, const double* __restrict__ qp,
                                                               const double* __restrict__ kp, Geom g, double thr,
                                                               double lambda, int win_t, int win_h, int win_w,
                                                               uint32_t* __restrict__ bitmap,
                                                               int32_t* __restrict__ counts, int words,
                                                               int32_t* __restrict__ flag_list,
                                                               int32_t* __restrict__ nflag, double inv_sqrt_d) {
  constexpr int SP = 64 * NS + 4;        // row pitch of the offsets (floats)
  __shared__ float vals[ROWS][SP];
  __shared__ uint64_t hist_all[kWaves][256];    // per bin: count << 44 | mass (2^-30 units)
  __shared__ uint32_t cand_all[kWaves][128];    // crossing candidates: block ids, then masses
  __shared__ uint32_t bm_all[kWaves][kMaxS / 32];
  __shared__ double rc_a[ROWS], rc_ub[ROWS], rc_eps[ROWS];
  __shared__ int rc_e[ROWS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = g.S;
  const int64_t bh = blockIdx.y;
  const int i0 = blockIdx.x * ROWS;
  const int64_t rbase = bh * S;          // CSR row of query block 0 of this head (also its key block 0)

  // per-row constants: a = D mu_i, ub_i, eps_i, scale exponent
  if (tid < ROWS) {
    const int i = i0 + tid;
    if (i < S) {
      const int64_t r = rbase + i;
      const double a = (double)D * ops.qmu[r];
      const double bmax = key_to_double(ops.hstat[3 * bh]), bmin = key_to_double(ops.hstat[3 * bh + 1]);
      const double cmax = key_to_double(ops.hstat[3 * bh + 2]);
      const double nq = ops.qn[r];
      rc_a[tid] = a;
      rc_ub[tid] = (a * (a >= 0.0 ? bmax : bmin) + nq * cmax) * inv_sqrt_d;
      rc_eps[tid] = kScreenErr * nq * cmax * inv_sqrt_d;
      rc_e[tid] = ops.qe[r];
    }
  }

  if (thr != 0.0) {
    // A operand: query block (i0 + lane % 16), channels 8 (lane / 16) + 32 s .. + 7, hi and lo
    f16x8 qa_hi[D / 32], qa_lo[D / 32];
    {
      const int ia = lane & 15;
      const bool ok = ia < ROWS && i0 + ia < S;
      const _Float16* src = ops.qs + (size_t)(rbase + min(i0 + ia, S - 1)) * 2 * D + 8 * (lane >> 4);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        qa_hi[s] = ok ? *(const f16x8*)(src + 32 * s) : (f16x8){};
        qa_lo[s] = ok ? *(const f16x8*)(src + D + 32 * s) : (f16x8){};
      }
    }
    __syncthreads();                     // the row constants
    double ra[4], rub[4];
    int re[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int rho = 4 * (lane >> 4) + x;
      const bool ok = rho < ROWS && i0 + rho < S;
      ra[x] = ok ? rc_a[rho] : 0.0;
      rub[x] = ok ? rc_ub[rho] : 0.0;
      re[x] = ok ? rc_e[rho] : 0;
    }
    const int ntile = (S + 15) / 16;
    const int jl = lane & 15;
    auto load_b = [&](int c, f16x8* bhi, f16x8* blo) {
      const int j = min(16 * c + jl, S - 1);
      const _Float16* src = ops.ks + (size_t)(rbase + j) * 2 * D + 8 * (lane >> 4);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        bhi[s] = *(const f16x8*)(src + 32 * s);
        blo[s] = *(const f16x8*)(src + D + 32 * s);
      }
    };
    f16x8 bh0[D / 32], bl0[D / 32];
    int c = wave;
    if (c < ntile) load_b(c, bh0, bl0);
    for (; c < ntile; c += kWaves) {
      f16x8 bh1[D / 32], bl1[D / 32];
      const bool more = c + kWaves < ntile;
      if (more) load_b(c + kWaves, bh1, bl1);
      const int j = 16 * c + jl;
      const int jc = min(j, S - 1);
      const double nu = ops.kmu[rbase + jc];
      const int ek = ops.ke[rbase + jc];
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[s], bh0[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[s], bl0[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[s], bh0[s], acc, 0, 0, 0);
      }
      if (j < S) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int rho = 4 * (lane >> 4) + x;
          if (rho < ROWS) {
            const double z = fma(ra[x], nu, ldexp((double)acc[x], -(re[x] + ek)));
            vals[rho][j] = (float)fma(z, inv_sqrt_d, -rub[x]);
          }
        }
      }
      if (more) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          bh0[s] = bh1[s];
          bl0[s] = bl1[s];
        }
      }
    }
  }
  __syncthreads();

  // ---- the cut, one wavefront per row --------------------------------------
  uint64_t* hist = hist_all[wave];
  uint32_t* cand = cand_all[wave];
  uint32_t* bm = bm_all[wave];
  auto u64add = [](uint64_t a, uint64_t b) { return a + b; };
  constexpr uint64_t kMassMask = (1ull << 44) - 1;
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  auto set_bit = [&](int j) { atomicOr(&bm[j >> 5], 1u << (j & 31)); };
  for (int rho = wave; rho < ROWS; rho += kWaves) {
    const int i = i0 + rho;
    if (i >= S) break;
    const int64_t r = rbase + i;
    bool flagged = false;
    if (thr == 0.0) {
      for (int x = lane; x < words; x += 64) {
        const int left = S - 32 * x;
        bm[x] = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
      }
    } else {
      for (int x = lane; x < words; x += 64) bm[x] = 0u;
      float v[NS];
      float mt = -FLT_MAX;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int j = lane + 64 * k;
        v[k] = j < S ? vals[rho][j] : -FLT_MAX;
        mt = fmaxf(mt, v[k]);
      }
      mt = wave_reduce(mt, lane, [](float a, float b) { return fmaxf(a, b); });
      // error of the offsets d = v - mt against the exact z - max: the screen (twice)
      // plus the float32 roundings of v and of d (|v| <= |mt| + lambda for candidates)
      const float eps_d = (float)(2.0 * rc_eps[rho]) + 0x1p-23f * (fabsf(mt) + (float)lambda + 1.f);
      if (!(eps_d <= kTrust)) {
        flagged = true;
      } else {
        uint32_t w[NS], t[NS];
        uint64_t total;
        float tscale, dmin = 0.f;
        {
          uint64_t wsum = 0;
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const float d = v[k] - mt;
            const bool cand_k = (lane + 64 * k < S) && d >= (float)-lambda;
            v[k] = d;
            const float e = cand_k ? __builtin_amdgcn_exp2f(d * 1.44269504088896341f) : 0.f;
            w[k] = (uint32_t)(e * 1073741824.0f);
            wsum += w[k];
            if (w[k] != 0u) dmin = fminf(dmin, d);
          }
          total = wave_reduce(wsum, lane, u64add);
          dmin = wave_reduce(dmin, lane, [](float a, float b) { return fminf(a, b); });
          tscale = dmin < 0.f ? 16777215.0f / (-dmin) : 0.f;
#pragma unroll
          for (int k = 0; k < NS; ++k)
            t[k] = w[k] != 0u ? (uint32_t)fminf((v[k] - dmin) * tscale, 16777215.0f) : 0u;
        }
        const double target = (1.0 - thr) * (double)total;
        // (count, mass) histogram of the candidates with bin(k) >= 0 in one 64-bit
        // word per bin, and the bin where the mass from the top first reaches the
        // target; false when no bin does
        auto crossing = [&](auto bin, uint64_t above_in, int& b_out, uint64_t& above_out, uint32_t& cnt_out) {
#pragma unroll
          for (int x = 0; x < 4; ++x) hist[4 * lane + x] = 0ull;
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const int b = w[k] != 0u ? bin(k) : -1;
            if (b >= 0) atomicAdd((unsigned long long*)&hist[b], (1ull << 44) | (unsigned long long)w[k]);
          }
          __builtin_amdgcn_wave_barrier();
          uint64_t mb[4];
          uint32_t cb[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint64_t hv = hist[4 * lane + x];
            mb[x] = hv & kMassMask;
            cb[x] = (uint32_t)(hv >> 44);
          }
          const uint64_t lane_tot = mb[0] + mb[1] + mb[2] + mb[3];
          uint64_t suf = lane_tot;
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
          __builtin_amdgcn_wave_barrier();
          const uint64_t ball = __ballot(found >= 0);
          if (ball == 0ull) return false;
          const int src = __ffsll((unsigned long long)ball) - 1;
          b_out = __builtin_amdgcn_readlane(found, src);
          cnt_out = (uint32_t)__builtin_amdgcn_readlane((int)f_cnt, src);
          above_out = readlane_u64(f_above, src);
          return true;
        };
        uint32_t tpre = 0;
        int tsh = 24;
        uint64_t above = 0;
        uint32_t cnt = 0;
        bool reach = true;
        while (tsh > 0) {
          const int sh = tsh - 8;
          const uint32_t pf = tpre;
          int b;
          uint64_t ab;
          uint32_t cb;
          if (!crossing([&](int k) { return (t[k] >> tsh) == pf ? (int)((t[k] >> sh) & 255u) : -1; }, above, b, ab,
                        cb)) {
            reach = false;
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
          for (int k = 0; k < NS; ++k)
            if (w[k] != 0u) set_bit(lane + 64 * k);
        } else {
          // candidates: the crossing bin widened by the error margin in key units;
          // blocks above it are kept, below it dropped
          const uint32_t mt_keys = (uint32_t)fminf(ceilf(2.f * eps_d * tscale), 16777215.0f) + 1u;
          const uint32_t lo_t = tpre << tsh, hi_t = lo_t + ((1u << tsh) - 1u);
          const uint32_t lo_m = lo_t > mt_keys ? lo_t - mt_keys : 0u;
          const uint32_t hi_m = hi_t + mt_keys;           // < 2^25: no wrap
          uint64_t sure = 0;
          uint32_t base = 0;
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const bool in = w[k] != 0u && t[k] >= lo_m && t[k] <= hi_m;
            if (w[k] != 0u && t[k] > hi_m) {
              set_bit(lane + 64 * k);
              sure += w[k];
            }
            const uint64_t ball = __ballot(in);
            const uint32_t rank = base + (uint32_t)__popcll(ball & lt_mask);
            if (in && rank < 64u) {
              cand[rank] = (uint32_t)(lane + 64 * k);
              cand[64 + rank] = w[k];
            }
            base += (uint32_t)__popcll(ball);
          }
          above = wave_reduce(sure, lane, u64add);
          const uint32_t ncand = base;
          if (ncand > 64u) {
            flagged = true;
          } else {
            __builtin_amdgcn_wave_barrier();
            // exact float64 logits of the candidates, eight lanes per candidate (each
            // 16 channels), eight candidates per pass
            const int sub = lane & 7, slot = lane >> 3;
            double zc[8];
            const double* qrow = qp + (size_t)r * D + sub * (D / 8);
#pragma unroll
            for (int pass = 0; pass < 8; ++pass) {
              zc[pass] = 0.0;
              const uint32_t cidx = 8u * pass + slot;
              if (8u * pass < ncand) {
                const uint32_t j = cidx < ncand ? cand[cidx] : cand[0];
                const double* krow = kp + (size_t)(rbase + j) * D + sub * (D / 8);
                double zz = 0.0;
#pragma unroll
                for (int d = 0; d < D / 8; d += 2) {
                  const double2 qv = *(const double2*)(qrow + d);
                  const double2 kv = *(const double2*)(krow + d);
                  zz = fma(qv.x, kv.x, zz);
                  zz = fma(qv.y, kv.y, zz);
                }
                zc[pass] = zz;
              }
            }
            // sum the eight partial dots of each candidate (lanes 8s .. 8s+7) and hand
            // candidate c to lane c
            double z = 0.0;
#pragma unroll
            for (int pass = 0; pass < 8; ++pass) {
              double part = zc[pass];
              part += __shfl_xor(part, 1, 8);
              part += __shfl_xor(part, 2, 8);
              part += __shfl_xor(part, 4, 8);
              const double mine = __shfl(part, 8 * (lane & 7), 64);   // candidate 8 pass + lane % 8 -> lane
              if ((lane >> 3) == pass) z = mine;
            }
            const bool have = (uint32_t)lane < ncand;
            const uint32_t my_j = have ? cand[lane] : 0u;
            const uint32_t my_w = have ? cand[64 + lane] : 0u;
            const uint64_t my_key = have ? order_key(z * inv_sqrt_d) : 0ull;   // as the float64 path scales
            uint64_t before = 0;
            for (uint32_t y = 0; y < ncand; ++y) {
              const uint64_t ky = readlane_u64(my_key, (int)y);
              const uint32_t jy = (uint32_t)__builtin_amdgcn_readlane((int)my_j, (int)y);
              const uint32_t wy = (uint32_t)__builtin_amdgcn_readlane((int)my_w, (int)y);
              if (ky > my_key || (ky == my_key && jy < my_j)) before += wy;
            }
            if (have && (double)(above + before) < target) set_bit((int)my_j);
          }
        }
      }
    }
    if (flagged) {                       // the float64 path owns this row
      if (lane == 0) flag_list[atomicAdd(nflag, 1)] = (int32_t)r;
      continue;
    }
    if (win_t >= 0) for_each_window_block(g, i, win_t, win_h, win_w, lane, 64, set_bit);
    __builtin_amdgcn_wave_barrier();
    uint32_t pc = 0;
    for (int x = lane; x < words; x += 64) {
      const uint32_t b = bm[x];
      bitmap[r * words + x] = b;
      pc += __popc(b);
    }
    pc = wave_reduce(pc, lane, [](uint32_t a, uint32_t b2) { return a + b2; });
    if (lane == 0) counts[r] = (int32_t)pc;
    __builtin_amdgcn_wave_barrier();     // bm is reused by the next row
  }
}

}  // namespace scr

hipError_t launch_screen_ops(const Geom& g, const double* qp, const double* kp, const ScreenOps& ops, int32_t* nflag,
                             hipStream_t s) {
  const int64_t heads = (int64_t)g.B * g.nh;
  scr::hstat_init_kernel<<<(unsigned)((heads + 255) / 256), 256, 0, s>>>(ops.hstat, nflag, heads);
  dim3 grid((unsigned)((g.S + 31) / 32), (unsigned)heads, 2);
  if (g.D == 64)
    scr::screen_ops_kernel<64><<<grid, 256, 0, s>>>(qp, kp, ops, g);
  else
    scr::screen_ops_kernel<128><<<grid, 256, 0, s>>>(qp, kp, ops, g);
  return hipGetLastError();
}

hipError_t launch_screen_select(const Geom& g, const ScreenOps& ops, const double* qp, const double* kp, double thr,
                                double lambda, int win_t, int win_h, int win_w, uint32_t* bitmap, int32_t* counts,
                                int words, int32_t* flag_list, int32_t* nflag, hipStream_t s) {
  const double inv = 1.0 / sqrt((double)g.D);
  const unsigned heads = (unsigned)((int64_t)g.B * g.nh);
#define BSA_SCREEN(D_, NS_, ROWS_)                                                                                \
  scr::screen_select_kernel<D_, NS_, ROWS_><<<dim3((unsigned)((g.S + ROWS_ - 1) / ROWS_), heads), 512, 0, s>>>( \
      ops, qp, kp, g, thr, lambda, win_t, win_h, win_w, bitmap, counts, words, flag_list, nflag, inv)
#define BSA_SCREEN_D(NS_, ROWS_) \
  do {                           \
    if (g.D == 64)               \
      BSA_SCREEN(64, NS_, ROWS_); \
    else                         \
      BSA_SCREEN(128, NS_, ROWS_); \
  } while (0)
  if (g.S <= 128) BSA_SCREEN_D(2, 16);
  else if (g.S <= 512) BSA_SCREEN_D(8, 16);
  else if (g.S <= 1024) BSA_SCREEN_D(16, 16);
  else if (g.S <= 2048) BSA_SCREEN_D(32, 16);
  else BSA_SCREEN_D(64, 8);
#undef BSA_SCREEN_D
#undef BSA_SCREEN
  return hipGetLastError();
}

}  // namespace bsa
