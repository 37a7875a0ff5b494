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
// by a power of two into [2^13, 2^14); the pooling pass writes these operands),
// three products per k-step accumulated in float32.  Its error is at most
// 2^-15 |c_i| |e_j| (split error 3 * 2^-22 plus 384 float32 additions), so every
// screened logit of row i is within
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

constexpr double kScreenErr = 0x1p-15;   // relative error of the screened centred dot product
constexpr float kTrust = 4e-5f;          // largest offset error (logit units) a screened row may carry
constexpr int kWaves = 8;


__global__ void __launch_bounds__(256) screen_init_kernel(uint64_t* __restrict__ hstat, int32_t* __restrict__ nflag,
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
// two per SIMD).
//
// Map: the GEMM of the workgroup's ROWS query blocks against the S key blocks
// (16 x 16 tiles of v_mfma_f32_16x16x32_f16; A[i][k] in lane 16 (k / 8) + i,
// register k % 8, B[k][j] likewise with j, C[i][j] in lane 16 (i / 4) + j,
// register i % 4; wave w takes tiles w, w + 8, ..., with the key operands of the
// next two of its tiles in flight) writes the offsets zt_ij = z_ij - ub_i
// (float32, ub_i an upper bound of the row's largest logit, so the offsets of the
// heavy blocks are small numbers) to LDS.
//
// LDS layout of a row: lane l's NS blocks NS l .. NS l + NS - 1 are contiguous,
// each lane's segment padded by 4 floats so that the cut reads them with 16-byte
// loads free of bank conflicts, and the row pitch is 4 (mod 64) floats so that the
// four row groups of an MFMA result land in distinct banks.  Once a wave holds
// its row in registers, the row's LDS is that wave's scratch for the cut
// (histogram, candidate list, bitmap).
//
// Cut: one wavefront per row (ROWS / 8 rows each); the kept blocks of a lane's
// segment form that lane's bits of the bitmap row.
// ---------------------------------------------------------------------------
template <int NS>
struct CutShape {
  static constexpr int kSeg = NS + 4;                        // floats per lane segment
  static constexpr int kPitchV = 64 * kSeg + 4;              // = 4 (mod 64)
  static constexpr int kPitch = kPitchV < 900 ? 900 : kPitchV;   // also >= the 3.5 KB of cut scratch
  static constexpr int kHist = 0, kCand = 512, kBm = 640, kSink = 768;   // scratch offsets (floats)
};

template <int D, int NS, int ROWS>
__global__ void __launch_bounds__(512, 1) screen_select_kernel(ScreenOps ops, const double* __restrict__ qp,
                                                               const double* __restrict__ kp, Geom g, double thr,
                                                               double lambda, int win_t, int win_h, int win_w,
                                                               uint32_t* __restrict__ bitmap,
                                                               int32_t* __restrict__ counts, int words,
                                                               int32_t* __restrict__ flag_list,
                                                               int32_t* __restrict__ nflag, double inv_sqrt_d) {
  using CS = CutShape<NS>;
  static_assert(NS == 2 || (NS % 16 == 0 || NS == 8), "segment shape");
  __shared__ __attribute__((aligned(16))) float vals[ROWS * CS::kPitch];
  __shared__ double rc_a[ROWS], rc_ub[ROWS], rc_eps[ROWS];
  __shared__ int rc_e[ROWS], rc_t[ROWS], rc_y[ROWS], rc_x[ROWS];
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
      rc_x[tid] = i % g.Wp;                 // the block's tile coordinates (window)
      rc_y[tid] = (i / g.Wp) % g.Hp;
      rc_t[tid] = i / (g.Wp * g.Hp);
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
    struct BTile {
      f16x8 hi[D / 32], lo[D / 32];
      double2 rec;                       // (nu_j, scale exponent of key block j)
    };
    // key operands in tile order (see the pooling pass): one contiguous 1 KB per
    // 32-channel step and half; a tile past the end loads the last tile (kept in
    // bounds, result unused), whose slots beyond block S - 1 are never stored
    const int ntile_pad = (S + 15) / 16;
    const _Float16* ksh = ops.ks + (size_t)bh * ntile_pad * (D / 32) * 1024 + 8 * lane;
    auto load_b = [&](int c, BTile& b) {
      const _Float16* src = ksh + (size_t)min(c, ntile_pad - 1) * (D / 32) * 1024;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        b.hi[s] = *(const f16x8*)(src + 1024 * s);
        b.lo[s] = *(const f16x8*)(src + 1024 * s + 512);
      }
      b.rec = ops.krec[rbase + min(16 * c + jl, S - 1)];
    };
    auto tile = [&](int c, const BTile& b) {
      if (c >= ntile) return;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[s], b.hi[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_hi[s], b.lo[s], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa_lo[s], b.hi[s], acc, 0, 0, 0);
      }
      const int j = 16 * c + jl;
      if (j < S) {
        const int ek = (int)b.rec.y;
        float* dst = vals + (j / NS) * CS::kSeg + (j % NS);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int rho = 4 * (lane >> 4) + x;
          if (rho < ROWS) {
            const double z = fma(ra[x], b.rec.x, ldexp((double)acc[x], -(re[x] + ek)));
            dst[rho * CS::kPitch] = (float)fma(z, inv_sqrt_d, -rub[x]);
          }
        }
      }
    };
    // the scheduling barriers keep the three load groups in ring order, so that the
    // loads pending at the loop head are the same on entry and on the back edge and
    // each tile waits only for its own group
    BTile b0, b1, b2;
    int c = wave;
    load_b(c, b0);
    __builtin_amdgcn_sched_barrier(0);
    load_b(c + kWaves, b1);
    __builtin_amdgcn_sched_barrier(0);
    for (; c < ntile; c += 3 * kWaves) {
      load_b(c + 2 * kWaves, b2);
      __builtin_amdgcn_sched_barrier(0);
      tile(c, b0);
      __builtin_amdgcn_sched_barrier(0);
      load_b(c + 3 * kWaves, b0);
      __builtin_amdgcn_sched_barrier(0);
      tile(c + kWaves, b1);
      __builtin_amdgcn_sched_barrier(0);
      load_b(c + 4 * kWaves, b1);
      __builtin_amdgcn_sched_barrier(0);
      tile(c + 2 * kWaves, b2);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();

  // ---- the cut, one wavefront per row --------------------------------------
  auto u64add = [](uint64_t a, uint64_t b) { return a + b; };
  constexpr uint64_t kMassMask = (1ull << 44) - 1;
  const int jbase = NS * lane;           // this lane's first block
  for (int rho = wave; rho < ROWS; rho += kWaves) {
    const int i = i0 + rho;
    if (i >= S) break;
    const int64_t r = rbase + i;
    float* row = vals + rho * CS::kPitch;
    uint64_t* hist = (uint64_t*)(row + CS::kHist);   // bin b at hist[255 - b]
    uint32_t* cand = (uint32_t*)(row + CS::kCand);   // crossing candidates: block ids, then masses
    uint32_t* bm = (uint32_t*)(row + CS::kBm);
    uint64_t bits = 0;                   // bit k: block jbase + k is kept
    // blocks of this lane below S, opaque per row: the compiler would otherwise hoist
    // NS loop-invariant lane masks out of the row loop and spill them
    int nv = S - jbase;
    asm volatile("" : "+v"(nv));
    bool flagged = false;
    bool keep_c = false;                 // lane c < ncand: exactly ranked candidate c is kept
    uint32_t my_j = 0;
    if (thr == 0.0) {
#pragma unroll
      for (int k = 0; k < NS; ++k)
        if (k < nv) bits |= 1ull << k;
    } else {
      float v[NS];
      if constexpr (NS == 2) {
        const float2 x = *(const float2*)(row + lane * CS::kSeg);
        v[0] = x.x;
        v[1] = x.y;
      } else {
#pragma unroll
        for (int m = 0; m < NS / 4; ++m) {
          const float4 x = *(const float4*)(row + lane * CS::kSeg + 4 * m);
          v[4 * m] = x.x;
          v[4 * m + 1] = x.y;
          v[4 * m + 2] = x.z;
          v[4 * m + 3] = x.w;
        }
      }
      asm volatile("" ::: "memory");     // the row's LDS becomes scratch below
      // this lane's slice of the query block for the exact dots (8 lanes per candidate)
      const int sub = lane & 7, slot = lane >> 3;
      constexpr int kQV = D / 16;        // double2 per slice
      double2 qv[kQV];
      auto load_q = [&]() {
        const double2* qrow = (const double2*)(qp + (size_t)r * D + sub * (D / 8));
#pragma unroll
        for (int e = 0; e < kQV; ++e) qv[e] = qrow[e];
      };
      if constexpr (NS <= 32) load_q();   // early, in flight during the cut (registers allowing)
      float mt = -FLT_MAX;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        v[k] = k < nv ? v[k] : -FLT_MAX;
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
            const bool cand_k = d >= (float)-lambda;   // blocks past S hold -FLT_MAX
            v[k] = d;
            const float e = cand_k ? __builtin_amdgcn_exp2f(d * 1.44269504088896341f) : 0.f;
            w[k] = (uint32_t)(e * 1073741824.0f);
            wsum += w[k];
            dmin = fminf(dmin, w[k] != 0u ? d : 0.f);
          }
          total = wave_reduce(wsum, lane, u64add);
          dmin = wave_reduce(dmin, lane, [](float a, float b) { return fminf(a, b); });
          tscale = dmin < 0.f ? 16777215.0f / (-dmin) : 0.f;
          // non-candidates get key 2^31: no radix prefix matches it, it is negative as an
          // int, and above every margin unsigned (no per-block predicate stays live)
#pragma unroll
          for (int k = 0; k < NS; ++k)
            t[k] = w[k] != 0u ? (uint32_t)fminf((v[k] - dmin) * tscale, 16777215.0f) : 0x80000000u;
        }
        const double target = (1.0 - thr) * (double)total;
        // (count, mass) histogram of the candidates with bin(k) >= 0 in one 64-bit
        // word per bin, and the bin where the mass from the top first reaches the
        // target; false when no bin does
        auto crossing = [&](auto bin, uint64_t above_in, int& b_out, uint64_t& above_out, uint32_t& cnt_out) {
          *(uint4*)(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
          *(uint4*)(hist + 4 * lane + 2) = make_uint4(0u, 0u, 0u, 0u);
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const int b = bin(k);
            if (b >= 0) atomicAdd((unsigned long long*)&hist[255 - b], (1ull << 44) | (unsigned long long)w[k]);
          }
          __builtin_amdgcn_wave_barrier();
          // lane l holds bins 255 - 4l .. 252 - 4l, highest first
          const uint4 h01 = *(const uint4*)(hist + 4 * lane), h23 = *(const uint4*)(hist + 4 * lane + 2);
          const uint64_t hv[4] = {((uint64_t)h01.y << 32) | h01.x, ((uint64_t)h01.w << 32) | h01.z,
                                  ((uint64_t)h23.y << 32) | h23.x, ((uint64_t)h23.w << 32) | h23.z};
          uint64_t mb[4];
          uint32_t cb[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            mb[x] = hv[x] & kMassMask;
            cb[x] = (uint32_t)(hv[x] >> 44);
          }
          const uint64_t lane_tot = mb[0] + mb[1] + mb[2] + mb[3];
          uint64_t run = wave_prefix_u64(lane_tot, lane) - lane_tot;   // mass of the higher bins
          int found = -1;
          uint64_t f_above = 0;
          uint32_t f_cnt = 0;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint64_t excl = run;
            run += mb[x];
            if (cb[x] != 0u && (double)(above_in + excl) < target && target <= (double)(above_in + run)) {
              found = 255 - 4 * lane - x;
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
            if ((int)t[k] >= 0) bits |= 1ull << k;
        } else {
          // candidates: the crossing bin widened by the error margin in key units;
          // blocks above it are kept, below it dropped
          const uint32_t mt_keys = (uint32_t)fminf(ceilf(2.f * eps_d * tscale), 16777215.0f) + 1u;
          const uint32_t lo_t = tpre << tsh, hi_t = lo_t + ((1u << tsh) - 1u);
          const uint32_t lo_m = lo_t > mt_keys ? lo_t - mt_keys : 0u;
          const uint32_t hi_m = hi_t + mt_keys;           // < 2^25: no wrap
          uint64_t sure = 0, inbits = 0;
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            if ((int)t[k] > (int)hi_m) {
              bits |= 1ull << k;
              sure += w[k];
            }
            if (t[k] >= lo_m && t[k] <= hi_m) inbits |= 1ull << k;
          }
          // candidate slots: this lane's come after those of the lower lanes
          const uint32_t nin = (uint32_t)__popcll(inbits);
          const uint64_t incl = wave_prefix_u64(nin, lane);
          const uint32_t ncand = (uint32_t)readlane_u64(incl, 63);
          if (ncand <= 64u) {
            // branch-free: a block that is no candidate is written to this lane's own
            // sink slot (distinct per lane, so the stores never collide)
            uint32_t slot_c = (uint32_t)incl - nin;
            uint32_t* sink = (uint32_t*)(row + CS::kSink) + lane;
#pragma unroll
            for (int k = 0; k < NS; ++k) {
              const bool in = (inbits >> k) & 1ull;
              uint32_t* dj = in ? cand + slot_c : sink;
              uint32_t* dw = in ? cand + 64 + slot_c : sink + 64;
              *dj = (uint32_t)(jbase + k);
              *dw = w[k];
              slot_c += in ? 1u : 0u;
            }
          }
          above = wave_reduce(sure, lane, u64add);
          if (ncand > 64u) {
            flagged = true;
          } else if (ncand > 0u) {
            __builtin_amdgcn_wave_barrier();
            // exact float64 logits of the candidates: eight lanes per candidate (each
            // D / 8 channels), eight candidates per pass, the next pass's key slices
            // in flight while the current one is summed
            const int np = (int)((ncand + 7u) / 8u);
            auto load_k = [&](int p, double2* kv) {
              const uint32_t cidx = min(8u * (uint32_t)p + (uint32_t)slot, ncand - 1u);
              const double2* krow = (const double2*)(kp + (size_t)(rbase + cand[cidx]) * D + sub * (D / 8));
#pragma unroll
              for (int e = 0; e < kQV; ++e) kv[e] = krow[e];
            };
            double z = 0.0;
            auto pass = [&](int p, const double2* kv) {
              double part = 0.0;
#pragma unroll
              for (int e = 0; e < kQV; ++e) {
                part = fma(qv[e].x, kv[e].x, part);
                part = fma(qv[e].y, kv[e].y, part);
              }
              part = sum8(part);
              const double mine = __shfl(part, 8 * (lane & 7), 64);   // candidate 8 p + lane % 8 -> lane
              if ((lane >> 3) == p) z = mine;
            };
            if constexpr (NS > 32) load_q();
            double2 ka[kQV], kb[kQV];
            load_k(0, ka);
            for (int p = 0; p < np; p += 2) {
              load_k(min(p + 1, np - 1), kb);
              pass(p, ka);
              if (p + 1 >= np) break;
              load_k(min(p + 2, np - 1), ka);
              pass(p + 1, kb);
            }
            const bool have = (uint32_t)lane < ncand;
            my_j = have ? cand[lane] : 0u;
            const uint32_t my_w = have ? cand[64 + lane] : 0u;
            const uint64_t my_key = have ? order_key(z * inv_sqrt_d) : 0ull;   // as the float64 path scales
            uint64_t before = 0;
            for (uint32_t y = 0; y < ncand; ++y) {
              const uint64_t ky = readlane_u64(my_key, (int)y);
              const uint32_t jy = (uint32_t)__builtin_amdgcn_readlane((int)my_j, (int)y);
              const uint32_t wy = (uint32_t)__builtin_amdgcn_readlane((int)my_w, (int)y);
              if (ky > my_key || (ky == my_key && jy < my_j)) before += wy;
            }
            keep_c = have && (double)(above + before) < target;
          }
        }
      }
    }
    if (flagged) {                       // the float64 path owns this row
      if (lane == 0) flag_list[atomicAdd(nflag, 1)] = (int32_t)r;
      continue;
    }
    // this lane's bits into the bitmap row, then the exactly ranked candidates and
    // the window on top
    if constexpr (NS == 64) {
      *(uint64_t*)(bm + 2 * lane) = bits;
    } else if constexpr (NS == 32) {
      bm[lane] = (uint32_t)bits;
    } else {
      constexpr int G = 32 / NS;         // lanes per bitmap word
      uint32_t x = (uint32_t)bits << ((lane % G) * NS);
#pragma unroll
      for (int s = 1; s < G; s <<= 1) x |= (uint32_t)__shfl_xor((int)x, s, 64);
      if (lane % G == 0) bm[lane / G] = x;
    }
    __builtin_amdgcn_wave_barrier();
    if (keep_c) atomicOr(&bm[my_j >> 5], 1u << (my_j & 31));
    if (win_t >= 0) {
      // the window's runs of consecutive blocks, as word masks
      for_each_window_run(g, rc_t[rho], rc_y[rho], rc_x[rho], win_t, win_h, win_w, lane, 64, [&](int a, int b) {
        for (int wd = a >> 5; wd <= (b >> 5); ++wd) {
          const int lo = max(a - 32 * wd, 0), hi = min(b - 32 * wd, 31);
          const uint32_t m = hi - lo == 31 ? 0xffffffffu : ((1u << (hi - lo + 1)) - 1u) << lo;
          atomicOr(&bm[wd], m);
        }
      });
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t pc = 0;
    for (int x = lane; x < words; x += 64) {
      const uint32_t b = bm[x];
      bitmap[r * words + x] = b;
      pc += __popc(b);
    }
    pc = wave_reduce(pc, lane, [](uint32_t a, uint32_t b2) { return a + b2; });
    if (lane == 0) counts[r] = (int32_t)pc;
  }
}

}  // namespace scr

hipError_t launch_screen_init(const Geom& g, const ScreenOps& ops, int32_t* nflag, hipStream_t s) {
  const int64_t heads = (int64_t)g.B * g.nh;
  scr::screen_init_kernel<<<(unsigned)((heads + 255) / 256), 256, 0, s>>>(ops.hstat, nflag, heads);
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
