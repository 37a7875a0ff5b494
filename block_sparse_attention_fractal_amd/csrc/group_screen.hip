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
// channels and the two cross products hi*lo, lo*hi go to four float32
// accumulators: with at most 64 additions per hi*hi accumulator (D = 128) the
// float32 sums are within 2^-17 of the sum of |products| (the cross products are
// 2^-10 smaller), the split and the dropped lo*lo term add
// 3 * 2^-22 and the float32 epilogue (the accumulators summed, scaled and added to
// the rank-one part minus the row's bound) 2^-22, so every screened logit of row i
// is within
//   eps_i = 1.1875 * 2^-17 |c_i| max_j |e_j| / sqrt(D)
// of the exact one (four times tighter than the single-accumulator bound of the
// block screen: the group means average 4 tokens instead of 64, so their centred
// norms are about 4 times larger), and the stored float32 offset v adds 2^-22 |v|.
//
//   * pool_groups_screen_kernel: the screen operands of every group (from the
//     float64 means of its 4 keys), in MFMA tile order;
//   * group_logits_screen_kernel: the screened map of a chunk of heads as float32
//     offsets (z - ub_i) log2(e) (ub_i an upper bound of the row's largest logit;
//     log2 units, so a mass is one exp2), written to HBM (4 bytes per entry
//     instead of 8);
//   * group_screen_select_kernel: one 1024-thread workgroup per row, each thread
//     holding 32 consecutive entries in registers (so its bits are one bitmap
//     word).  The cut is the block screen's: masses in fixed point from the
//     screened offsets, a 24-bit key radix-selected 8 bits per pass with one
//     histogram per pair of wavefronts, the crossing bin widened by the error
//     margin; the entries above it are kept, those inside it (at most 64) are
//     handed with the mass above them to group_rank_kernel; the rows' counts are
//     taken from the bitmap afterwards (bitmap_count_kernel).  Rows whose margin the screen cannot
//     guarantee, or with more than 64 entries inside it, are listed for the exact
//     float64 path (group_mask.hip);
//   * group_rank_kernel: the handed-over entries get their exact float64 logits
//     (group means formed again from the 4 keys) and are ranked exactly, one
//     wavefront per row with many rows in flight (so their loads do not stall a
//     whole workgroup).
#include <float.h>

#include <algorithm>

#include "kernels.h"
#include "mask_util.h"

namespace bsa {
namespace gscr {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr double kScreenErr = 0x1.3p-17;   // relative error of the screened centred dot product
constexpr float kTrust = 4e-5f;            // largest offset error (logit units) a screened row may carry
constexpr int kNT = 1024;                  // select: threads per row
constexpr int kNW = kNT / 64;
constexpr int kPer = 32;                   // entries per thread: 32768 groups per head at most
constexpr int kMaxCand = 64;               // exactly ranked entries per row
constexpr int kRowsWG = 256;               // map: query blocks per workgroup (32 per wave)
constexpr int kMapWaves = kRowsWG / 32;     // map: waves per workgroup
constexpr int kStep = 64;                  // map: key groups per LDS stage (4 tiles of 16)

// ---------------------------------------------------------------------------
// Screen operands of the key groups.  grid = (ceil(L/4 / 64), B * heads), 256
// threads: wave w takes the 16 groups of tile 4 x + w, lane l the group l % 16 and
// its 8-channel chunks l / 16 + 4 u (u < D / 32), so that each fp16 store of a
// wave fills 1 KB of the tile layout (16-group tiles, per 32-channel step u and
// half (hi, lo) 1 KB holding, at lane slot 16 (chunk % 4) + group % 16, the 8
// channels that lane of v_mfma_f32_16x16x32_f16 takes).  The group means are not
// stored: the exact recomputations form them again from the 4 keys.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) pool_groups_screen_kernel(const T* __restrict__ k, ScreenOps ops, Geom g) {
  constexpr int KS = D / 32;
  constexpr int EPC = 16 / sizeof(T);        // elements per 16-byte load
  constexpr int NLD = 8 / EPC;               // loads per 8-channel chunk
  __shared__ uint64_t red[3][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t bh = blockIdx.y;
  const int SG = g.L / 4, ntg = (SG + 15) / 16, gpb = g.N / 4;
  const int tile = blockIdx.x * 4 + wave;
  const int g16 = lane & 15, cq = lane >> 4;
  const int gid = tile * 16 + g16;
  const bool ok = gid < SG;
  const int gq = min(gid, SG - 1);
  const int blk = gq / gpb, m0 = (gq % gpb) * 4;
  uint4 raw[4][KS][NLD];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const T* src = k + ((size_t)bh * g.L + block_token_row(g, blk, m0 + t)) * D;
#pragma unroll
    for (int u = 0; u < KS; ++u)
#pragma unroll
      for (int x = 0; x < NLD; ++x) raw[t][u][x] = *(const uint4*)(src + 8 * (cq + 4 * u) + x * EPC);
  }
  double acc[KS][8];
#pragma unroll
  for (int u = 0; u < KS; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[u][e] = 0.0;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < KS; ++u)
#pragma unroll
      for (int x = 0; x < NLD; ++x) add_chunk<T>(&acc[u][x * EPC], raw[t][u][x]);
  double s = 0.0;
#pragma unroll
  for (int u = 0; u < KS; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[u][e] *= 0.25;                                   // sums of 4 inputs are exact in float64
      s += acc[u][e];
    }
  s += xor16(s, lane);                                     // the group's 4 lanes: l, l ^ 16, l ^ 32, l ^ 48
  s += xor32(s, lane);
  const double mu = s * (1.0 / D);
  double amax = 0.0, n2 = 0.0;
#pragma unroll
  for (int u = 0; u < KS; ++u)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      acc[u][e] -= mu;
      amax = fmax(amax, fabs(acc[u][e]));
      n2 = fma(acc[u][e], acc[u][e], n2);
    }
  amax = fmax(amax, xor16(amax, lane));
  amax = fmax(amax, xor32(amax, lane));
  n2 += xor16(n2, lane);
  n2 += xor32(n2, lane);
  const int ex = amax > 0.0 ? 13 - ilogb(amax) : 0;     // scaled magnitudes in [2^13, 2^14)
  if (ok) {
#pragma unroll
    for (int u = 0; u < KS; ++u) {
      _Float16 hv[8], lv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // double -> float -> fp16 on the hardware converts (the opaque copies keep the
        // compiler from fusing them into a software double -> fp16 rounding)
        const double x = ldexp(acc[u][e], ex);
        float xf = (float)x;
        asm volatile("" : "+v"(xf));
        const _Float16 hi = (_Float16)xf;
        float rf = (float)(x - (double)hi);
        asm volatile("" : "+v"(rf));
        hv[e] = hi;
        lv[e] = (_Float16)rf;
      }
      _Float16* dst = ops.ks + (((size_t)(bh * ntg + tile) * KS + u) * 2) * 512 + (16 * cq + g16) * 8;
      *(uint4*)dst = *(const uint4*)hv;
      *(uint4*)(dst + 512) = *(const uint4*)lv;
    }
  }
  const double nrm = sqrt(n2) * (1.0 + 0x1p-50);          // rounded up: an upper bound of |e|
  if (ok && cq == 0) ops.krec[(size_t)bh * SG + gid] = make_double2(mu, (double)ex);
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
// logits times sqrt(D) and the error bound eps_i (identical expressions in both
// kernels)
struct RowScreen {
  double a, u, eps;
};
__device__ __forceinline__ RowScreen row_screen(const ScreenOps& ops, int64_t r, int64_t bh, int D, double inv_sqrt_d) {
  const double a = (double)D * ops.qmu[r];
  const double bmax = key_to_double(ops.hstat[3 * bh]), bmin = key_to_double(ops.hstat[3 * bh + 1]);
  const double cmax = key_to_double(ops.hstat[3 * bh + 2]);
  const double nq = ops.qn[r];
  RowScreen rs;
  rs.a = a;
  rs.u = a * (a >= 0.0 ? bmax : bmin) + nq * cmax;
  rs.eps = kScreenErr * nq * cmax * inv_sqrt_d;
  return rs;
}

// ---------------------------------------------------------------------------
// Screened map of heads h0 .. h0 + gridDim.z - 1: zt[(h - h0) S + i][j] =
// (z~_ij - ub_i) log2(e) in float32 (log2 units), row pitch `pitch` floats.  grid =
// (column slices, ceil(S / 256), heads), 512 threads.  Wave w holds the operands
// (hi, lo) of query blocks i0 + 32 w .. + 31 in registers; the workgroup streams
// its slice of key groups through LDS 64 at a time, by direct-to-LDS buffer loads
// into two stage buffers (the next stage in flight while the current one is
// multiplied; 256 query blocks share every group operand read).  MFMA layouts as in
// mask_screen.hip: A[i][k] in lane 16 (k / 8) + i, B[k][j] in lane 16 (k / 8) + j,
// C[i][j] in lane 16 (i / 4) + j, register i % 4.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kMapWaves * 64, 1) group_logits_screen_kernel(ScreenOps ops, float* __restrict__ zt, Geom g,
                                                                     int64_t h0, int steps_per_slice, int pitch,
                                                                     double inv_sqrt_d) {
  constexpr int KS = D / 32;                 // k-steps of 32 channels
  constexpr int kTileB = KS * 2048;          // bytes per 16-group tile (hi and lo)
  constexpr int kStageB = 4 * kTileB;        // bytes per stage (4 tiles)
  constexpr int kLoads = kStageB / (kMapWaves * 1024);   // 1 KB direct-to-LDS loads per wave per stage
  static_assert(kLoads * kMapWaves * 1024 == kStageB, "stage shape");
  __shared__ __attribute__((aligned(16))) uint8_t bs[2][kStageB];   // two stages: the one in use, the next
  __shared__ __attribute__((aligned(16))) double2 recs[2][kStep];  // (nu_j, exponent) of the stage's groups
  __shared__ double rc_a[kRowsWG], rc_u[kRowsWG];
  __shared__ float rc_s[kRowsWG];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = g.S, SG = g.L / 4, ntg = (SG + 15) / 16;
  const int64_t bh = h0 + blockIdx.z;
  const int i0 = blockIdx.y * kRowsWG;
  const int64_t rbase = bh * S;
  const float sc = (float)(inv_sqrt_d * 1.4426950408889634);   // offsets in log2 units
  if (tid < kRowsWG) {
    const int i = i0 + tid;
    if (i < S) {
      const RowScreen rs = row_screen(ops, rbase + i, bh, D, inv_sqrt_d);
      rc_a[tid] = rs.a;
      rc_u[tid] = rs.u;
      rc_s[tid] = ldexpf(sc, -ops.qe[rbase + i]);          // undoes the row's scaling, then log2(e)/sqrt(D)
    } else {
      rc_a[tid] = 0.0;
      rc_u[tid] = 0.0;
      rc_s[tid] = 0.f;
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
  // the head's group operands and (mean, exponent) pairs behind buffer resources:
  // reads past the end (the last stage's missing tiles) return zeros
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(ops.ks + (size_t)bh * ntg * (kTileB / 2)), (short)0, ntg * kTileB,
                                        0x00020000);
  const __amdgpu_buffer_rsrc_t rrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(ops.krec + (size_t)bh * SG), (short)0, SG * 16, 0x00020000);
  // this head's rows of the map: a store whose offset is past the end (rows >= S,
  // groups >= L/4) is dropped by the hardware, so every lane stores on every tile and
  // each stage issues the same number of stores
  const int zbytes = S * pitch * 4;                        // < 2^31 (S <= 4096, pitch <= 32768)
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zt + (size_t)blockIdx.z * S * (size_t)pitch), (short)0, zbytes, 0x00020000);
  // stage st into LDS buffer st & 1: kLoads 1 KB loads per wave (wave 0 also the
  // stage's 64 (mean, exponent) pairs)
  auto issue = [&](int st) __attribute__((always_inline)) {
    const int buf = st & 1;
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(&bs[buf][(wave * kLoads + u) * 1024]), 16,
                                               lane * 16 + (wave * kLoads + u) * 1024, st * kStageB, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rrs, (lds_void*)(&recs[buf][0]), 16, lane * 16, st * kStep * 16, 0, 0);
  };
  if (st0 < st1) issue(st0);
  __builtin_amdgcn_s_waitcnt(0x0F70);                      // vmcnt(0): the A operands and the first stage
  __syncthreads();                                         // ... in every wave, and the row constants
  // the transposed product C^T[g][q] = sum_k E[g][k] Q[q][k] (group operands in the A
  // position): lane l holds query row l % 16 of a row tile and the 4 consecutive
  // groups 4 (l / 16) .. + 3 of a tile, i.e. 16 contiguous bytes of a map row
  double ra[2], ru[2];
  float rsc[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int rho = 32 * wave + 16 * rt + (lane & 15);
    ra[rt] = rc_a[rho];
    ru[rt] = rc_u[rho];
    rsc[rt] = rc_s[rho];
  }
  const int gq = 4 * (lane >> 4);                          // this lane's first group of a tile
  for (int st = st0; st < st1; ++st) {
    const int buf = st & 1;
    if (st + 1 < st1) issue(st + 1);                       // into the buffer read two stages ago
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = (4 * st + u) * 16 + gq;
      const _Float16* tb = (const _Float16*)&bs[buf][u * kTileB];
      f16x8 bhi[KS], blo[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        bhi[s] = *(const f16x8*)(tb + s * 1024 + 8 * lane);
        blo[s] = *(const f16x8*)(tb + s * 1024 + 512 + 8 * lane);
      }
      double2 rec[4];
      float csc[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        rec[x] = recs[buf][16 * u + gq + x];
        csc[x] = ldexpf(1.f, -(int)rec[x].y);             // undoes the group's scaling
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        // hi*hi of the two channel halves, and the two cross products, each its own
        // accumulator (short dependency chains)
        f32x4 p0 = {0.f, 0.f, 0.f, 0.f}, p1 = p0, pa = p0, pb = p0;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          if (s < KS / 2)
            p0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(bhi[s], ah[rt][s], p0, 0, 0, 0);
          else
            p1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(bhi[s], ah[rt][s], p1, 0, 0, 0);
          pa = __builtin_amdgcn_mfma_f32_16x16x32_f16(blo[s], ah[rt][s], pa, 0, 0, 0);
          pb = __builtin_amdgcn_mfma_f32_16x16x32_f16(bhi[s], al[rt][s], pb, 0, 0, 0);
        }
        const int i = i0 + 32 * wave + 16 * rt + (lane & 15);
        f32x4 v;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          // (a nu_j - sqrt(D) ub_i) in float64, then everything in float32
          const float dot = (p0[x] + p1[x]) + (pa[x] + pb[x]);
          const float rk = (float)fma(ra[rt], rec[x].x, -ru[rt]);
          v[x] = fmaf(dot, rsc[rt] * csc[x], rk * sc);
        }
        // groups j .. j + 3 of row i (past L/4 they land in the row's padding, which the
        // pitch leaves up to a multiple of 32); rows >= S and groups >= L/4: dropped
        const int off = (i < S && j < SG) ? (i * pitch + j) * 4 : zbytes;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), zrs, off, 0, 0);
      }
    }
    // this wave's loads of the next stage have landed once at most the 8 stores issued
    // after them (4 tiles x 2 row tiles) are outstanding; the barrier then publishes
    // every wave's loads and frees this stage's buffer (the compiler's own barrier
    // would wait for the stores as well)
    static_assert(4 * 2 == 8, "stores per stage counted by the wait");
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// ---------------------------------------------------------------------------
// The cut of rows row0 .. row0 + gridDim.x - 1 (zt: those rows, pitch floats apart,
// offsets in log2 units), one 1024-thread workgroup per row.  Thread t holds
// entries 32 t .. 32 t + 31 of the row in registers, so its bits are one bitmap
// word; the row's count is taken from the bitmap afterwards.
// ---------------------------------------------------------------------------
constexpr int kHist = kNW / 2;             // radix histograms: one per pair of waves

struct SelSmem {
  uint64_t hist[kHist][256];          // per wave pair: (count << 44) | mass, top bin first
  uint32_t bm[kNT];                   // the row's bitmap words
  uint32_t cj[kMaxCand], cw[kMaxCand];   // entries inside the margin: index, mass
  uint64_t red_u[kNW];
  float red_f[kNW], red_g[kNW];
  uint64_t scan[4];
  uint64_t found_above;
  int found_bin;
  uint32_t found_cnt, ncand;
};

__global__ void __launch_bounds__(kNT) group_screen_select_kernel(
    const float* __restrict__ zt, int pitch, ScreenOps ops, int64_t row0, Geom g, double thr, int win_t, int win_h,
    int win_w, uint32_t* __restrict__ bitmap, int words, int32_t* __restrict__ flag_list,
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
  constexpr float kLog2e = 1.44269504088896341f;
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

  uint32_t bits = 0;                                       // bit k: entry jb + k is kept
  uint32_t nrank = 0;                                      // entries left to group_rank_kernel
  if (thr == 0.0) {
    bits = nv >= 32 ? 0xffffffffu : (nv > 0 ? (1u << nv) - 1u : 0u);
  } else {
    const double nq = ops.qn[r];                           // the screen bound's inputs, early
    const uint64_t cm = ops.hstat[3 * bh + 2];
    float v[kPer];
    if (nv > 0) {
      const float4* src = (const float4*)(zt + (size_t)blockIdx.x * pitch + jb);   // pitch: a multiple of 32
#pragma unroll
      for (int m = 0; m < kPer / 4; ++m) {
        const float4 q = src[m];
        v[4 * m] = q.x;
        v[4 * m + 1] = q.y;
        v[4 * m + 2] = q.z;
        v[4 * m + 3] = q.w;
      }
    }
    float mt = -FLT_MAX, mn = FLT_MAX;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const bool ok = k < nv;
      v[k] = ok ? v[k] : -FLT_MAX;
      mt = fmaxf(mt, v[k]);
      mn = fminf(mn, ok ? v[k] : FLT_MAX);
    }
    if (tid == 0) sm.ncand = 0u;
    ((uint4*)&sm.hist[0][0])[tid] = make_uint4(0u, 0u, 0u, 0u);   // kHist * 256 words of 8 bytes
    static_assert(kHist * 256 * 8 == kNT * 16, "one 16-byte clear per thread");
    mt = wave_reduce(mt, lane, [](float a, float b) { return fmaxf(a, b); });
    mn = wave_reduce(mn, lane, [](float a, float b) { return fminf(a, b); });
    if (lane == 0) {
      sm.red_f[wv] = mt;
      sm.red_g[wv] = mn;
    }
    __syncthreads();
    for (int y = 0; y < kNW; ++y) {
      mt = fmaxf(mt, sm.red_f[y]);
      mn = fminf(mn, sm.red_g[y]);
    }
    // error of the offsets d = v - mt (log2 units) against the exact ones: the screen
    // (twice), 2^-22 |v| from the map's float32 epilogue for v and for mt, and the
    // rounding of d (|d| <= 30 for an entry with mass, |v| <= |mt| + |d|)
    const double eps_i = kScreenErr * nq * key_to_double(cm) * inv_sqrt_d;   // as in row_screen
    const float eps_d = (float)(2.0 * (double)kLog2e * eps_i) + 0x1p-21f * (fabsf(mt) + 19.f);
    if (!(eps_d <= kTrust * kLog2e)) {                     // uniform: the float64 path owns this row
      if (tid == 0) {
        flag_list[atomicAdd(nflag, 1)] = (int32_t)r;
        cn[r] = 0;
      }
      return;
    }
    // masses in fixed point, 2^30 at the row max: exp2(d + 30), 0 below d = -30
    const float mref = mt - 30.f;
    const float vlo = fmaxf(mn, mref);                     // at or below every entry with mass
    const float tscale = mt > vlo ? 16777215.0f / (mt - vlo) : 0.f;
    uint32_t w[kPer], t[kPer];
    uint64_t wsum = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      w[k] = (uint32_t)__builtin_amdgcn_exp2f(v[k] - mref);
      wsum += w[k];
      // entries without mass get key 2^31: no radix prefix matches it, it is negative
      // as an int and above every margin unsigned
      t[k] = w[k] != 0u ? (uint32_t)fminf((v[k] - vlo) * tscale, 16777215.0f) : 0x80000000u;
    }
    const uint64_t total = bsum(wsum);
    const double target = (1.0 - thr) * (double)total;     // keep while the mass before < target

    // one radix pass: (count, mass) histogram of bin(k) >= 0 per wave pair, summed over
    // the pairs by threads 0..255 (thread y: bin 255 - y), a prefix over the bins from
    // the top, and the bin in which the mass reaches the target; the histograms are
    // cleared for the next pass once they have been read
    auto crossing = [&](auto bin, uint64_t above_in, int& b_out, uint64_t& above_out, uint32_t& cnt_out)
                        __attribute__((always_inline)) {
      uint64_t* hw = sm.hist[wv >> 1];
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
        for (int y = 0; y < kHist; ++y) {
          const uint64_t h = sm.hist[y][tid];
          mb += h & kMassMask;
          cb += (uint32_t)(h >> 44);
        }
      }
      uint64_t incl = wave_prefix_u64(mb, lane);
      if (tid == 0) sm.found_bin = -1;
      if (wv < 4 && lane == 63) sm.scan[wv] = incl;
      __syncthreads();
      if (tid < 256) {
        for (int y = 0; y < wv; ++y) incl += sm.scan[y];
        const uint64_t excl = incl - mb;
        if (cb != 0u && (double)(above_in + excl) < target && target <= (double)(above_in + incl)) {
          sm.found_bin = 255 - tid;
          sm.found_above = above_in + excl;
          sm.found_cnt = cb;
        }
      }
      ((uint4*)&sm.hist[0][0])[tid] = make_uint4(0u, 0u, 0u, 0u);   // for the next pass
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
      for (int k = 0; k < kPer; ++k) bits |= ((int)t[k] >= 0 ? 1u : 0u) << k;
    } else {
      // the crossing bin widened by the error margin in key units; entries above it
      // are kept, those inside it handed to group_rank_kernel, those below dropped
      const uint32_t mt_keys = (uint32_t)fminf(ceilf(2.f * eps_d * tscale), 16777215.0f) + 1u;
      const uint32_t lo_t = tpre << tsh, hi_t = lo_t + ((1u << tsh) - 1u);
      const uint32_t lo_m = lo_t > mt_keys ? lo_t - mt_keys : 0u;
      const uint32_t hi_m = hi_t + mt_keys;                // < 2^25: no wrap
      uint64_t sure = 0;
      uint32_t inm = 0;                                    // bit k: register k inside the margin
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const bool up = (int)t[k] > (int)hi_m;
        bits |= (up ? 1u : 0u) << k;
        sure += up ? w[k] : 0u;
        inm |= (t[k] >= lo_m && t[k] <= hi_m ? 1u : 0u) << k;
      }
      // the few entries inside the margin (a handful per row): only the waves holding
      // one take the per-register path
      if (__builtin_amdgcn_ballot_w64(inm != 0u) != 0ull) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          if ((inm >> k) & 1u) {
            const uint32_t slot = atomicAdd(&sm.ncand, 1u);
            if (slot < (uint32_t)kMaxCand) {
              sm.cj[slot] = (uint32_t)(jb + k);
              sm.cw[slot] = w[k];
            }
          }
        }
      }
      above = bsum(sure);                                  // (its barriers also publish the entries)
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
  // the bitmap row: this thread's word, then the window on top (every group of every
  // window block)
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
  if (tid < words) bitmap[r * words + tid] = sm.bm[tid];
}

// Kept counts of rows from their bitmap rows (after the screened cut, the exact
// ranking and the float64 path): one wavefront per row.
__global__ void __launch_bounds__(256) bitmap_count_kernel(const uint32_t* __restrict__ bitmap, int words,
                                                           int64_t rows, int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;                                   // whole wavefronts
  uint32_t c = 0;
  for (int x = lane; x < words; x += 64) c += __popc(bitmap[r * words + x]);
  c = wave_reduce(c, lane, [](uint32_t a, uint32_t b) { return a + b; });
  if (lane == 0) counts[r] = (int32_t)c;
}

// The entries a screened cut left inside its margin, ranked on their exact float64
// logits (logit descending, index ascending): one wavefront per row, eight lanes per
// entry (each D / 8 channels), eight entries per pass; the kept ones are added to
// the row's bits.
template <typename T, int D>
__global__ void __launch_bounds__(256) group_rank_kernel(const int32_t* __restrict__ cn, const double2* __restrict__ cab,
                                                         const uint2* __restrict__ cjw, const double* __restrict__ qp,
                                                         const T* __restrict__ k, Geom g, int64_t rows,
                                                         uint32_t* __restrict__ bitmap, int words, double inv_sqrt_d) {
  constexpr int per = D / 8;                 // channels per lane
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;                                   // whole wavefronts
  const uint32_t ncand = (uint32_t)cn[r];
  if (ncand == 0u) return;
  const int64_t bh = r / g.S;
  const int sub = lane & 7, slot = lane >> 3;
  const bool have = (uint32_t)lane < ncand;
  const uint2 mine_jw = cjw[r * kMaxCand + min((uint32_t)lane, ncand - 1u)];
  double qv[per];
#pragma unroll
  for (int e = 0; e < per; e += 2) {
    const double2 x = *(const double2*)(qp + (size_t)r * D + sub * per + e);
    qv[e] = x.x;
    qv[e + 1] = x.y;
  }
  double z = 0.0;
  for (int p = 0; p < (int)((ncand + 7u) / 8u); ++p) {
    const uint32_t cidx = min(8u * (uint32_t)p + (uint32_t)slot, ncand - 1u);
    const int cj = __shfl((int)mine_jw.x, (int)cidx, 64);
    double mk[per];
    group_mean<T, per>(k, g, bh, cj, sub * per, mk);
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < per; ++e) part = fma(qv[e], mk[e], part);
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
  if (have && at.x + (double)before < at.y) atomicOr(&bitmap[r * words + (my_j >> 5)], 1u << (my_j & 31));
}

}  // namespace gscr

hipError_t launch_pool_groups_screen(const Geom& g, const void* k, const ScreenOps& ops, hipStream_t s) {
  const int ntg = (g.L / 4 + 15) / 16;
  const dim3 grid((unsigned)((ntg + 3) / 4), (unsigned)((int64_t)g.B * g.nh));
  if (g.dtype == 1 && g.D == 64)
    gscr::pool_groups_screen_kernel<uint16_t, 64><<<grid, 256, 0, s>>>((const uint16_t*)k, ops, g);
  else if (g.dtype == 1)
    gscr::pool_groups_screen_kernel<uint16_t, 128><<<grid, 256, 0, s>>>((const uint16_t*)k, ops, g);
  else if (g.D == 64)
    gscr::pool_groups_screen_kernel<float, 64><<<grid, 256, 0, s>>>((const float*)k, ops, g);
  else
    gscr::pool_groups_screen_kernel<float, 128><<<grid, 256, 0, s>>>((const float*)k, ops, g);
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
    gscr::group_logits_screen_kernel<64><<<grid, gscr::kMapWaves * 64, 0, s>>>(ops, zt, g, h0, per, pitch, inv);
  else
    gscr::group_logits_screen_kernel<128><<<grid, gscr::kMapWaves * 64, 0, s>>>(ops, zt, g, h0, per, pitch, inv);
  return hipGetLastError();
}

hipError_t launch_group_screen_select(const Geom& g, const float* zt, int pitch, const ScreenOps& ops, int64_t row0,
                                      int64_t nrows, double thr, int win_t, int win_h, int win_w, uint32_t* bitmap,
                                      int words, int32_t* flag_list, int32_t* nflag, const GroupRankBufs& rb,
                                      hipStream_t s) {
  const double inv = 1.0 / sqrt((double)g.D);
  gscr::group_screen_select_kernel<<<(unsigned)nrows, gscr::kNT, 0, s>>>(zt, pitch, ops, row0, g, thr, win_t, win_h,
                                                                         win_w, bitmap, words, flag_list, nflag, rb.cn,
                                                                         rb.cab, rb.cjw, inv);
  return hipGetLastError();
}

hipError_t launch_group_rank(const Geom& g, const GroupRankBufs& rb, const double* qp, const void* k,
                             uint32_t* bitmap, int words, hipStream_t s) {
  const double inv = 1.0 / sqrt((double)g.D);
  const unsigned grid = (unsigned)((g.rows + 3) / 4);
#define BSA_RANK(T_, D_)                                                                                        \
  gscr::group_rank_kernel<T_, D_><<<grid, 256, 0, s>>>(rb.cn, rb.cab, rb.cjw, qp, (const T_*)k, g, g.rows, bitmap, \
                                                       words, inv)
  if (g.dtype == 1 && g.D == 64) BSA_RANK(uint16_t, 64);
  else if (g.dtype == 1) BSA_RANK(uint16_t, 128);
  else if (g.D == 64) BSA_RANK(float, 64);
  else BSA_RANK(float, 128);
#undef BSA_RANK
  return hipGetLastError();
}

hipError_t launch_bitmap_counts(const uint32_t* bitmap, int words, int64_t rows, int32_t* counts, hipStream_t s) {
  gscr::bitmap_count_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, s>>>(bitmap, words, rows, counts);
  return hipGetLastError();
}

}  // namespace bsa
