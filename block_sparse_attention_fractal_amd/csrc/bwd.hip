// Backward of the block-sparse attention, for training with the mask (NABLA
// page, gist.science/es/paper/2507.13546, Metodologia item 2, "Expansion": the
// attention runs on the kept N x N tiles only, and so does its gradient).
//
//   P = softmax over the kept keys of z = q.k / sqrt(D)   (recomputed from lse)
//   dV_k = sum_n P[n,k] dO_n          dP[n,k] = dO_n . v_k
//   dZ[n,k] = P[n,k] (dP[n,k] - Delta_n),   Delta_n = sum_k P[n,k] dP[n,k]
//   dQ_n = sum_k dZ[n,k] k_k / sqrt(D)      dK_k = sum_n dZ[n,k] q_n / sqrt(D)
//
// The row term Delta is formed here from the very P and dP values the dQ pass
// uses (Delta = sum P dP / sum P over the query's kept keys), not as dO . o from
// a stored output: the dZ of one query then sum to zero up to float32 rounding,
// so a component common to every key (the positional term of the video tokens)
// cancels from dQ.  A rounded output in the row term breaks that sum and leaks
// the common component into dQ at the percent level.
//
// Three passes, no atomics on the gradients (deterministic):
//   * Delta: query-major over the CSR, the dQ pass's walk and products without
//     the dQ product (S^T = K Q^T and dP^T = V dO^T), sums per query -- or, for
//     the training pair, Delta = dO . (o + o_lo) from the training forward's
//     output pair (O to ~2^-16 with P fed to its PV product as a bf16 pair), whose
//     error against sum P dP / sum P is far below what the dQ cancellation
//     amplifies into a visible error;
//   * dQ: query-major over the CSR, a pair of query blocks per workgroup (the
//     forward kernel's schedule): S^T = K Q^T and dP^T = V dO^T with the
//     32x32x16 bf16 MFMA (each lane holds 32 keys of one query), dZ^T in
//     registers, then dQ^T += K^T dZ^T with K^T read from the natural K tile by
//     transposing LDS reads;
//   * dK, dV: key-major over the transposed mask (built here: a bitmap per key
//     block, counted, scanned and compacted), a pair of key blocks per
//     workgroup of producer and consumer waves: S = Q K^T and dP = dO V^T with
//     the key fragments in registers (each lane holds 32 queries of one key),
//     then dV^T += dO^T P and dK^T += Q^T dZ with Q^T and dO^T read from the
//     natural tiles by transposing LDS reads.
// float32 tensors take two plain kernels with float64 arithmetic (accuracy
// rather than speed, as in the forward's float32 path); their dQ kernel forms
// Delta the same way in a first walk over the row.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "bsa.h"
#include "kernels.h"

namespace bsa {
namespace bwd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kD = 128;
constexpr int kTile = 16384;          // one 64 x 128 bf16 tile (natural or transposed)

// natural tile (64 rows x 256 B), chunk c of row r at c ^ (r & 15)
__device__ __forceinline__ int nat_lds(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
// transposed tile (128 rows x 128 B), chunk c of row d at c ^ ((d >> 1) & 7)
__device__ __forceinline__ int tr_lds(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

struct Args {
  const uint16_t* q;       // natural [B*nh, L, D] (tensor layout)
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  float2* ld;              // per token: (lse * log2 e, Delta); Delta written by the Delta pass
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const int32_t* ptr;      // CSR (dQ pass) or transposed CSR (dK/dV pass)
  const int32_t* idx;
  int32_t* counters;       // 8 per-XCD item counters
  const int32_t* order;    // items in processing order: XCD x takes order[bounds[x] .. bounds[x+1])
  const int32_t* bounds;   // 9 entries
  Geom g;
  float c_log2;            // log2(e) / sqrt(D)
  float inv_sqrt_d;
  int32_t pairs, items;
};

// first token row of block j in the tensor's own layout (rs*(m/8) + m%8 further for token m)
__device__ __forceinline__ int block_base_row(const Geom& g, int j) {
  if (g.layout == 1) return j * 64;
  const int px = j % g.Wp;
  const int rest = j / g.Wp;
  const int py = rest % g.Hp;
  const int t = rest / g.Hp;
  return (t * g.H + py * 8) * g.W + px * 8;
}

// Union walk over the ascending lists of rows r0 and r0+1 (wave-uniform).  Each
// list is read through a 64-entry window held one entry per lane.
struct PairWalk {
  int pa, ea, pb, eb, wa_base, wb_base, wa, wb;
  __device__ __forceinline__ void init(const Args& a, int64_t r0, bool two, int lane) {
    pa = a.ptr[r0];
    ea = a.ptr[r0 + 1];
    pb = two ? a.ptr[r0 + 1] : 0;
    eb = two ? a.ptr[r0 + 2] : 0;
    wa_base = pa;
    wb_base = pb;
    wa = wa_base + lane < ea ? a.idx[wa_base + lane] : 0x7fffffff;
    wb = wb_base + lane < eb ? a.idx[wb_base + lane] : 0x7fffffff;
  }
  __device__ __forceinline__ int peek(const Args& a, int& p, int e, int& base, int& w, int lane) {
    if (p >= e) return 0x7fffffff;
    if (p - base >= 64) {
      base = p;
      w = base + lane < e ? a.idx[base + lane] : 0x7fffffff;
    }
    return __builtin_amdgcn_readlane(w, p - base);
  }
  __device__ __forceinline__ void next(const Args& a, int lane, int& j, bool& ka, bool& kb) {
    const int ja = peek(a, pa, ea, wa_base, wa, lane);
    const int jb = peek(a, pb, eb, wb_base, wb, lane);
    j = min(ja, jb);
    ka = ja == j;
    kb = jb == j;
    pa += ka;
    pb += kb;
  }
};

// Stores a pair of 64 x 128 bf16 blocks from the transposed accumulators of
// four waves (wave w: block w >> 1, columns 32 (w & 1) .. +31), through LDS.
// Every thread of the workgroup calls it (two barriers); `valid` threads stage
// their accumulators, and the 256 threads with `stores` (index tid among them)
// write the blocks out.
__device__ __forceinline__ void store_pair(uint8_t* stage, const f32x16 (&acc)[4], float mul, bool valid, int wave,
                                           int lane, int tid, const Geom& g, int i0, bool two, uint16_t* out_head,
                                           bool stores = true) {
  const int h = lane >> 5, l32 = lane & 31;
  const int blk = wave >> 1, col = 32 * (wave & 1) + l32;   // col = token of the block
  __syncthreads();
  if (valid) {
    uint8_t* ob = stage + blk * 16384;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int unit = 8 * u + 2 * rq + h;
        uint2 w;
        w.x = pack_bf16x2(acc[u][4 * rq + 0] * mul, acc[u][4 * rq + 1] * mul);
        w.y = pack_bf16x2(acc[u][4 * rq + 2] * mul, acc[u][4 * rq + 3] * mul);
        *(uint2*)(ob + col * 256 + ((unit ^ (col & 31)) << 3)) = w;
      }
    }
  }
  __syncthreads();
  const int sb = tid >> 7;
  if (stores && (sb == 0 || two)) {
    const int rs = g.layout == 1 ? 8 : g.W;
    const int t7 = tid & 127;
    const int lchunk = t7 & 15;
    const int base = block_base_row(g, i0 + sb);
    const uint8_t* ob = stage + sb * 16384;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = (t7 >> 4) + 8 * u;
      const uint2 lo = *(const uint2*)(ob + row * 256 + (((2 * lchunk) ^ (row & 31)) << 3));
      const uint2 hi = *(const uint2*)(ob + row * 256 + (((2 * lchunk + 1) ^ (row & 31)) << 3));
      const int tok = base + (row >> 3) * rs + (row & 7);
      *(uint4*)(out_head + (size_t)tok * kD + lchunk * 8) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
}

// ---------------------------------------------------------------------------
// dQ pass (bf16).  Stage: natural K | natural V, 32 KB; two stages; two
// workgroups per CU (249 VGPRs).  The K^T operand of the dQ product comes from
// the natural K tile through gfx950's transposing LDS reads.
// kDelta: the Delta pass -- the same walk, loads and S / dP products, but only
// sum P and sum P dP per query are kept, and Delta = sum P dP / sum P is stored
// (P computed by the same instructions as in the dQ pass, so both passes see
// bit-identical P and dP).
// ---------------------------------------------------------------------------
template <bool kDelta>
__global__ void __launch_bounds__(256, 2) dq_bf16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem_dq[4 * kTile];
  uint8_t* const stage0 = smem_dq;
  uint8_t* const stage1 = smem_dq + 2 * kTile;
  __shared__ int s_item;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int qb = wave >> 1, wq = wave & 1;
  const Geom g = a.g;
  const int rs = g.layout == 1 ? 8 : g.W;
  const float c_log2 = a.c_log2;

  int noff[4];                       // per-lane byte offsets of the 16-byte chunks this thread loads
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int c = (4 * wave + u) * 64 + lane;
    const int m = c >> 4;
    const int lc = (lane & 15) ^ (m & 15);
    noff[u] = (((m >> 3) * rs + (m & 7)) * kD + lc * 8) * 2;
  }
  // byte offset in the natural K tile of this lane's transposing read for k-step s,
  // channel tile u, read r2 (keys 16s + 4h + 0..3, or + 8): row 16s + 8r2 + 4h + j/4,
  // 16-byte chunk 4u + c0 swizzled by the row's low 4 bits.  Those bits are
  // 8r2 + 4h + j/4, so the swizzled chunk is 4(u ^ (2r2 + h)) + (c0 ^ j/4): four
  // per-lane bases (one per u ^ h) plus immediates cover all 32 reads of a tile.
  int trp[4];
  {
    const int trj = lane & 15, trg = lane >> 4, hh = trg >> 1;
    const int c0 = 2 * (trg & 1) + ((trj & 3) >> 1);
    const int b0 = (4 * hh + (trj >> 2)) * 256 + 16 * (c0 ^ (trj >> 2)) + 8 * (trj & 1);
#pragma unroll
    for (int x = 0; x < 4; ++x) trp[x] = b0 + 64 * (x ^ hh);
  }
  auto tr_off = [&](int u, int s, int r2) { return trp[u ^ (2 * r2)] + 2048 * r2 + 4096 * s; };
  const int xcd = blockIdx.x & 7;
  const int lo_t = a.bounds[xcd], hi_t = a.bounds[xcd + 1];   // this XCD's stretch of the work order

  for (;;) {
    if (tid == 0) s_item = lo_t + atomicAdd(&a.counters[xcd], 1);
    __syncthreads();
    const int idx = __builtin_amdgcn_readfirstlane(s_item);
    if (idx >= hi_t) break;
    const int64_t item = a.order[idx];
    const int64_t bh = item / a.pairs;
    const int i0 = 2 * (int)(item - bh * a.pairs);
    const int64_t r0 = bh * g.S + i0;
    const bool two = i0 + 1 < g.S;
    const bool has_q = qb == 0 || two;
    PairWalk wk;
    wk.init(a, r0, two, lane);

    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + (size_t)bh * g.L * kD), (short)0, g.L * kD * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + (size_t)bh * g.L * kD), (short)0, g.L * kD * 2, 0x00020000);
    auto issue = [&](int j, uint8_t* st) {
      const int jc = min(max(j, 0), g.S - 1);
      const int ns = block_base_row(g, jc) * kD * 2;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int slot = (4 * wave + u) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(st + slot), 16, noff[u], ns, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(st + kTile + slot), 16, noff[u], ns, 0, 0);
      }
    };

    bf16x8 qreg[8], doreg[8];
    float lse2 = 0.f, dlt = 0.f;
    float sum_p = 0.f, sum_pdp = 0.f;   // Delta pass: per-lane partial sums
    const int qtok = block_base_row(g, min(i0 + qb, g.S - 1)) + ((32 * wq + l32) >> 3) * rs + (l32 & 7);
    if (has_q) {
      const uint16_t* qrow = a.q + ((size_t)bh * g.L + qtok) * kD + 8 * h;
      const uint16_t* drow = a.dout + ((size_t)bh * g.L + qtok) * kD + 8 * h;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        qreg[s] = *(const bf16x8*)(qrow + 16 * s);
        doreg[s] = *(const bf16x8*)(drow + 16 * s);
      }
      const float2 ld = a.ld[(size_t)bh * g.L + qtok];
      lse2 = ld.x;
      if (!kDelta) dlt = ld.y;
    }
    f32x16 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[u][e] = 0.f;

    int j;
    bool ka, kb;
    wk.next(a, lane, j, ka, kb);
    if (j != 0x7fffffff) issue(j, stage0);
    auto step = [&](uint8_t* st, uint8_t* other) {
      int jn;
      bool kan, kbn;
      wk.next(a, lane, jn, kan, kbn);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (jn != 0x7fffffff) issue(jn, other);
      const bool mine = qb == 0 ? ka : kb;
      if (mine) {
        // one 32-key half of the tile at a time keeps only one S / dP pair live
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          f32x16 sacc, pacc;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            sacc[e] = 0.f;
            pacc[e] = 0.f;
          }
#pragma unroll
          for (int s0 = 0; s0 < 8; s0 += 4) {
            bf16x8 ak[4], av[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              ak[s] = *(const bf16x8*)(st + nat_lds(32 * t + l32, 2 * (s0 + s) + h));
              av[s] = *(const bf16x8*)(st + kTile + nat_lds(32 * t + l32, 2 * (s0 + s) + h));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[s], qreg[s0 + s], sacc, 0, 0, 0);
              pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[s], doreg[s0 + s], pacc, 0, 0, 0);
            }
          }
          if constexpr (kDelta) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], c_log2, -lse2));
              sum_p += p;
              sum_pdp = fmaf(p, pacc[e], sum_pdp);
            }
          } else {
            // dZ = hi + lo, two bf16 terms: the dZ of one query sum to zero, so dQ is a
            // small difference of large terms when K has a large common part, and a
            // single bf16 rounding of dZ (2^-9) would show in it at the percent level.
            bf16x8 dsh[2], dsl[2];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], c_log2, -lse2));
              const float ds = p * (pacc[e] - dlt);
              const __bf16 hi = (__bf16)ds;
              dsh[e >> 3][e & 7] = hi;
              dsl[e >> 3][e & 7] = (__bf16)(ds - (float)hi);
            }
            // K^T operand straight from the natural K tile with transposing LDS reads:
            // in each 16-lane group, source lane j reads keys-row kbase + j/4 at channels
            // dbase + 4(j%4) .. +3 and lane i receives keys kbase .. kbase+3 of channel
            // dbase + i; two reads give the 8 keys of a lane's operand
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const int s = 2 * t + s2;
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + tr_off(u, s, 0)));
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + tr_off(u, s, 1)));
                const bf16x8 at =
                    __builtin_bit_cast(bf16x8, (v8i16){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
                acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, dsh[s2], acc[u], 0, 0, 0);
                acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, dsl[s2], acc[u], 0, 0, 0);
              }
            }
          }
        }
      }
      j = jn;
      ka = kan;
      kb = kbn;
    };
    while (j != 0x7fffffff) {
      step(stage0, stage1);
      if (j == 0x7fffffff) break;
      step(stage1, stage0);
    }
    if constexpr (kDelta) {
      // lanes l32 and l32 + 32 hold complementary keys of the same query
      sum_p += __shfl_xor(sum_p, 32);
      sum_pdp += __shfl_xor(sum_pdp, 32);
      if (has_q && h == 0) a.ld[(size_t)bh * g.L + qtok].y = sum_pdp / sum_p;
    } else {
      store_pair(stage0, acc, a.inv_sqrt_d, has_q, wave, lane, tid, g, i0, two, a.dq + (size_t)bh * g.L * kD);
    }
  }
}

// ---------------------------------------------------------------------------
// dK/dV pass (bf16), producer / consumer form: 512 threads, waves 0-3 produce
// and waves 4-7 consume; waves w and w + 4 own the same 32 keys (key block
// (w & 3) >> 1 of the pair, keys 32 (w & 1) .. +31).  In phase n the producers
// compute S = Q K^T, dP = dO V^T (K, V fragments in registers), P and dZ of
// tile n+1 while the consumers accumulate dV^T += dO^T P and dK^T += Q^T dZ of
// tile n, with P and dZ handed over through LDS in the consumers' operand
// layout and Q^T, dO^T read from the natural tiles by transposing LDS reads.
// Two waves per SIMD (one of each role) where the four-wave kernel had one, so
// one wave's exponentials overlap the other's matrix products.  LDS: three
// stages of natural Q | natural dO | (lse2, Delta) (tile n for the consumers,
// n+1 for the producers, n+2 in flight) and the 32 KB hand-over buffer.  The
// roles run separate loops (so the compiler never keeps both roles' registers
// live) with the same barriers: two per phase.
// ---------------------------------------------------------------------------
constexpr int kStagePC = 2 * kTile + 512;
constexpr int kLdOffPC = 2 * kTile;
constexpr int kHandOff = 3 * kStagePC;             // 4 producers x 8 KB
constexpr int kLdsPC = kHandOff + 4 * 8192;

__global__ void __launch_bounds__(512, 1) dkdv_pc_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem_pc[kLdsPC];
  __shared__ int s_item;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int w4 = wave & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const int kbk = w4 >> 1, wkk = w4 & 1;     // key block of the pair, which 32 keys of it
  const Geom g = a.g;
  const int rs = g.layout == 1 ? 8 : g.W;
  const float c_log2 = a.c_log2;
  const int xcd = blockIdx.x & 7;
  const int lo_t = a.bounds[xcd], hi_t = a.bounds[xcd + 1];   // this XCD's stretch of the work order

  int noff[2];                       // this thread's two 16-byte chunks of each natural tile
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = (2 * wave + u) * 64 + lane;
    const int m = c >> 4;
    noff[u] = (((m >> 3) * rs + (m & 7)) * kD + (((lane & 15) ^ (m & 15)) * 8)) * 2;
  }
  const int ldm = 2 * (lane & 31);   // (lse2, Delta) of the 64 queries: 32 chunks of 2 tokens, wave 0
  const int ldoff = (((ldm >> 3) * rs + (ldm & 7))) * 8;
  // transposing reads (as in the dQ pass, rows = queries here): byte offset in the
  // natural tile of this lane's read for query step s, channel tile u, read r2
  int trp[4];
  {
    const int trj = lane & 15, trg = lane >> 4, hh = trg >> 1;
    const int c0 = 2 * (trg & 1) + ((trj & 3) >> 1);
    const int b0 = (4 * hh + (trj >> 2)) * 256 + 16 * (c0 ^ (trj >> 2)) + 8 * (trj & 1);
#pragma unroll
    for (int x = 0; x < 4; ++x) trp[x] = b0 + 64 * (x ^ hh);
  }
  auto tr_off = [&](int u, int s, int r2) { return trp[u ^ (2 * r2)] + 2048 * r2 + 4096 * s; };
  uint8_t* const hand = smem_pc + kHandOff + w4 * 8192;   // this key slice's P / dZ hand-over
  auto hand_off = [&](int s, int which) { return ((2 * s + which) * 64 + lane) * 16; };

  // item prologue shared by both roles: claim, walk, resources
  struct Item {
    int64_t bh;
    int j0;
    bool two;
  };
  auto claim = [&](Item& it) -> bool {
    if (tid == 0) s_item = lo_t + atomicAdd(&a.counters[xcd], 1);
    __syncthreads();
    const int idx = __builtin_amdgcn_readfirstlane(s_item);
    if (idx >= hi_t) return false;
    const int64_t item = a.order[idx];
    it.bh = item / a.pairs;
    it.j0 = 2 * (int)(item - it.bh * a.pairs);
    it.two = it.j0 + 1 < g.S;
    return true;
  };
  auto issue = [&](const Item& it, int i, int slot) {
    const size_t hoff = (size_t)it.bh * g.L * kD;
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + hoff), (short)0, g.L * kD * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t drs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.dout + hoff), (short)0, g.L * kD * 2, 0x00020000);
    uint8_t* st = smem_pc + slot * kStagePC;
    const int ic = min(max(i, 0), g.S - 1);
    const int base = block_base_row(g, ic);
    const int ns = base * kD * 2;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int sl = (2 * wave + u) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (lds_void*)(st + sl), 16, noff[u], ns, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (lds_void*)(st + kTile + sl), 16, noff[u], ns, 0, 0);
    }
    if (wave == 0 && lane < 32) {
      const __amdgpu_buffer_rsrc_t lrs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(a.ld + (size_t)it.bh * g.L), (short)0, g.L * 8, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (lds_void*)(st + kLdOffPC), 16, ldoff, base * 8, 0, 0);
    }
  };

  if (wave < 4) {
    // ---- producers ----
    Item it;
    while (claim(it)) {
      const int64_t r0 = it.bh * g.S + it.j0;
      const bool has_k = kbk == 0 || it.two;
      PairWalk wk;
      wk.init(a, r0, it.two, lane);
      bf16x8 kreg[8], vreg[8];
      if (has_k) {
        const int ktok = block_base_row(g, it.j0 + kbk) + ((32 * wkk + l32) >> 3) * rs + (l32 & 7);
        const uint16_t* krow = a.k + ((size_t)it.bh * g.L + ktok) * kD + 8 * h;
        const uint16_t* vrow = a.v + ((size_t)it.bh * g.L + ktok) * kD + 8 * h;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          kreg[s] = *(const bf16x8*)(krow + 16 * s);
          vreg[s] = *(const bf16x8*)(vrow + 16 * s);
        }
      }
      bf16x8 pb[4], db[4];
      // P and dZ of the tile in `slot` (this wave's 32 keys x 64 queries) into pb, db
      auto produce = [&](int slot) {
        const uint8_t* st = smem_pc + slot * kStagePC;
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            sacc[t][e] = 0.f;
            pacc[t][e] = 0.f;
          }
          bf16x8 aq[8], ad[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            aq[s] = *(const bf16x8*)(st + nat_lds(32 * t + l32, 2 * s + h));
            ad[s] = *(const bf16x8*)(st + kTile + nat_lds(32 * t + l32, 2 * s + h));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[s], kreg[s], sacc[t], 0, 0, 0);
            pacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad[s], vreg[s], pacc[t], 0, 0, 0);
          }
        }
        // accumulator register e of tile t holds query 32t + 8(e/4) + 4h + e%4
        const float2* ldt = (const float2*)(st + kLdOffPC);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float2 ld = ldt[32 * t + 8 * (e >> 2) + 4 * h + (e & 3)];
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][e], c_log2, -ld.x));
            pb[2 * t + (e >> 3)][e & 7] = (__bf16)p;
            db[2 * t + (e >> 3)][e & 7] = (__bf16)(p * (pacc[t][e] - ld.y));
          }
        }
      };
      auto hand_over = [&]() {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          *(bf16x8*)(hand + hand_off(s, 0)) = pb[s];
          *(bf16x8*)(hand + hand_off(s, 1)) = db[s];
        }
      };
      int i0t, i1t;
      bool ka0, kb0, ka1, kb1;
      wk.next(a, lane, i0t, ka0, kb0);
      wk.next(a, lane, i1t, ka1, kb1);
      if (i0t != 0x7fffffff) issue(it, i0t, 0);
      if (i1t != 0x7fffffff) issue(it, i1t, 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const bool mine0 = kbk == 0 ? ka0 : kb0;
      if (i0t != 0x7fffffff && mine0) {
        produce(0);
        hand_over();
      }
      __syncthreads();
      // phase loop: the consumers take tile `cur` (slot cs), the producers tile `nxt`
      int cur = i0t, nxt = i1t;
      bool kan = ka1, kbn = kb1;
      int cs = 0;
      while (cur != 0x7fffffff) {
        int i2t;
        bool ka2, kb2;
        wk.next(a, lane, i2t, ka2, kb2);
        const int ns = cs == 2 ? 0 : cs + 1, ns2 = ns == 2 ? 0 : ns + 1;
        if (i2t != 0x7fffffff) issue(it, i2t, ns2);
        const bool mine = nxt != 0x7fffffff && (kbk == 0 ? kan : kbn);
        if (mine) produce(ns);
        __syncthreads();                 // the consumers have read tile cur's hand-over
        if (mine) hand_over();
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // tile i2t landed
        __syncthreads();
        cur = nxt;
        nxt = i2t;
        kan = ka2;
        kbn = kb2;
        cs = ns;
      }
      f32x16 none[4];
      store_pair(smem_pc, none, 1.f, false, w4, lane, tid, g, it.j0, it.two, a.dv + (size_t)it.bh * g.L * kD, false);
      store_pair(smem_pc, none, 1.f, false, w4, lane, tid, g, it.j0, it.two, a.dk + (size_t)it.bh * g.L * kD, false);
    }
  } else {
    // ---- consumers ----
    Item it;
    while (claim(it)) {
      const int64_t r0 = it.bh * g.S + it.j0;
      const bool has_k = kbk == 0 || it.two;
      PairWalk wk;
      wk.init(a, r0, it.two, lane);
      f32x16 dka[4], dva[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          dka[u][e] = 0.f;
          dva[u][e] = 0.f;
        }
      int i0t, i1t;
      bool ka0, kb0, ka1, kb1;
      wk.next(a, lane, i0t, ka0, kb0);
      wk.next(a, lane, i1t, ka1, kb1);
      if (i0t != 0x7fffffff) issue(it, i0t, 0);
      if (i1t != 0x7fffffff) issue(it, i1t, 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      __syncthreads();                   // the producers hand over tile i0t
      int cur = i0t, nxt = i1t;
      bool kac = ka0, kbc = kb0, kan = ka1, kbn = kb1;
      int cs = 0;
      while (cur != 0x7fffffff) {
        int i2t;
        bool ka2, kb2;
        wk.next(a, lane, i2t, ka2, kb2);
        const int ns = cs == 2 ? 0 : cs + 1, ns2 = ns == 2 ? 0 : ns + 1;
        if (i2t != 0x7fffffff) issue(it, i2t, ns2);
        if (kbk == 0 ? kac : kbc) {
          const uint8_t* st = smem_pc + cs * kStagePC;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 pbs = *(const bf16x8*)(hand + hand_off(s, 0));
            const bf16x8 dbs = *(const bf16x8*)(hand + hand_off(s, 1));
            bf16x8 adt[4], aqt[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const v4i16 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + kTile + tr_off(u, s, 0)));
              const v4i16 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + kTile + tr_off(u, s, 1)));
              adt[u] = __builtin_bit_cast(bf16x8, (v8i16){dlo[0], dlo[1], dlo[2], dlo[3], dhi[0], dhi[1], dhi[2], dhi[3]});
              const v4i16 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + tr_off(u, s, 0)));
              const v4i16 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(st + tr_off(u, s, 1)));
              aqt[u] = __builtin_bit_cast(bf16x8, (v8i16){qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]});
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              dva[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(adt[u], pbs, dva[u], 0, 0, 0);
              dka[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aqt[u], dbs, dka[u], 0, 0, 0);
            }
          }
        }
        __syncthreads();                 // tile cur's hand-over read
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // tile i2t landed
        __syncthreads();                 // tile nxt handed over
        cur = nxt;
        nxt = i2t;
        kac = kan;
        kbc = kbn;
        kan = ka2;
        kbn = kb2;
        cs = ns;
      }
      (void)nxt;
      store_pair(smem_pc, dva, 1.f, has_k, w4, lane, tid - 256, g, it.j0, it.two, a.dv + (size_t)it.bh * g.L * kD);
      store_pair(smem_pc, dka, a.inv_sqrt_d, has_k, w4, lane, tid - 256, g, it.j0, it.two,
                 a.dk + (size_t)it.bh * g.L * kD);
    }
  }
}

// ---------------------------------------------------------------------------
// float32 tensors: plain kernels, float64 arithmetic, one workgroup per row of
// the (transposed) mask; head_dim 64 or 128.
// ---------------------------------------------------------------------------
// The query/key rows a thread works on live in LDS (not registers): at D = 128
// they would not fit; dZ is kept in float64 at D = 64 and float32 at D = 128 so
// that the four 64 x D tiles plus dZ stay within the 160 KB of LDS.
template <int D>
using ZT = typename std::conditional<D == 64, double, float>::type;

template <int D>
__global__ void __launch_bounds__(256) dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                     const float* __restrict__ v, const float* __restrict__ dout,
                                                     float2* __restrict__ ld, float* __restrict__ dq,
                                                     const int32_t* __restrict__ ptr, const int32_t* __restrict__ idx,
                                                     Geom g, double scale) {
  constexpr int DS = D / 4;
  __shared__ float Qs[64][D + 1];
  __shared__ float Os[64][D + 1];       // dO rows of the query block
  __shared__ float Ks[64][D + 1];
  __shared__ float Vs[64][D + 1];
  __shared__ ZT<D> Zs[64][65];
  const int64_t r = blockIdx.x;
  const int64_t bh = r / g.S;
  const int i = (int)(r - bh * g.S);
  const int tid = threadIdx.x, qi = tid >> 2, sl = tid & 3;
  const size_t hoff = (size_t)bh * g.L * D;
  const int qtok = block_token_row(g, i, qi);
  for (int e = tid; e < 64 * D; e += 256) {
    const int row = e / D, d = e % D;
    const size_t off = hoff + (size_t)block_token_row(g, i, row) * D + d;
    Qs[row][d] = q[off];
    Os[row][d] = dout[off];
  }
  const double lse = (double)ld[(size_t)bh * g.L + qtok].x * 0.69314718055994530942;
  // Delta = sum P dP / sum P over the row's keys, from the P and dP the main walk
  // recomputes below (thread (qi, sl) sums keys sl, sl + 4, ...; the four slices
  // of a query are neighbouring lanes)
  double sp = 0.0, spd = 0.0;
  for (int it = ptr[r]; it < ptr[r + 1]; ++it) {
    const int j = min(max(idx[it], 0), g.S - 1);
    __syncthreads();
    for (int e = tid; e < 64 * D; e += 256) {
      const int row = e / D, d = e % D;
      const size_t off = hoff + (size_t)block_token_row(g, j, row) * D + d;
      Ks[row][d] = k[off];
      Vs[row][d] = v[off];
    }
    __syncthreads();
    for (int c = 0; c < 16; ++c) {
      const int kk = sl + 4 * c;
      double s = 0.0, dp = 0.0;
      for (int d = 0; d < D; ++d) {
        s = __fma_rn((double)Qs[qi][d], (double)Ks[kk][d], s);
        dp = __fma_rn((double)Os[qi][d], (double)Vs[kk][d], dp);
      }
      const double p = exp(s * scale - lse);
      sp += p;
      spd = __fma_rn(p, dp, spd);
    }
  }
  sp += __shfl_xor(sp, 1, 4);
  sp += __shfl_xor(sp, 2, 4);
  spd += __shfl_xor(spd, 1, 4);
  spd += __shfl_xor(spd, 2, 4);
  const double dlt = spd / sp;
  if (sl == 0) ld[(size_t)bh * g.L + qtok].y = (float)dlt;   // for the dK/dV kernel
  double acc[DS];
#pragma unroll
  for (int d = 0; d < DS; ++d) acc[d] = 0.0;
  for (int it = ptr[r]; it < ptr[r + 1]; ++it) {
    const int j = min(max(idx[it], 0), g.S - 1);
    __syncthreads();
    for (int e = tid; e < 64 * D; e += 256) {
      const int row = e / D, d = e % D;
      const size_t off = hoff + (size_t)block_token_row(g, j, row) * D + d;
      Ks[row][d] = k[off];
      Vs[row][d] = v[off];
    }
    __syncthreads();
    for (int c = 0; c < 16; ++c) {
      const int kk = sl + 4 * c;
      double s = 0.0, dp = 0.0;
      for (int d = 0; d < D; ++d) {
        s = __fma_rn((double)Qs[qi][d], (double)Ks[kk][d], s);
        dp = __fma_rn((double)Os[qi][d], (double)Vs[kk][d], dp);
      }
      const double p = exp(s * scale - lse);
      Zs[qi][kk] = (ZT<D>)(p * (dp - dlt));
    }
    __syncthreads();
    for (int kk = 0; kk < 64; ++kk) {
      const double z = Zs[qi][kk];
#pragma unroll 8
      for (int d = 0; d < DS; ++d) acc[d] = __fma_rn(z, (double)Ks[kk][sl * DS + d], acc[d]);
    }
  }
#pragma unroll
  for (int d = 0; d < DS; ++d) dq[hoff + (size_t)qtok * D + sl * DS + d] = (float)(acc[d] * scale);
}

template <int D>
__global__ void __launch_bounds__(256) dkdv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, const float* __restrict__ dout,
                                                       const float2* __restrict__ ld, float* __restrict__ dk,
                                                       float* __restrict__ dv, const int32_t* __restrict__ ptr,
                                                       const int32_t* __restrict__ idx, Geom g, double scale) {
  constexpr int DS = D / 4;
  __shared__ float Ks[64][D + 1];
  __shared__ float Vs[64][D + 1];
  __shared__ float Qs[64][D + 1];
  __shared__ float Os[64][D + 1];       // dO rows of the query block
  __shared__ double Ls[64][2];
  const int64_t r = blockIdx.x;              // transposed row: key block j of head bh
  const int64_t bh = r / g.S;
  const int j = (int)(r - bh * g.S);
  const int tid = threadIdx.x, ki = tid >> 2, sl = tid & 3;
  const size_t hoff = (size_t)bh * g.L * D;
  const int ktok = block_token_row(g, j, ki);
  for (int e = tid; e < 64 * D; e += 256) {
    const int row = e / D, d = e % D;
    const size_t off = hoff + (size_t)block_token_row(g, j, row) * D + d;
    Ks[row][d] = k[off];
    Vs[row][d] = v[off];
  }
  double dka[DS], dva[DS];
#pragma unroll
  for (int d = 0; d < DS; ++d) {
    dka[d] = 0.0;
    dva[d] = 0.0;
  }
  for (int it = ptr[r]; it < ptr[r + 1]; ++it) {
    const int i = min(max(idx[it], 0), g.S - 1);
    __syncthreads();
    for (int e = tid; e < 64 * D; e += 256) {
      const int row = e / D, d = e % D;
      const size_t off = hoff + (size_t)block_token_row(g, i, row) * D + d;
      Qs[row][d] = q[off];
      Os[row][d] = dout[off];
    }
    if (tid < 64) {
      const float2 l = ld[(size_t)bh * g.L + block_token_row(g, i, tid)];
      Ls[tid][0] = (double)l.x * 0.69314718055994530942;
      Ls[tid][1] = l.y;
    }
    __syncthreads();
    // thread (key ki, slice sl): P and dZ of its key against every query (the four
    // slices of a key recompute them; this path is for accuracy, not speed)
    for (int qq = 0; qq < 64; ++qq) {
      double s = 0.0, dp = 0.0;
      for (int d = 0; d < D; ++d) {
        s = __fma_rn((double)Qs[qq][d], (double)Ks[ki][d], s);
        dp = __fma_rn((double)Os[qq][d], (double)Vs[ki][d], dp);
      }
      const double p = exp(s * scale - Ls[qq][0]);
      const double z = p * (dp - Ls[qq][1]);
#pragma unroll 8
      for (int d = 0; d < DS; ++d) {
        dva[d] = __fma_rn(p, (double)Os[qq][sl * DS + d], dva[d]);
        dka[d] = __fma_rn(z, (double)Qs[qq][sl * DS + d], dka[d]);
      }
    }
  }
#pragma unroll
  for (int d = 0; d < DS; ++d) {
    dk[hoff + (size_t)ktok * D + sl * DS + d] = (float)(dka[d] * scale);
    dv[hoff + (size_t)ktok * D + sl * DS + d] = (float)dva[d];
  }
}

// ---------------------------------------------------------------------------
// helpers: per-token lse * log2 e, the transposed mask
// ---------------------------------------------------------------------------
// per token: lse * log2(e) (the Delta half is written by the Delta pass)
__global__ void __launch_bounds__(256) lse2_kernel(const float* __restrict__ lse, float2* __restrict__ ld, int64_t ntok) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row < ntok) ld[row] = make_float2(lse[row] * 1.44269504088896341f, 0.f);
}

__global__ void __launch_bounds__(256) zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) p[x] = 0u;
}

// bit (j, i) of the transposed bitmap for every kept tile (i, j); one wavefront per CSR row
__global__ void __launch_bounds__(256) transpose_bits_kernel(const int32_t* __restrict__ row_ptr,
                                                             const int32_t* __restrict__ col_idx,
                                                             uint32_t* __restrict__ tbits, Geom g, int words) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= g.rows) return;
  const int64_t bh = r / g.S;
  const int i = (int)(r - bh * g.S);
  for (int e = row_ptr[r] + lane; e < row_ptr[r + 1]; e += 64) {
    const int j = min(max(col_idx[e], 0), g.S - 1);
    atomicOr(&tbits[(bh * g.S + j) * words + (i >> 5)], 1u << (i & 31));
  }
}

__global__ void __launch_bounds__(256) popcount_rows_kernel(const uint32_t* __restrict__ bits,
                                                            int32_t* __restrict__ counts, int64_t rows, int words) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  int c = 0;
  for (int x = lane; x < words; x += 64) c += __popc(bits[r * words + x]);
  for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, 64);
  if (lane == 0) counts[r] = c;
}

// Delta = dO . (o + o_lo) per token (float32; products of bf16 values are exact),
// 16 threads per token, eight channels each.
__global__ void __launch_bounds__(256) delta_from_output_kernel(const uint16_t* __restrict__ o,
                                                                const uint16_t* __restrict__ olo,
                                                                const uint16_t* __restrict__ dout,
                                                                float2* __restrict__ ld, int64_t ntok) {
  const int64_t tok = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c8 = threadIdx.x & 15;
  float sum = 0.f;
  if (tok < ntok) {
    const size_t off = (size_t)tok * kD + 8 * c8;
    const uint4 a = *(const uint4*)(o + off), b = *(const uint4*)(olo + off), d = *(const uint4*)(dout + off);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w}, dv[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      sum = fmaf(__uint_as_float(dv[m] << 16), __uint_as_float(av[m] << 16) + __uint_as_float(bv[m] << 16), sum);
      sum = fmaf(__uint_as_float(dv[m] & 0xFFFF0000u),
                 __uint_as_float(av[m] & 0xFFFF0000u) + __uint_as_float(bv[m] & 0xFFFF0000u), sum);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 16);
  if (tok < ntok && c8 == 0) ld[tok].y = sum;
}

}  // namespace bwd

hipError_t launch_delta_from_output(const Geom& g, const void* o, const void* o_lo, const void* dout, float2* ld,
                                   hipStream_t s) {
  const int64_t ntok = (int64_t)g.B * g.nh * g.L;
  bwd::delta_from_output_kernel<<<(unsigned)((ntok + 15) / 16), 256, 0, s>>>(
      (const uint16_t*)o, (const uint16_t*)o_lo, (const uint16_t*)dout, ld, ntok);
  return hipGetLastError();
}

hipError_t launch_backward_prep(const Geom& g, const float* lse, float2* ld, const int32_t* row_ptr,
                                const int32_t* col_idx, uint32_t* tbits, int words, int32_t* tcounts, hipStream_t s) {
  const int64_t ntok = (int64_t)g.B * g.nh * g.L;
  bwd::lse2_kernel<<<(unsigned)((ntok + 255) / 256), 256, 0, s>>>(lse, ld, ntok);
  const int64_t nbits = g.rows * words;
  bwd::zero_u32_kernel<<<(unsigned)std::min<int64_t>((nbits + 255) / 256, 65536), 256, 0, s>>>(tbits, nbits);
  const unsigned rgrid = (unsigned)((g.rows + 3) / 4);
  bwd::transpose_bits_kernel<<<rgrid, 256, 0, s>>>(row_ptr, col_idx, tbits, g, words);
  bwd::popcount_rows_kernel<<<rgrid, 256, 0, s>>>(tbits, tcounts, g.rows, words);
  return hipGetLastError();
}

hipError_t launch_backward(const Geom& g, const void* q, const void* k, const void* v, const void* dout,
                           float2* ld, void* dq, void* dk,
                           void* dv, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* tcolptr,
                           const int32_t* trowidx, int32_t* counters, int32_t* cost, int32_t* order_q,
                           int32_t* order_k, int32_t* bounds, int num_cu, bool delta_walk, hipStream_t s) {
  const double scale = 1.0 / sqrt((double)g.D);
  if (g.dtype == BSA_F32) {
    const unsigned grid = (unsigned)g.rows;
    if (g.D == 64) {
      bwd::dq_f32_kernel<64><<<grid, 256, 0, s>>>((const float*)q, (const float*)k, (const float*)v,
                                                   (const float*)dout, ld, (float*)dq, row_ptr, col_idx, g, scale);
      bwd::dkdv_f32_kernel<64><<<grid, 256, 0, s>>>((const float*)q, (const float*)k, (const float*)v,
                                                     (const float*)dout, ld, (float*)dk, (float*)dv, tcolptr, trowidx,
                                                     g, scale);
    } else {
      bwd::dq_f32_kernel<128><<<grid, 256, 0, s>>>((const float*)q, (const float*)k, (const float*)v,
                                                    (const float*)dout, ld, (float*)dq, row_ptr, col_idx, g, scale);
      bwd::dkdv_f32_kernel<128><<<grid, 256, 0, s>>>((const float*)q, (const float*)k, (const float*)v,
                                                      (const float*)dout, ld, (float*)dk, (float*)dv, tcolptr,
                                                      trowidx, g, scale);
    }
    return hipGetLastError();
  }
  bwd::Args a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.dout = (const uint16_t*)dout;
  a.ld = ld;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.g = g;
  a.c_log2 = (float)(1.4426950408889634 * scale);
  a.inv_sqrt_d = (float)scale;
  a.pairs = (g.S + 1) / 2;
  a.items = (int32_t)((int64_t)g.B * g.nh * a.pairs);
  const int grid = ((num_cu + 7) / 8) * 8;        // one workgroup per CU (LDS-limited), a multiple of 8 XCDs
  // work orders as for the forward (pairs of query blocks over the CSR, pairs of
  // key blocks over the transposed one); the cost scratch is reused in stream order
  hipError_t e = launch_attn_schedule(g, row_ptr, col_idx, cost, order_q, bounds, s, 2);
  if (e != hipSuccess) return e;
  a.ptr = row_ptr;
  a.idx = col_idx;
  a.counters = counters + 16;
  a.order = order_q;
  a.bounds = bounds;
  const int grid2 = ((num_cu * 2 + 7) / 8) * 8;   // two workgroups per CU
  if (delta_walk) bwd::dq_bf16_kernel<true><<<grid2, 256, 0, s>>>(a);    // Delta
  a.counters = counters;
  bwd::dq_bf16_kernel<false><<<grid2, 256, 0, s>>>(a);   // dQ
  e = launch_attn_schedule(g, tcolptr, trowidx, cost, order_k, bounds + 16, s, 2);
  if (e != hipSuccess) return e;
  a.ptr = tcolptr;
  a.idx = trowidx;
  a.counters = counters + 8;
  a.order = order_k;
  a.bounds = bounds + 16;
  bwd::dkdv_pc_kernel<<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bsa
