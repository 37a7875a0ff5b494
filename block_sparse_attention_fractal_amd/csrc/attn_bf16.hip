// Block-sparse attention forward, bf16 inputs, head_dim 128, gfx950 MFMA.
//
// Computes, for every query token of block i, softmax attention over exactly
// the tokens of the key blocks listed in CSR row i (NABLA page,
// gist.science/es/paper/2507.13546, Metodologia item 2, bullet "Expansion":
// the block mask decides which N x N tiles are computed, all or nothing).
//
// Work decomposition
//   * one work item = one CSR row = one 64-query block; a persistent grid of
//     two-wave (128-thread) workgroups pulls items from an atomic counter;
//   * wave w owns queries 32w..32w+31 and keeps its Q operand in registers;
//   * per kept key block: K (64 x 128) and V^T (128 x 64) tiles are staged
//     global -> registers -> LDS (XOR-swizzled), the next tile's global loads
//     are issued before the current tile's math;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q
//     columns from registers); the accumulator then holds, per lane, 32 keys
//     of ONE query, so the online-softmax state (running max m, partial sum l)
//     is per lane and only the max needs one cross-half exchange per tile;
//   * O^T += V^T P^T with the same MFMA: A = V^T rows from LDS (pre-transposed
//     in HBM, keys stored in the accumulator's order), B = P^T taken straight
//     from the S^T accumulator registers after conversion to bf16;
//   * P is rounded to bf16 for the PV product; everything else is fp32.
//
// MFMA operand conventions used (32x32x16, bf16): A lane l holds row l%32 and
// eight consecutive k of half l/32; B lane l holds column l%32 likewise; the
// accumulator register r of lane l is element (8*(r/4) + 4*(l/32) + r%4, l%32).
// Both contractions pair "element e of half h" of A and B, so the physical k
// order inside the instruction is irrelevant.
#include <math.h>

#include "kernels.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

struct AttnBf16Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;
  uint16_t* o;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int32_t* counter;
  Geom g;
  float c_log2;   // log2(e) / sqrt(D)
};

constexpr int kD = 128;
constexpr int kVtOff = 16384;

// K tile: 64 rows x 256 B, 16-byte chunk c of row k at chunk c ^ (k & 15).
__device__ __forceinline__ int k_lds(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }
// V^T tile: 128 rows x 128 B, chunk c of row d at c ^ ((d >> 1) & 7).
__device__ __forceinline__ int v_lds(int row, int chunk) {
  return kVtOff + row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const __bf16 ha = (__bf16)a, hb = (__bf16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

__global__ void __launch_bounds__(128) attn_bf16_kernel(AttnBf16Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[32768];
  __shared__ int s_item;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const Geom g = a.g;
  const float c_log2 = a.c_log2;

  for (;;) {
    if (tid == 0) s_item = atomicAdd(a.counter, 1);
    __syncthreads();
    const int64_t r = s_item;
    if (r >= g.rows) break;
    const int64_t bh = r / g.S;
    const int i = (int)(r - bh * g.S);
    const int beg = a.row_ptr[r], end = a.row_ptr[r + 1];
    const uint16_t* kh = a.k + (size_t)bh * g.L * kD;
    const uint16_t* vth = a.vt + (size_t)bh * g.S * kD * 64;

    bf16x8 qreg[8];
    {
      const uint16_t* qrow = a.q + ((size_t)bh * g.L + block_token_row(g, i, 32 * wave + l32)) * kD + 8 * h;
#pragma unroll
      for (int s = 0; s < 8; ++s) qreg[s] = *(const bf16x8*)(qrow + 16 * s);
    }
    f32x16 oacc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[u][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    uint4 kst[8], vst[8];
    const int lrow = tid >> 4, lchunk = tid & 15;
    auto load_tile = [&](int j) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        kst[u] = *(const uint4*)(kh + (size_t)block_token_row(g, j, lrow + 8 * u) * kD + lchunk * 8);
      const uint16_t* vb = vth + (size_t)j * kD * 64;
#pragma unroll
      for (int u = 0; u < 8; ++u) vst[u] = *(const uint4*)(vb + (tid + 128 * u) * 8);
    };
    // ids outside [0, S) are clamped: a malformed CSR gives wrong values, never a stray access
    auto col = [&](int t) { return min(max(a.col_idx[t], 0), g.S - 1); };
    if (beg < end) load_tile(col(beg));

    for (int it = beg; it < end; ++it) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 8; ++u) *(uint4*)(smem + k_lds(lrow + 8 * u, lchunk)) = kst[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int cc = tid + 128 * u;
        *(uint4*)(smem + v_lds(cc >> 3, cc & 7)) = vst[u];
      }
      __syncthreads();
      if (it + 1 < end) load_tile(col(it + 1));

      f32x16 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[t][e] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 ak = *(const bf16x8*)(smem + k_lds(32 * t + l32, 2 * s + h));
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[s], sacc[t], 0, 0, 0);
        }
      }

      float mx = sacc[0][0];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[t][e]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx * c_log2);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[u][e] *= alpha;

      bf16x8 pb[4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][e], c_log2, -m_new));
          l_run += p;
          pb[2 * t + (e >> 3)][e & 7] = (__bf16)p;
        }
      }

#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 av = *(const bf16x8*)(smem + v_lds(32 * u + l32, 2 * s + h));
          oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[s], oacc[u], 0, 0, 0);
        }
      }
    }

    l_run = pair_sum(l_run);
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;   // an empty row yields zeros
    const int qrow = 32 * wave + l32;
    __syncthreads();
    // O tile [64 queries][128 d] bf16 in LDS, 8-byte unit x of row q at x ^ (q & 31)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int unit = 8 * u + 2 * rq + h;
        uint2 w;
        w.x = pack_bf16x2(oacc[u][4 * rq + 0] * inv, oacc[u][4 * rq + 1] * inv);
        w.y = pack_bf16x2(oacc[u][4 * rq + 2] * inv, oacc[u][4 * rq + 3] * inv);
        *(uint2*)(smem + qrow * 256 + ((unit ^ (qrow & 31)) << 3)) = w;
      }
    }
    if (a.lse && h == 0)
      a.lse[(size_t)bh * g.L + block_token_row(g, i, qrow)] = (m_run + log2f(l_run)) * 0.69314718055994531f;
    __syncthreads();
    uint16_t* oh = a.o + (size_t)bh * g.L * kD;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int row = lrow + 8 * u;
      const uint2 lo = *(const uint2*)(smem + row * 256 + (((2 * lchunk) ^ (row & 31)) << 3));
      const uint2 hi = *(const uint2*)(smem + row * 256 + (((2 * lchunk + 1) ^ (row & 31)) << 3));
      *(uint4*)(oh + (size_t)block_token_row(g, i, row) * kD + lchunk * 8) = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
}

hipError_t launch_attn_bf16(const Geom& g, const void* q, const void* k, const void* vt, void* o, float* lse,
                            const int32_t* row_ptr, const int32_t* col_idx, int32_t* counter, int num_cu,
                            hipStream_t s) {
  AttnBf16Args a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.vt = (const uint16_t*)vt;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.counter = counter;
  a.g = g;
  a.c_log2 = (float)(1.4426950408889634 / sqrt((double)g.D));
  int64_t grid = (int64_t)num_cu * 2;   // two resident workgroups per CU
  if (grid > g.rows) grid = g.rows;
  attn_bf16_kernel<<<(unsigned)grid, 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bsa
