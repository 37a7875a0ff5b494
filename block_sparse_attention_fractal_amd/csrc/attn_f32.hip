// Block-sparse attention forward for float32 tensors (any CSR; head_dim 64 or 128).
//
// Same operation as the bf16 kernel (NABLA page, gist.science/es/paper/2507.13546,
// Metodologia item 2, bullet "Expansion"; an optional per-entry logit shift
// carries the sampling weights of the SIP mask mode), written for accuracy rather than
// speed: logits, the online softmax and the output accumulation are float64
// (fp32 products are exact in float64), so the result stays within 1e-5 of a
// float64 evaluation even when logits reach ~10^2.  One workgroup per CSR row;
// the query tile sits in LDS; thread (query qi, slice sl) owns output channels [sl*D/4, (sl+1)*D/4) and the
// logits of keys sl, sl+4, ..., so four adjacent lanes cooperate per query.
#include <math.h>

#include "kernels.h"

namespace bsa {

// kGroups: col_idx lists 4-token key groups (AB-Attention page, "Los tres recursos
// de AB-Attention", third resource); every 16 entries form one 64-key tile and the
// padding keys of a row's last tile are masked.
template <int D, bool kGroups>
__global__ void __launch_bounds__(256) attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                       const float* __restrict__ v, float* __restrict__ o,
                                                       float* __restrict__ lse, const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx,
                                                       const float* __restrict__ shift, Geom g, double scale) {
  constexpr int DS = D / 4;
  __shared__ float Qs[64][D + 1];
  __shared__ float Ks[64][D + 1];
  __shared__ float Vs[64][D + 1];
  __shared__ double Ps[64][65];
  const int64_t r = blockIdx.x;
  const int64_t bh = r / g.S;
  const int i = (int)(r - bh * g.S);
  const int tid = threadIdx.x, qi = tid >> 2, sl = tid & 3;
  const float* qh = q + (size_t)bh * g.L * D;
  const float* kh = k + (size_t)bh * g.L * D;
  const float* vh = v + (size_t)bh * g.L * D;
  const int qtok = block_token_row(g, i, qi);
  for (int e = tid; e < 64 * D; e += 256) Qs[e / D][e % D] = qh[(size_t)block_token_row(g, i, e / D) * D + e % D];
  double oacc[DS];
#pragma unroll
  for (int d = 0; d < DS; ++d) oacc[d] = 0.0;
  double m = -INFINITY, l = 0.0;
  const int beg = row_ptr[r], end = row_ptr[r + 1];
  const int gpb = g.N / 4;   // groups per block
  for (int it = beg; it < end; it += kGroups ? 16 : 1) {
    const int j = kGroups ? 0 : min(max(col_idx[it], 0), g.S - 1);
    const double sh = !kGroups && shift ? (double)shift[it] : 0.0;   // the entry's logit shift, if any
    __syncthreads();
    for (int e = tid; e < 64 * D; e += 256) {
      const int row = e / D, d = e % D;
      int tok;
      bool valid = true;
      if (kGroups) {
        valid = it + (row >> 2) < end;
        const int gid = valid ? min(max(col_idx[it + (row >> 2)], 0), g.L / 4 - 1) : 0;
        tok = block_token_row(g, gid / gpb, (gid % gpb) * 4 + (row & 3));
      } else {
        tok = block_token_row(g, j, row);
      }
      const size_t off = (size_t)tok * D + d;
      Ks[row][d] = valid ? kh[off] : 0.f;
      Vs[row][d] = valid ? vh[off] : 0.f;
    }
    __syncthreads();
    double s[16];
    double mt = -INFINITY;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int kk = sl + 4 * c;
      double acc = 0.0;
#pragma unroll 4
      for (int d = 0; d < D; ++d) acc = __fma_rn((double)Qs[qi][d], (double)Ks[kk][d], acc);
      s[c] = kGroups && it + (kk >> 2) >= end ? -INFINITY : acc * scale + sh;
      mt = fmax(mt, s[c]);
    }
    mt = fmax(mt, __shfl_xor(mt, 1));
    mt = fmax(mt, __shfl_xor(mt, 2));
    const double m_new = fmax(m, mt);
    const double alpha = exp(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int d = 0; d < DS; ++d) oacc[d] *= alpha;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const double p = exp(s[c] - m_new);
      l += p;
      Ps[qi][sl + 4 * c] = p;
    }
    __syncthreads();
    for (int kk = 0; kk < 64; ++kk) {
      const double p = Ps[qi][kk];
#pragma unroll 8
      for (int d = 0; d < DS; ++d) oacc[d] = __fma_rn(p, (double)Vs[kk][sl * DS + d], oacc[d]);
    }
  }
  l += __shfl_xor(l, 1);
  l += __shfl_xor(l, 2);
  const double inv = l > 0.0 ? 1.0 / l : 0.0;
  float* orow = o + ((size_t)bh * g.L + qtok) * D + sl * DS;
#pragma unroll
  for (int d = 0; d < DS; ++d) orow[d] = (float)(oacc[d] * inv);
  if (lse && sl == 0) lse[(size_t)bh * g.L + qtok] = (float)(m + log(l));
}

hipError_t launch_attn_f32(const Geom& g, const float* q, const float* k, const float* v, float* o, float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, const float* shift, hipStream_t s) {
  const double scale = 1.0 / sqrt((double)g.D);
  if (g.D == 64)
    attn_f32_kernel<64, false><<<(unsigned)g.rows, 256, 0, s>>>(q, k, v, o, lse, row_ptr, col_idx, shift, g, scale);
  else
    attn_f32_kernel<128, false><<<(unsigned)g.rows, 256, 0, s>>>(q, k, v, o, lse, row_ptr, col_idx, shift, g, scale);
  return hipGetLastError();
}

hipError_t launch_attn_groups_f32(const Geom& g, const float* q, const float* k, const float* v, float* o,
                                  float* lse, const int32_t* row_ptr, const int32_t* col_idx, hipStream_t s) {
  const double scale = 1.0 / sqrt((double)g.D);
  if (g.D == 64)
    attn_f32_kernel<64, true><<<(unsigned)g.rows, 256, 0, s>>>(q, k, v, o, lse, row_ptr, col_idx, nullptr, g, scale);
  else
    attn_f32_kernel<128, true><<<(unsigned)g.rows, 256, 0, s>>>(q, k, v, o, lse, row_ptr, col_idx, nullptr, g,
                                                                scale);
  return hipGetLastError();
}

}  // namespace bsa
