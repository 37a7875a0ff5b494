// Device helpers shared by the block-mask and group-mask kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geom.h"

namespace bsa {

// order-preserving map of a double to uint64 (larger value -> larger key);
// -0.0 and +0.0 are equal values and must share one key
__device__ __forceinline__ uint64_t order_key(double z) {
  const uint64_t b = z == 0.0 ? 0ull : (uint64_t)__double_as_longlong(z);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// inverse of order_key
__device__ __forceinline__ double key_to_double(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)b);
}

// Wavefront-wide reduction with DPP moves inside each row of 16 lanes and lane
// swaps across rows and halves; every lane ends with the result.
__device__ __forceinline__ uint32_t dpp_step(uint32_t v, int step) {
  switch (step) {
    case 0: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false);   // lanes ^ 1
    case 1: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false);   // lanes ^ 2
    case 2: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false);  // half-row mirror
    default: return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false); // row mirror
  }
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, int lane, Op op) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  constexpr int kWords = sizeof(T) / 4;
  auto as_words = [](T x, uint32_t* w) { __builtin_memcpy(w, &x, sizeof(T)); };
  auto from_words = [](const uint32_t* w) {
    T x;
    __builtin_memcpy(&x, w, sizeof(T));
    return x;
  };
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    uint32_t w[kWords];
    as_words(v, w);
#pragma unroll
    for (int q = 0; q < kWords; ++q) w[q] = dpp_step(w[q], st);
    v = op(v, from_words(w));
  }
  {
    uint32_t w[kWords];
    as_words(v, w);
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      const auto r = __builtin_amdgcn_permlane16_swap(w[q], w[q], false, false);
      w[q] = (lane & 16) ? r[0] : r[1];   // the other row of the pair
    }
    v = op(v, from_words(w));
  }
  {
    uint32_t w[kWords];
    as_words(v, w);
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      const auto r = __builtin_amdgcn_permlane32_swap(w[q], w[q], false, false);
      w[q] = (lane & 32) ? r[0] : r[1];   // the other half
    }
    v = op(v, from_words(w));
  }
  return v;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// ---- pooling sums and lane reductions --------------------------------------
// add_chunk: one 16-byte chunk of a token row (8 bf16 or 4 float32 values) added
// into float64 sums (exact for bf16 and for sums of a few float32 values).
template <typename T>
__device__ __forceinline__ void add_chunk(double* acc, const uint4& c);

template <>
__device__ __forceinline__ void add_chunk<uint16_t>(double* acc, const uint4& c) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += (double)__uint_as_float(w[e] << 16);
    acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void add_chunk<float>(double* acc, const uint4& c) {
  acc[0] += (double)__uint_as_float(c.x);
  acc[1] += (double)__uint_as_float(c.y);
  acc[2] += (double)__uint_as_float(c.z);
  acc[3] += (double)__uint_as_float(c.w);
}

// value of lane ^ 16 / lane ^ 32 (VALU lane swaps, no LDS round trip)
__device__ __forceinline__ double xor16(double x, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  const uint32_t l = (lane & 16) ? lo[0] : lo[1], h = (lane & 16) ? hi[0] : hi[1];
  return __longlong_as_double((long long)(((uint64_t)h << 32) | l));
}
__device__ __forceinline__ double xor32(double x, int lane) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
  const uint32_t l = (lane & 32) ? lo[0] : lo[1], h = (lane & 32) ? hi[0] : hi[1];
  return __longlong_as_double((long long)(((uint64_t)h << 32) | l));
}

// Reduction over the lanes of one row group (lane bits below log2(LPR)): DPP
// steps inside 8 / 16 lanes, then the 16-lane swap.
template <int LPR, typename Op>
__device__ __forceinline__ double group_reduce(double v, int lane, Op op) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "lanes per row");
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if (st == 3 && LPR == 8) break;
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = dpp_step((uint32_t)b, st), hi = dpp_step((uint32_t)(b >> 32), st);
    v = op(v, __longlong_as_double((long long)(((uint64_t)hi << 32) | lo)));
  }
  if constexpr (LPR == 32) v = op(v, xor16(v, lane));
  return v;
}

// float64 means of channels c0 .. c0 + NC - 1 of the 4 keys of group gid (4
// consecutive tokens of the fractal order) of head bh: sums of 4 bf16 or float32
// values in float64, then a quarter (NC a multiple of 8; c0 a multiple of NC)
template <typename T, int NC>
__device__ __forceinline__ void group_mean(const T* __restrict__ k, const Geom& g, int64_t bh, int gid, int c0,
                                           double (&m)[NC]) {
  constexpr int EPC = 16 / sizeof(T);
  const int gpb = g.N / 4, blk = gid / gpb, m0 = (gid % gpb) * 4;
#pragma unroll
  for (int e = 0; e < NC; ++e) m[e] = 0.0;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint4* src = (const uint4*)(k + ((size_t)bh * g.L + block_token_row(g, blk, m0 + t)) * g.D + c0);
#pragma unroll
    for (int x = 0; x < NC / EPC; ++x) add_chunk<T>(m + x * EPC, src[x]);
  }
#pragma unroll
  for (int e = 0; e < NC; ++e) m[e] *= 0.25;
}

// ---- prefix sums and row sums over lanes ----------------------------------
// value of lane - N inside each row of 16 lanes (0 where that is outside the row)
template <int N>
__device__ __forceinline__ uint64_t row_shr64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, 0x110 + N, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), 0x110 + N, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
// inclusive prefix sum over the 64 lanes (lane 0 first): shifts inside the rows of
// 16 lanes, then the totals of the lower rows read back as scalars
__device__ __forceinline__ uint64_t wave_prefix_u64(uint64_t v, int lane) {
  v += row_shr64<1>(v);
  v += row_shr64<2>(v);
  v += row_shr64<4>(v);
  v += row_shr64<8>(v);
  const uint64_t r0 = readlane_u64(v, 15), r1 = readlane_u64(v, 31), r2 = readlane_u64(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0ull) + (row >= 2 ? r1 : 0ull) + (row >= 3 ? r2 : 0ull);
}
// sum over each aligned group of 8 lanes (every lane of the group gets it)
__device__ __forceinline__ double sum8(double v) {
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = dpp_step((uint32_t)b, st), hi = dpp_step((uint32_t)(b >> 32), st);
    v += __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
  }
  return v;
}

// Sliding-tile window (NABLA page, Metodologia item 3): block ids are tiles
// (t, y, x) of Hp x Wp patches per frame; ids i and j are within the window when
// every coordinate differs by at most the given extent.
__device__ __forceinline__ bool in_window(const Geom& g, int i, int j, int win_t, int win_h, int win_w) {
  const int HW = g.Hp * g.Wp;
  const int ti = i / HW, yi = (i / g.Wp) % g.Hp, xi = i % g.Wp;
  const int tj = j / HW, yj = (j / g.Wp) % g.Hp, xj = j % g.Wp;
  return abs(ti - tj) <= win_t && abs(yi - yj) <= win_h && abs(xi - xj) <= win_w;
}

// Calls f(j) for every block j in the (clipped) window of block i, the threads of
// a group splitting the work: thread `first` of `stride` takes entries first,
// first + stride, ...  Enumerates the box of at most (2w_t+1)(2w_h+1)(2w_w+1)
// tiles directly, so the cost does not grow with the number of blocks per row.
template <typename F>
__device__ __forceinline__ void for_each_window_block(const Geom& g, int i, int win_t, int win_h, int win_w, int first,
                                                      int stride, F f) {
  const int HW = g.Hp * g.Wp, T = g.S / HW;
  const int ti = i / HW, yi = (i / g.Wp) % g.Hp, xi = i % g.Wp;
  const int wt = min(win_t, T), wh = min(win_h, g.Hp), ww = min(win_w, g.Wp);   // no overflow below
  const int t0 = max(ti - wt, 0), t1 = min(ti + wt, T - 1);
  const int y0 = max(yi - wh, 0), y1 = min(yi + wh, g.Hp - 1);
  const int x0 = max(xi - ww, 0), x1 = min(xi + ww, g.Wp - 1);
  const int nx = x1 - x0 + 1, nyx = (y1 - y0 + 1) * nx, n = (t1 - t0 + 1) * nyx;
  for (int e = first; e < n; e += stride) {
    const int dt = e / nyx, rem = e - dt * nyx, dy = rem / nx, dx = rem - dy * nx;
    f(((t0 + dt) * g.Hp + y0 + dy) * g.Wp + x0 + dx);
  }
}

// The same window as runs of consecutive block ids: f(a, b) for blocks a .. b, one
// run per (frame, patch row) of the clipped box around block (ti, yi, xi); thread
// `first` of `stride` takes runs first, first + stride, ...
template <typename F>
__device__ __forceinline__ void for_each_window_run(const Geom& g, int ti, int yi, int xi, int win_t, int win_h,
                                                    int win_w, int first, int stride, F f) {
  const int T = g.S / (g.Hp * g.Wp);
  const int wt = min(win_t, T), wh = min(win_h, g.Hp), ww = min(win_w, g.Wp);   // no overflow below
  const int t0 = max(ti - wt, 0), t1 = min(ti + wt, T - 1);
  const int y0 = max(yi - wh, 0), y1 = min(yi + wh, g.Hp - 1);
  const int x0 = max(xi - ww, 0), x1 = min(xi + ww, g.Wp - 1);
  const int ny = y1 - y0 + 1, n = (t1 - t0 + 1) * ny;
  for (int e = first; e < n; e += stride) {
    const int dt = e / ny, dy = e - dt * ny;
    const int base = ((t0 + dt) * g.Hp + y0 + dy) * g.Wp;
    f(base + x0, base + x1);
  }
}

}  // namespace bsa
