// Attention over gathered 4-token key groups, bf16 inputs, head_dim 128, gfx950 MFMA.
//
// The mask lists, for every query block of 64 tokens, the kept key GROUPS of 4
// consecutive fractal-order tokens (AB-Attention page, news.hamidun.com/es/news/14960,
// "Los tres recursos de AB-Attention", third resource: small key/value blocks
// gathered by index into full matrix-core tiles, without reordering tokens).
// Every 16 kept groups of a row (ascending) form one 64-key tile; the last tile of
// a row is padded and its padding keys take no part in the softmax.
//
// Work decomposition
//   * a work item is ONE query block (tiles of different rows rarely coincide,
//     so there is nothing to share between neighbouring rows); 256-thread
//     workgroups, wave w owns queries 32*(w&1).. and the 32 keys of slots
//     8*(w>>1).. of every tile; the two waves of a query range merge their
//     online-softmax states at the end;
//   * persistent grid, two workgroups per CU; the rows are split into 8 XCD
//     ranges of equal cost (64-key tiles plus a fixed per-row cost) and each
//     range runs its long rows first (the block kernel's work order);
//   * a K tile slot is 4 key rows (1 KB) loaded with ONE direct-to-LDS 16-byte
//     buffer load per wave (lane -> row lane/16, chunk lane%16, swizzled
//     chunk c ^ (row & 15)); a V slot is the group's 128 x 4 transposed block
//     of the prepared V (1 KB, contiguous), also one load;
//   * LDS holds a ring of three K tiles and a ring of two V tiles (80 KB): at
//     step t the workgroup issues V of tile t+1 and then K of tile t+2, so one
//     wait for all but the newest four loads and one barrier per tile make
//     tile t resident while two more are in flight; the group ids of tile t+3
//     are loaded at step t (older than that step's tile loads, so the same
//     wait covers them);
//   * S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16.  The V tile
//     stores the group of tile entry e at slot e with bits 0 and 1 swapped, so
//     the two 4-key halves of a lane's V^T operand (entries 8(w>>1) + 4s + h and
//     that + 2) sit in neighbouring slots: two 8-byte LDS reads land directly in
//     the operand registers, in exactly the key order P leaves the S^T
//     accumulator.
#include <math.h>

#include "kernels.h"

namespace bsa {
namespace grp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// volatile: each 8-byte V read stays a read of its own (the compiler would pair
// neighbouring reads of one operand half and then copy the halves together)
typedef __attribute__((address_space(3))) const volatile u32x2 lds_u2;

constexpr int kD = 128;
constexpr int kTile = 16384;      // 16 slots of 1 KB: one K or one V tile
constexpr int kVRing = 3 * kTile;  // K ring: 3 tiles at 0; V ring: 2 tiles from here
constexpr int kLds = 5 * kTile;    // 80 KB: two workgroups fill a CU's 160 KB
constexpr int kItemSlot = kLds - 4;     // the item index, only live between items (last word of V slot 1)
constexpr float kLazy = 8.0f;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

struct Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vg;     // [B*nh, L/4, D, 4]
  uint16_t* o;
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;  // group ids
  int32_t* counters;
  const int32_t* order;    // rows in processing order: XCD x takes order[bounds[x] .. bounds[x+1])
  const int32_t* bounds;   // 9 entries
  Geom g;
  float c_log2;
  uint32_t magic_wp, magic_hp;   // floor(2^31/d)+1 (exact n/d = (n*magic)>>31 for n, d <= 4096); fractal order: magic_wp = 0
  int32_t pxmul, rs;             // row offset of patch column px (8 or 64) and of patch row m / 8 (W or 8)
  int32_t groups;                // L / 4 per head
};

__device__ __forceinline__ int k_lds(int row, int chunk) { return row * 256 + ((chunk ^ (row & 15)) << 4); }

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
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t magic) {
  return (uint32_t)(((uint64_t)n * magic) >> 31);
}

// First row (tensor layout) of block j: fractal order -> 64 j; original order ->
// the patch's top-left token (block ids and patch counts <= 4096: multiply-high).
__device__ __forceinline__ int block_base_row(const Args& a, int j) {
  const Geom& g = a.g;
  if (g.layout == 1) return j * 64;
  const int rest = (int)div_magic((uint32_t)j, a.magic_wp);
  const int px = j - rest * g.Wp;
  const int t = (int)div_magic((uint32_t)rest, a.magic_hp);
  const int py = rest - t * g.Hp;
  return (t * g.H + py * 8) * g.W + px * 8;
}
// First row of group gid: tokens 4(gid % 16) .. +3 of block gid / 16, which sit
// in one patch row (P = 8), so the group's 4 rows are consecutive in memory.
// Written without a branch on the layout: in fractal order the host passes
// magic_wp = 0 (so the patch coordinates beyond px vanish), pxmul = 64, rs = 8.
__device__ __forceinline__ int group_base_row(const Args& a, int gid) {
  const Geom& g = a.g;
  const int j = gid >> 4;
  const int rest = (int)div_magic((uint32_t)j, a.magic_wp);
  const int px = j - rest * g.Wp;
  const int t = (int)div_magic((uint32_t)rest, a.magic_hp);
  const int py = rest - t * g.Hp;
  return (t * g.H + py * 8) * g.W + px * a.pxmul + ((gid & 15) >> 1) * a.rs + (gid & 1) * 4;
}

__global__ void __launch_bounds__(256, 2) attn_groups_bf16_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];   // K ring (3 tiles) + V ring (2 tiles)
  int& s_item = *(int*)(smem + kItemSlot);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int wq = wave & 1;       // which 32 queries
  const int kh = wave >> 1;      // which 8 slots (32 keys) of every tile
  const Geom g = a.g;
  const float c_log2 = a.c_log2;
  const int rs = g.layout == 1 ? 8 : g.W;

  // per-lane parts of this wave's four slot loads (slots 4*wave + u)
  int koff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int slot = 4 * wave + u;
    const int row = 4 * slot + (lane >> 4);
    const int lc = (lane & 15) ^ (row & 15);
    koff[u] = (lane >> 4) * kD * 2 + lc * 16;
  }
  // LDS addresses of this lane's operands in ring slot 0 (reads add an immediate);
  // opaque to the optimiser, which would otherwise split each back into the
  // array base plus an offset and add the two before every read
  uint32_t kaddr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kaddr[s] = (uint32_t)(uintptr_t)(lds_void*)(smem + k_lds(32 * kh + l32, 2 * s + h));
  uint32_t vaddr = (uint32_t)(uintptr_t)(lds_void*)(smem + kVRing + (8 * kh + 2 * h) * 1024 + l32 * 8);
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(kaddr[s]));
  asm volatile("" : "+v"(vaddr));

  const int xcd = blockIdx.x & 7;
  const int lo_t = a.bounds[xcd], hi_t = a.bounds[xcd + 1];   // this XCD's stretch of the work order

  for (;;) {
    if (tid == 0) s_item = lo_t + atomicAdd(&a.counters[xcd], 1);
    __syncthreads();
    const int idx = __builtin_amdgcn_readfirstlane(s_item);
    if (idx >= hi_t) break;
    const int64_t r = a.order[idx];
    const int64_t bh = r / g.S;
    const int i = (int)(r - bh * g.S);
    const int p0 = a.row_ptr[r], e0 = a.row_ptr[r + 1];
    const int ng = e0 - p0;
    const int ntiles = (ng + 15) >> 4;

    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.k + (size_t)bh * g.L * kD), (short)0, g.L * kD * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.vg + (size_t)bh * g.L * kD), (short)0, g.L * kD * 2, 0x00020000);

    // The row's group ids through a buffer over its own entries: lane l holds entry
    // 16t + l % 16 of tile t, and entries past the row's end read as group 0 (those
    // keys are masked, and tiles past the end are loaded but never read)
    const __amdgpu_buffer_rsrc_t grs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.col_idx + p0), (short)0, ng * 4, 0x00020000);
    const int goff = (lane & 15) * 4;
    auto gids_of = [&](int t) { return __builtin_amdgcn_raw_buffer_load_b32(grs, goff, 64 * t, 0); };
    // this wave's four group ids of a tile, as scalars
    struct Ids { int v[4]; };
    auto ids_of = [&](int gl) {
      Ids r;
#pragma unroll
      for (int u = 0; u < 4; ++u) r.v[u] = min(max(__builtin_amdgcn_readlane(gl, 4 * wave + u), 0), a.groups - 1);
      return r;
    };
    // byte offset of each lane's group in this head's K, computed by all lanes at
    // once and read back per slot (cheaper than the same arithmetic on scalars
    // for each of the wave's four slots)
    auto kbytes_of = [&](int gl) { return group_base_row(a, min(max(gl, 0), a.groups - 1)) * kD * 2; };
    auto issue_k = [&](int kb, auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(smem + slot * kTile + (4 * wave + u) * 1024), 16,
                                                 koff[u], __builtin_amdgcn_readlane(kb, 4 * wave + u), 0, 0);
    };
    auto issue_v = [&](const Ids& id, auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(smem + kVRing + slot * kTile + (4 * wave + u) * 1024),
                                                 16, lane * 16, id.v[(u >> 1) | ((u & 1) << 1)] * 1024, 0, 0);
    };
    auto wait_barrier4 = [&]() {
      asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    bf16x8 qreg[8];
    {
      const int qtok = block_base_row(a, i) + ((32 * wq + l32) >> 3) * rs + (l32 & 7);
      const uint16_t* qrow = a.q + ((size_t)bh * g.L + qtok) * kD + 8 * h;
#pragma unroll
      for (int s = 0; s < 8; ++s) qreg[s] = *(const bf16x8*)(qrow + 16 * s);
    }
    f32x16 oacc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[u][e] = 0.f;
    // l_run: sum of the float32 P (for the LSE); l_pv: sum of the bf16-rounded P the
    // PV product uses, the normaliser of O (O is then a convex combination of the
    // kept V rows with exactly the weights the MFMA applied)
    float m_ref = -INFINITY, l_run = 0.f, l_pv = 0.f;

    if (ntiles > 0) {
      // ids: tile t+1 as scalars (its V is issued at step t), tile t+2 in a VGPR
      // (its K offsets are computed and issued at step t), tile t+3 loaded at step t
      const int g1v = gids_of(1);
      Ids s1 = ids_of(g1v);
      int g2 = gids_of(2);
      {
        const int g0v = gids_of(0);
        const Ids s0 = ids_of(g0v);
        issue_v(s0, std::integral_constant<int, 0>{});
        issue_k(kbytes_of(g0v), std::integral_constant<int, 0>{});
      }
      issue_k(kbytes_of(g1v), std::integral_constant<int, 1>{});
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      int t = 0;
      auto step = [&](auto ks_c, auto vs_c) {
        constexpr int KS = decltype(ks_c)::value;
        constexpr int VS = decltype(vs_c)::value;
        wait_barrier4();                                   // K(t) and V(t) resident everywhere
        const int g3 = gids_of(t + 3);                     // older than the tile loads below
        const Ids s2 = ids_of(g2);
        issue_v(s1, std::integral_constant<int, VS ^ 1>{});
        issue_k(kbytes_of(g2), std::integral_constant<int, (KS + 2) % 3>{});
        const int nvalid = min(16, ng - 16 * t);
        if (8 * kh < nvalid) {
          // all eight K operand reads in flight before the first product
          bf16x8 ak[8];
#pragma unroll
          for (int s = 0; s < 8; ++s) ak[s] = *(lds_bf16x8*)(uintptr_t)(kaddr[s] + KS * kTile);
          __builtin_amdgcn_sched_barrier(0);
          f32x16 sacc;
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
          for (int s = 0; s < 8; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[s], qreg[s], sacc, 0, 0, 0);
          // the V operands (keys 16s + 4h + 0..3 and 16s + 8 + 4h + 0..3 of channel
          // 32u + l32) are read while the softmax runs
          u32x2 vlo[2][4], vhi[2][4];
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              vlo[s][u] = *(lds_u2*)(uintptr_t)(vaddr + VS * kTile + s * 4096 + u * 256);
              vhi[s][u] = *(lds_u2*)(uintptr_t)(vaddr + VS * kTile + s * 4096 + u * 256 + 1024);
            }
          // register e holds key 8(e/4) + 4h + e%4 of this wave's 32, i.e. slot 8kh + 2(e/4) + h
          if (nvalid < 16) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
              if (8 * kh + 2 * (e >> 2) + h >= nvalid) sacc[e] = -INFINITY;
          }
          float m5[5];
#pragma unroll
          for (int x = 0; x < 5; ++x) m5[x] = fmaxf(fmaxf(sacc[3 * x], sacc[3 * x + 1]), sacc[3 * x + 2]);
          float mx = fmaxf(fmaxf(fmaxf(m5[0], m5[1]), m5[2]), fmaxf(fmaxf(m5[3], m5[4]), sacc[15]));
          mx = pair_max(mx) * c_log2;
          if (__builtin_amdgcn_ballot_w64(mx > m_ref + kLazy) != 0) {
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
            m_ref = m_new;
            l_run *= alpha;
            l_pv *= alpha;
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int e = 0; e < 16; ++e) oacc[u][e] *= alpha;
          }
          bf16x8 pbv[2];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[e], c_log2, -m_ref));
            l_run += p;
            pbv[e >> 3][e & 7] = (__bf16)p;
          }
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            l_pv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pbv[s], pbv[s], 0, 1), kOnes2, l_pv, false);
            l_pv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pbv[s], pbv[s], 2, 3), kOnes2, l_pv, false);
            l_pv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pbv[s], pbv[s], 4, 5), kOnes2, l_pv, false);
            l_pv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pbv[s], pbv[s], 6, 7), kOnes2, l_pv, false);
          }
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const bf16x8 av = __builtin_bit_cast(
                  bf16x8, (u32x4){vlo[s][u].x, vlo[s][u].y, vhi[s][u].x, vhi[s][u].y});
              oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pbv[s], oacc[u], 0, 0, 0);
            }
        }
        s1 = s2;
        g2 = g3;
        ++t;
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      for (;;) {
        step(I0{}, I0{});
        if (t >= ntiles) break;
        step(I1{}, I1{});
        if (t >= ntiles) break;
        step(I2{}, I0{});
        if (t >= ntiles) break;
        step(I0{}, I1{});
        if (t >= ntiles) break;
        step(I1{}, I0{});
        if (t >= ntiles) break;
        step(I2{}, I1{});
        if (t >= ntiles) break;
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the loads past the row's end have landed
    }

    // merge the two key halves of each query range, then normalise and store
    __syncthreads();
    float* xo = (float*)smem + wq * (64 * 64);               // partner accumulators, [reg][lane]
    float4* xm = (float4*)(smem + 32768) + wq * 64;          // partner (m_ref, l_run, l_pv)
    if (kh == 1) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) xo[(16 * u + e) * 64 + lane] = oacc[u][e];
      xm[lane] = make_float4(m_ref, l_run, l_pv, 0.f);
    }
    __syncthreads();
    if (kh == 0) {
      const float4 pm = xm[lane];
      const float m_tot = fmaxf(m_ref, pm.x);
      const float a0 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_tot);
      const float a1 = pm.x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm.x - m_tot);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[u][e] = a0 * oacc[u][e] + a1 * xo[(16 * u + e) * 64 + lane];
      l_run = pair_sum(a0 * l_run + a1 * pm.y);
      l_pv = pair_sum(a0 * l_pv + a1 * pm.z);
      m_ref = m_tot;
    }
    __syncthreads();
    const int qrow = 32 * wq + l32;
    if (kh == 0) {
      const float inv = l_pv > 0.f ? 1.f / l_pv : 0.f;       // an empty row yields zeros
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
      if (a.lse && h == 0) {
        const int tok = block_base_row(a, i) + (qrow >> 3) * rs + (qrow & 7);
        a.lse[(size_t)bh * g.L + tok] = (m_ref + log2f(l_run)) * 0.69314718055994531f;
      }
    }
    __syncthreads();
    {
      const int lchunk = tid & 15;
      const int base = block_base_row(a, i);
      uint16_t* oh = a.o + (size_t)bh * g.L * kD;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = (tid >> 4) + 16 * u;
        const uint2 lo = *(const uint2*)(smem + row * 256 + (((2 * lchunk) ^ (row & 31)) << 3));
        const uint2 hi = *(const uint2*)(smem + row * 256 + (((2 * lchunk + 1) ^ (row & 31)) << 3));
        const int tok = base + (row >> 3) * rs + (row & 7);
        *(uint4*)(oh + (size_t)tok * kD + lchunk * 8) = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
  }
}

// V -> [B*nh, L/4, D, 4]: each 4-token group transposed to channel-major (4 keys
// of one channel are 8 contiguous bytes).  One thread per (group, 8 channels).
__global__ void __launch_bounds__(256) prep_vg_kernel(const uint16_t* __restrict__ v, uint16_t* __restrict__ vg,
                                                      Geom g) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (bh, group, chunk of 8 channels)
  const int chunks = g.D / 8;
  const int64_t ng = (int64_t)g.B * g.nh * (g.L / 4);
  if (idx >= ng * chunks) return;
  const int c = (int)(idx % chunks);
  const int64_t gg = idx / chunks;
  const int64_t bh = gg / (g.L / 4);
  const int gid = (int)(gg - bh * (g.L / 4));
  const int blk = gid / (g.N / 4), m0 = (gid % (g.N / 4)) * 4;
  const int row0 = block_token_row(g, blk, m0);        // the group's 4 rows are consecutive
  const uint16_t* src = v + ((size_t)bh * g.L + row0) * g.D + 8 * c;
  uint4 rows[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) rows[t] = *(const uint4*)(src + (size_t)t * g.D);
  // channel d of token t is 16-bit half (d & 1) of word d / 2 of rows[t]
  auto half = [&](int t, int d) -> uint32_t {
    const uint32_t w = ((const uint32_t*)&rows[t])[d >> 1];
    return (d & 1) ? (w >> 16) : (w & 0xffffu);
  };
  uint4* dst = (uint4*)(vg + (gg * g.D + 8 * c) * 4);
#pragma unroll
  for (int x = 0; x < 4; ++x) {      // channels 2x and 2x+1: keys 0-3 of each
    const int d0 = 2 * x, d1 = 2 * x + 1;
    dst[x] = make_uint4(half(0, d0) | (half(1, d0) << 16), half(2, d0) | (half(3, d0) << 16),
                        half(0, d1) | (half(1, d1) << 16), half(2, d1) | (half(3, d1) << 16));
  }
}

// cost of every row: its 64-key tiles plus a fixed per-row cost (Q load, ring prologue, output)
__global__ void __launch_bounds__(256) row_cost_kernel(const int32_t* __restrict__ row_ptr, int64_t rows,
                                                       int32_t* __restrict__ cost) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r < rows) cost[r] = (row_ptr[r + 1] - row_ptr[r] + 15) / 16 + 4;
}

}  // namespace grp

hipError_t launch_prep_vg(const Geom& g, const void* v, void* vg, hipStream_t s) {
  const int64_t n = (int64_t)g.B * g.nh * (g.L / 4) * (g.D / 8);
  grp::prep_vg_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>((const uint16_t*)v, (uint16_t*)vg, g);
  return hipGetLastError();
}

hipError_t launch_attn_groups_bf16(const Geom& g, const void* q, const void* k, const void* vg, void* o, float* lse,
                                   const int32_t* row_ptr, const int32_t* col_idx, int32_t* counters, int32_t* cost,
                                   int32_t* order, int32_t* bounds, int num_cu, hipStream_t s) {
  grp::row_cost_kernel<<<(unsigned)((g.rows + 255) / 256), 256, 0, s>>>(row_ptr, g.rows, cost);
  hipError_t e = launch_schedule_costs(cost, (int)g.rows, order, bounds, s);
  if (e != hipSuccess) return e;
  grp::Args a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.vg = (const uint16_t*)vg;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.counters = counters;
  a.order = order;
  a.bounds = bounds;
  a.g = g;
  a.c_log2 = (float)(1.4426950408889634 / sqrt((double)g.D));
  a.magic_wp = g.layout == 1 ? 0u : (uint32_t)((1ull << 31) / (uint64_t)g.Wp + 1);
  a.magic_hp = (uint32_t)((1ull << 31) / (uint64_t)g.Hp + 1);
  a.pxmul = g.layout == 1 ? 64 : 8;
  a.rs = g.layout == 1 ? 8 : g.W;
  a.groups = g.L / 4;
  const int grid = ((num_cu * 2 + 7) / 8) * 8;
  grp::attn_groups_bf16_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace bsa
