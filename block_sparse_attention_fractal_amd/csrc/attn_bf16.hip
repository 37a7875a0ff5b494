// Block-sparse attention forward, bf16 inputs, head_dim 128, gfx950 MFMA.
//
// Computes, for every query token of block i, softmax attention over exactly
// the tokens of the key blocks listed in CSR row i (NABLA page,
// gist.science/es/paper/2507.13546, Metodologia item 2, bullet "Expansion":
// the block mask decides which N x N tiles are computed, all or nothing), with
// an optional per-entry logit shift (the inclusion-probability weights of a SIP
// mask, AB-Attention page, "Los tres recursos de AB-Attention").
//
// Work decomposition
//   * a work item is a PAIR of adjacent query blocks (i, i+1) of one head; the
//     item walks the union of their two ascending key lists, so a key/value tile
//     kept by both is fetched once and used by both (halves L2/MALL traffic on
//     the common case where neighbouring blocks keep almost the same keys);
//   * 256-thread workgroups: waves 0-1 own block i, waves 2-3 own block i+1,
//     32 queries per wave, the Q operand held in registers;
//   * persistent grid, two workgroups per CU; workgroup b runs on XCD b % 8 and
//     pulls items from its XCD's own stretch of a work order built by two small
//     kernels before it: the items are split into 8 contiguous ranges of about
//     equal cost (distinct key blocks of the pair plus a fixed per-item cost),
//     so concurrently running items of one XCD share a head and its K/V tiles in
//     that XCD's L2, and each range runs its longest items first;
//   * K (64 x 128) and V^T (128 x 64) tiles move global -> LDS with direct
//     (VGPR-free) 16-byte buffer loads into a ring of three K and two V^T tiles:
//     the per-lane part of each address is a constant register, the tile part a
//     scalar offset; at step j the workgroup issues V^T of tile j+1 and K of
//     tile j+2, and the loop is unrolled over the ring positions so every LDS
//     address is a per-lane constant plus an immediate;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q
//     columns from registers): each lane's accumulator holds 32 keys of ONE
//     query, so the online-softmax state is per lane;
//   * the running max is refreshed lazily and found only when needed:
//     exponentials use a reference max, P of a tile is formed under it first,
//     and the reference is raised (the tile's row max taken, O rescaled, P formed
//     again) only when some lane's sum of its 32 values exceeds 2^13, so every p
//     stays <= 2^13, the common tile spends no instructions on its max, and the
//     64 output accumulators are rarely rescaled;
//   * O^T += V^T P^T with the same MFMA: A = V^T rows from LDS (pre-transposed
//     in HBM, keys stored in the accumulator's order), B = P^T straight from the
//     S^T accumulator registers after rounding to bf16.
//
// MFMA operand conventions (32x32x16, bf16): A lane l holds row l%32 and eight
// k of half l/32; B lane l holds column l%32 likewise; accumulator register r
// of lane l is element (8*(r/4) + 4*(l/32) + r%4, l%32).  Both contractions
// pair "element e of half h" of A and B, so the physical k order inside the
// instruction does not matter.
#include <float.h>
#include <math.h>

#include <algorithm>

#include <type_traits>

#include "kernels.h"

namespace bsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(1))) const void gbl_void;

struct AttnBf16Args {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;
  uint16_t* o;
  uint16_t* o_lo;      // training variant: O - bf16(O) in bf16 (null otherwise)
  float* lse;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const float* shift;  // per-entry natural-log logit shift, or null
  int32_t* counters;   // 8 per-XCD item counters
  const int32_t* order;    // items in processing order: XCD x takes order[bounds[x] .. bounds[x+1])
  const int32_t* bounds;   // 9 entries
  Geom g;
  float c_log2;        // log2(e) / sqrt(D)
  uint32_t magic_wp, magic_hp;   // floor(2^31/d)+1: exact n/d = (n*magic)>>31 for n, d <= 4096 (d = 1 included)
  int32_t pxmul;                 // rows per patch column step: 8 (original order) or 64 (fractal, magic_wp = 0)
  int32_t pairs;       // query-block pairs per head = ceil(S/2)
  int32_t items;       // B*heads*pairs
};

// Tile geometry for head dim D (128 or 64): a K tile is 64 rows x 2D bytes, a V^T
// tile D rows x 128 bytes; both are moved by kLoads direct 16-byte loads per thread.
template <int D>
struct Shape {
  static constexpr int kTile = 64 * D * 2;            // one K or V^T tile (bytes)
  static constexpr int kChunks = D / 8;               // 16-byte chunks per K row
  static constexpr int kLoads = kTile / (256 * 16);   // direct loads per thread per tile
  static constexpr int kVRing = 3 * kTile;            // K ring: 3 slots at 0; V^T ring: 2 slots from here
  static constexpr int kLds = 5 * kTile;              // 80 KB at D = 128: two workgroups fill a CU's 160 KB
  static constexpr int kItemSlot = kLds - 4;          // the item index, only live between items
};
constexpr float kSumCap = 4096.0f;     // a lane's P sum over a key half above which the reference max is raised
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

// K tile: 64 rows x 2D bytes, 16-byte chunk c of row k stored at chunk c ^ (k mod D/8).
template <int D>
__device__ __forceinline__ int k_lds(int row, int chunk) {
  return row * (2 * D) + ((chunk ^ (row & (D / 8 - 1))) << 4);
}
// V^T tile: 128 rows x 128 B, chunk c of row d stored at c ^ ((d >> 1) & 7).
__device__ __forceinline__ int v_lds(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }

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

// First token row (in the tensor's own layout) of block j; token m of the block
// sits rs*(m/8) + m%8 rows further (rs = W for original order, 8 for fractal).
// Block ids and patch counts are <= 4096, so the divisions use multiply-high
// with a 31-bit shift (exact for every divisor, 1 included).
__device__ __forceinline__ int block_base_row(const AttnBf16Args& a, int j) {
  const Geom& g = a.g;
  const int rest = (int)div_magic((uint32_t)j, a.magic_wp);   // 0 in fractal order (magic_wp = 0)
  const int px = j - rest * g.Wp;
  const int t = (int)div_magic((uint32_t)rest, a.magic_hp);
  const int py = rest - t * g.Hp;
  return (t * g.H + py * 8) * g.W + px * a.pxmul;
}

// Hides a value from the optimiser (a VGPR operand of an empty asm statement).  A
// plain device function, so that the VGPR constraint is never checked for the host
// inside the kernel template.
__device__ __forceinline__ void opaque_vgpr(uint32_t& x) { asm volatile("" : "+v"(x)); }

// The body is compiled for the device only: instantiated in the host pass, its
// LDS address-space casts and VGPR asm operands (dependent on D) would make the
// instantiation invalid there and drop the launch stub.
// kTrain: the PV product takes P as a pair of bf16 terms (hi and the rounding
// residual lo), O is normalised by the float32 sum of P and written as a bf16
// pair (o and o_lo), so that o + o_lo carries O = sum P v / sum P to ~2^-16 and
// the backward can form its row term dO . O from it.
template <int D, bool kShift, bool kTrain>   // head dim; per-entry logit shifts; training variant
__global__ void __launch_bounds__(256, 2) attn_bf16_kernel(AttnBf16Args a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using Sh = Shape<D>;
  constexpr int kTile = Sh::kTile, kVRing = Sh::kVRing, kLoads = Sh::kLoads, kItemSlot = Sh::kItemSlot;
  constexpr int kQS = D / 16;      // k-steps of the QK product
  constexpr int kOU = D / 32;      // 32-channel blocks of the output
  __shared__ __attribute__((aligned(16))) uint8_t smem[Sh::kLds];   // K ring (3 slots) + V^T ring (2 slots)
  int& s_item = *(int*)(smem + kItemSlot);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: its derived LDS offsets stay scalar
  const int h = lane >> 5, l32 = lane & 31;
  const int qb = wave >> 1;      // which block of the pair
  const int wq = wave & 1;       // which 32 queries of that block
  const Geom g = a.g;
  const float c_log2 = a.c_log2;
  const int rs = g.layout == 1 ? 8 : g.W;

  // per-thread byte offsets of this thread's direct-load chunks (independent of the tile)
  int koff[kLoads], voff[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int c = (kLoads * wave + u) * 64 + lane;
    const int m = c / Sh::kChunks;                          // key row in the tile
    const int lc = (c % Sh::kChunks) ^ (m & (Sh::kChunks - 1));   // logical chunk stored at this slot
    koff[u] = (((m >> 3) * rs + (m & 7)) * D + lc * 8) * 2;
    const int d = c >> 3;                                   // V^T row
    const int lv = (lane & 7) ^ ((d >> 1) & 7);
    voff[u] = d * 128 + lv * 16;
  }

  // LDS addresses of this lane's MFMA operands in stage 0: the row term of the
  // swizzle is the same for both key halves (K) and all four row blocks (V^T), so
  // a K read is kaddr[s] plus an immediate and a V^T read vaddr[s] plus one
  uint32_t kaddr[kQS], vaddr[4];
#pragma unroll
  for (int s = 0; s < kQS; ++s) kaddr[s] = (uint32_t)(uintptr_t)(lds_void*)(smem + k_lds<D>(l32, 2 * s + h));
#pragma unroll
  for (int s = 0; s < 4; ++s) vaddr[s] = (uint32_t)(uintptr_t)(lds_void*)(smem + kVRing + v_lds(l32, 2 * s + h));
  // opaque to the optimiser: otherwise it splits each address back into the array
  // base (a relocated symbol, so never an immediate) plus the offset, and adds the
  // two before every read
#pragma unroll
  for (int s = 0; s < kQS; ++s) opaque_vgpr(kaddr[s]);
#pragma unroll
  for (int s = 0; s < 4; ++s) opaque_vgpr(vaddr[s]);

  // this workgroup's XCD and its stretch of the item order (the schedule kernels
  // below balance the stretches by estimated cost and put long items first)
  const int xcd = blockIdx.x & 7;
  const int lo_t = a.bounds[xcd], hi_t = a.bounds[xcd + 1];

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
    int pa = a.row_ptr[r0], ea = a.row_ptr[r0 + 1];
    int pb = two ? a.row_ptr[r0 + 1] : 0, eb = two ? a.row_ptr[r0 + 2] : 0;

    const uint8_t* kh = (const uint8_t*)(a.k + (size_t)bh * g.L * D);
    const uint8_t* vth = (const uint8_t*)(a.vt + (size_t)bh * g.S * D * 64);

    // Each key list is read through a 64-entry window held one entry per lane and
    // indexed with readlane, so the union walk costs no memory round trip per tile;
    // a window is refilled (one coalesced load) every 64 entries.
    int wa_base = pa, wb_base = pb;
    constexpr bool has_shift = kShift;
    auto shift_at = [&](int idx, int end) -> int {   // the shift of entry idx, as float bits, one per lane
      return has_shift && idx < end ? __float_as_int(a.shift[idx]) : 0;
    };
    int wa = wa_base + lane < ea ? a.col_idx[wa_base + lane] : 0x7fffffff;
    int wb = wb_base + lane < eb ? a.col_idx[wb_base + lane] : 0x7fffffff;
    int sa = shift_at(wa_base + lane, ea), sb = shift_at(wb_base + lane, eb);
    auto peek_a = [&]() -> int {
      if (pa >= ea) return 0x7fffffff;
      if (pa - wa_base >= 64) {
        wa_base = pa;
        wa = wa_base + lane < ea ? a.col_idx[wa_base + lane] : 0x7fffffff;
        sa = shift_at(wa_base + lane, ea);
        // wait here, on the rare refill path, so that no path reaches the readlane
        // below with a load pending (the compiler would otherwise wait for every
        // outstanding load, tile loads included, before each readlane)
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      }
      return __builtin_amdgcn_readlane(wa, pa - wa_base);
    };
    auto peek_b = [&]() -> int {
      if (pb >= eb) return 0x7fffffff;
      if (pb - wb_base >= 64) {
        wb_base = pb;
        wb = wb_base + lane < eb ? a.col_idx[wb_base + lane] : 0x7fffffff;
        sb = shift_at(wb_base + lane, eb);
        // wait here, on the rare refill path, so that no path reaches the readlane
        // below with a load pending (the compiler would otherwise wait for every
        // outstanding load, tile loads included, before each readlane)
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      }
      return __builtin_amdgcn_readlane(wb, pb - wb_base);
    };
    // union walk over the two ascending key lists (wave-uniform scalars); shl is
    // the logit shift of this wave's block for the tile, in log2 units
    auto next_tile = [&](int& j, int& mine, float& shl) {
      const int ja = peek_a();
      const int jb = peek_b();
      j = min(ja, jb);
      const bool ka = ja == j;
      const bool kb = jb == j;
      mine = qb == 0 ? (int)ka : (int)kb;   // an int: a bool carried across steps becomes a lane mask
      shl = 0.f;
      if (has_shift) {
        const float sha = ka ? __int_as_float(__builtin_amdgcn_readlane(sa, pa - wa_base)) : 0.f;
        const float shb = kb ? __int_as_float(__builtin_amdgcn_readlane(sb, pb - wb_base)) : 0.f;
        shl = (qb == 0 ? sha : shb) * 1.44269504088896341f;
      }
      pa += ka;
      pb += kb;
    };
    // K and V^T of this head as raw buffers: the per-lane part of each 16-byte load
    // is a constant VGPR offset, the tile part a scalar offset; loads past the
    // head's extent return zeros instead of touching other memory
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)kh, (short)0, g.L * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)vth, (short)0, g.S * D * 64 * 2, 0x00020000);
    // a tile id past the end of the walk is clamped: every step issues exactly
    // kLoads K and kLoads V^T loads per thread, which keeps the vmcnt arithmetic exact
    auto issue_k = [&](int j, auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      const int jc = min(max(j, 0), g.S - 1);
      const int ks = block_base_row(a, jc) * D * 2;
#pragma unroll
      for (int u = 0; u < kLoads; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(smem + slot * kTile + (kLoads * wave + u) * 1024), 16,
                                                 koff[u], ks, 0, 0);
    };
    auto issue_v = [&](int j, auto slot_c) {
      constexpr int slot = decltype(slot_c)::value;
      // readfirstlane: the tile id is wave-uniform, and saying so keeps the load's
      // offset in an SGPR (else each load becomes a one-trip waterfall loop)
      const int jc = __builtin_amdgcn_readfirstlane(min(max(j, 0), g.S - 1));
      const int vs = jc * D * 64 * 2;
#pragma unroll
      for (int u = 0; u < kLoads; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(smem + kVRing + slot * kTile + (kLoads * wave + u) * 1024),
                                                 16, voff[u], vs, 0, 0);
    };
    // wait for this thread's older loads, then a plain barrier (the compiler's own
    // barrier would first wait for every outstanding load, including the ones
    // meant to stay in flight); lgkmcnt(0) keeps LDS writes ordered as well
    auto wait_barrier4 = [&]() {   // the newest kLoads K loads stay in flight
      if constexpr (kLoads == 4)
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };

    bf16x8 qreg[kQS];
    if (has_q) {
      const int qtok = block_base_row(a, i0 + qb) + ((32 * wq + l32) >> 3) * rs + (l32 & 7);
      const uint16_t* qrow = a.q + ((size_t)bh * g.L + qtok) * D + 8 * h;
#pragma unroll
      for (int s = 0; s < kQS; ++s) qreg[s] = *(const bf16x8*)(qrow + 16 * s);
    }
    f32x16 oacc[kOU];
#pragma unroll
    for (int u = 0; u < kOU; ++u)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[u][e] = 0.f;
    // l_run: sum of the float32 P (for the LSE); l_pv: sum of the bf16-rounded P that
    // the PV product uses, so that O = sum bf16(P) v / sum bf16(P) is a convex
    // combination of the kept V rows with exactly the weights the MFMA applied (P of
    // the dominant key is not exactly 1 under the lazy reference, and its 2^-9
    // rounding would otherwise show at full size in O)
    float m_ref = -FLT_MAX, l_run = 0.f, l_pv = 0.f;

    // tiles j (current), j1, j2: K of a tile is loaded two steps ahead of its QK
    // products, V^T one step ahead (issued first, so a step's wait can leave the
    // newest K in flight)
    int j, j1, j2;
    int m0, m1, m2;
    float shl, shl1, shl2;
    next_tile(j, m0, shl);
    next_tile(j1, m1, shl1);
    issue_v(j, std::integral_constant<int, 0>{});
    issue_k(j, std::integral_constant<int, 0>{});
    issue_k(j1, std::integral_constant<int, 1>{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // one tile in K slot KS = j % 3 and V^T slot VS = j % 2: QK and the softmax
    // update, then (after V^T is everywhere) PV; the loop is unrolled six times so
    // every LDS address is a per-lane constant plus an immediate
    auto step = [&](auto ks_c, auto vs_c) {
      constexpr int KS = decltype(ks_c)::value;
      constexpr int VS = decltype(vs_c)::value;
      next_tile(j2, m2, shl2);
      wait_barrier4();                                        // K(j) and V(j) resident everywhere
      issue_v(j1, std::integral_constant<int, VS ^ 1>{});     // into the slot V(j-1) used
      issue_k(j2, std::integral_constant<int, (KS + 2) % 3>{});   // into the slot K(j-1) used
      bf16x8 pbv[4], pbl[4];
      if (m0) {
        f32x16 sacc[2];
        // the products of key half t (keys 32t .. 32t+31 of the tile)
        auto qk = [&](auto t_c) {
          constexpr int t = decltype(t_c)::value;
          bf16x8 ak[kQS];   // every operand read issued ahead of the products
#pragma unroll
          for (int s = 0; s < kQS; ++s) ak[s] = *(lds_bf16x8*)(uintptr_t)(kaddr[s] + KS * kTile + t * (kTile / 2));
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[t][e] = 0.f;
#pragma unroll
          for (int s = 0; s < kQS; ++s) sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[s], qreg[s], sacc[t], 0, 0, 0);
        };
        // P of key half t under the current reference (bf16 operands of its two PV
        // k-steps); returns this lane's float32 sum of its 16 values
        auto softmax = [&](auto t_c) -> float {
          constexpr int t = decltype(t_c)::value;
          float lt = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][e], c_log2, shl - m_ref));
            lt += p;
            const __bf16 ph = (__bf16)p;
            pbv[2 * t + (e >> 3)][e & 7] = ph;
            if constexpr (kTrain) pbl[2 * t + (e >> 3)][e & 7] = (__bf16)(p - (float)ph);
          }
          return lt;
        };
        // raise the reference to cover the row max of key half t (a tree of
        // three-input maxima over its 16 values): O and the sums rescaled
        auto raise_ref = [&](auto t_c) {
          constexpr int t = decltype(t_c)::value;
          float m5[6];
#pragma unroll
          for (int x = 0; x < 5; ++x) m5[x] = fmaxf(fmaxf(sacc[t][3 * x], sacc[t][3 * x + 1]), sacc[t][3 * x + 2]);
          m5[5] = sacc[t][15];
          float mx = fmaxf(fmaxf(fmaxf(m5[0], m5[1]), m5[2]), fmaxf(fmaxf(m5[3], m5[4]), m5[5]));
          mx = pair_max(mx) * c_log2 + shl;
          const float m_new = fmaxf(m_ref, mx);
          const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
          m_ref = m_new;
          l_run *= alpha;
          l_pv *= alpha;
#pragma unroll
          for (int u = 0; u < kOU; ++u)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[u][e] *= alpha;
        };
        // l_pv: the float32 sum of the bf16 P of key half t, as the PV product uses it
        auto sum_pv = [&](auto t_c) {
          constexpr int t = decltype(t_c)::value;
          if constexpr (!kTrain) {
#pragma unroll
            for (int s = 2 * t; s < 2 * t + 2; ++s) {
              l_pv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pbv[s], pbv[s], 0, 1), kOnes2, l_pv, false);
              l_pv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pbv[s], pbv[s], 2, 3), kOnes2, l_pv, false);
              l_pv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pbv[s], pbv[s], 4, 5), kOnes2, l_pv, false);
              l_pv = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pbv[s], pbv[s], 6, 7), kOnes2, l_pv, false);
            }
          }
        };
        // O^T += V^T P^T over the 32 keys of half t (two 16-key k-steps)
        auto pv = [&](auto t_c) {
          constexpr int t = decltype(t_c)::value;
#pragma unroll
          for (int s = 2 * t; s < 2 * t + 2; ++s) {
#pragma unroll
            for (int u = 0; u < kOU; ++u) {
              const bf16x8 av = *(lds_bf16x8*)(uintptr_t)(vaddr[s] + VS * kTile + u * 4096);
              oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pbv[s], oacc[u], 0, 0, 0);
              if constexpr (kTrain) oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pbl[s], oacc[u], 0, 0, 0);
            }
          }
        };
        using T0 = std::integral_constant<int, 0>;
        using T1 = std::integral_constant<int, 1>;
        {
          // The reference max is raised only when it must be: P of a key half is
          // formed under the current reference and kept unless some lane's sum of
          // its 16 values passes 2^12 (p >= 0, so every kept p is <= 2^12; an
          // overflow shows as an infinite sum, and so does every sum of the item's
          // first tile, whose reference starts at -FLT_MAX); then that half's
          // products are formed again from the K tile (still in its slot), O
          // rescaled and its P formed afresh.  The halves are staggered so that
          // each one's exponentials run beside the other half's matrix products:
          // QK of half 1 with the softmax of half 0, PV of half 0 with the softmax
          // of half 1.
          __builtin_amdgcn_s_setprio(1);
          qk(T0{});
          // half 0's products first (the scheduler would otherwise interleave the two
          // accumulation chains and leave half 0 unfinished until the end), with its
          // operand reads kept four ahead of the products
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // 4 LDS reads
#pragma unroll
          for (int x = 0; x < kQS - 4; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // 4 MFMA
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_setprio(0);
          qk(T1{});
          float lt = softmax(T0{});
          if (__builtin_amdgcn_ballot_w64(lt > kSumCap) != 0) {
            // a compiler-level memory clobber: the products are formed again from
            // LDS rather than kept alive through the fast path
            asm volatile("" ::: "memory");
            qk(T0{});
            raise_ref(T0{});
            lt = softmax(T0{});
          }
          l_run += lt;
          sum_pv(T0{});
          pv(T0{});
          lt = softmax(T1{});
          if (__builtin_amdgcn_ballot_w64(lt > kSumCap) != 0) {
            asm volatile("" ::: "memory");
            qk(T1{});
            raise_ref(T1{});
            lt = softmax(T1{});
          }
          l_run += lt;
          // raised priority again for the step's MFMA-only tail (PV of half 1)
          __builtin_amdgcn_s_setprio(1);
          sum_pv(T1{});
          pv(T1{});
          __builtin_amdgcn_s_setprio(0);
        }
      }
      j = j1; m0 = m1; shl = shl1;
      j1 = j2; m1 = m2; shl1 = shl2;
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    while (j != 0x7fffffff) {
      step(I0{}, I0{});
      if (j == 0x7fffffff) break;
      step(I1{}, I1{});
      if (j == 0x7fffffff) break;
      step(I2{}, I0{});
      if (j == 0x7fffffff) break;
      step(I0{}, I1{});
      if (j == 0x7fffffff) break;
      step(I1{}, I0{});
      if (j == 0x7fffffff) break;
      step(I2{}, I1{});
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the clamped loads past the end have landed

    // epilogue: normalise, stage O through LDS (block qb at qb * 16 KB), store coalesced
    __syncthreads();
    const int qrow = 32 * wq + l32;
    if (has_q) {
      l_run = pair_sum(l_run);
      l_pv = pair_sum(l_pv);
      const float lnorm = kTrain ? l_run : l_pv;
      const float inv = lnorm > 0.f ? 1.f / lnorm : 0.f;   // an empty row yields zeros
      uint8_t* ob = smem + qb * (kTile);       // block qb's 64 x 2D bytes of O
      uint8_t* obl = smem + (2 + qb) * kTile;  // training variant: block qb's O - bf16(O)
#pragma unroll
      for (int u = 0; u < kOU; ++u) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int unit = 8 * u + 2 * rq + h;
          const int off = qrow * (2 * D) + ((unit ^ (qrow & (D / 4 - 1))) << 3);
          float ov[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) ov[x] = oacc[u][4 * rq + x] * inv;
          *(uint2*)(ob + off) = make_uint2(pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3]));
          if constexpr (kTrain) {
            float lo[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) lo[x] = ov[x] - (float)(__bf16)ov[x];
            *(uint2*)(obl + off) = make_uint2(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]));
          }
        }
      }
      if (a.lse && h == 0) {
        const int tok = block_base_row(a, i0 + qb) + (qrow >> 3) * rs + (qrow & 7);
        a.lse[(size_t)bh * g.L + tok] = (m_ref + log2f(l_run)) * 0.69314718055994531f;
      }
    }
    __syncthreads();
    {
      const int sb = tid >> 7;                 // block of the pair this thread stores
      if (sb == 0 || two) {
        constexpr int kCh = D / 8;             // 16-byte chunks per output row
        constexpr int kRowsPer = 128 / kCh;    // rows one pass of 128 threads covers
        const int t7 = tid & 127;
        const int lchunk = t7 % kCh;
        const int base = block_base_row(a, i0 + sb);
#pragma unroll
        for (int part = 0; part < (kTrain ? 2 : 1); ++part) {
          uint16_t* oh = (part ? a.o_lo : a.o) + (size_t)bh * g.L * D;
          const uint8_t* ob = smem + (2 * part + sb) * kTile;
#pragma unroll
          for (int u = 0; u < 64 / kRowsPer; ++u) {
            const int row = t7 / kCh + kRowsPer * u;
            const uint2 lo = *(const uint2*)(ob + row * (2 * D) + (((2 * lchunk) ^ (row & (D / 4 - 1))) << 3));
            const uint2 hi = *(const uint2*)(ob + row * (2 * D) + (((2 * lchunk + 1) ^ (row & (D / 4 - 1))) << 3));
            const int tok = base + (row >> 3) * rs + (row & 7);
            *(uint4*)(oh + (size_t)tok * D + lchunk * 8) = make_uint4(lo.x, lo.y, hi.x, hi.y);
          }
        }
      }
    }
  }
#endif
}

// ---------------------------------------------------------------------------
// Work order.  An item's cost is the number of distinct key blocks its two query
// blocks keep (the steps of its union walk) plus a fixed per-item cost.  The
// order splits the items, in index order, into 8 ranges of about equal total
// cost (one per XCD; splitting by kept tiles instead left the ranges of heads
// with many short, less overlapping rows ~8 % longer) and starts each range with
// its long items, so that the short ones fill the end (a long item started last
// would otherwise decide when the kernel ends).
// ---------------------------------------------------------------------------
constexpr int kItemOverhead = 4;   // per-item cost in tile steps (Q load, ring prologue, output)
constexpr int kMaxBitmapWords = 128;   // S <= 4096 blocks

// cost[it] for every item: the key lists of its nb query blocks marked in an LDS
// bitmap and counted
__global__ void __launch_bounds__(256) item_cost_kernel(const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ col_idx, int S, int groups,
                                                        int nb, int items, int32_t* __restrict__ cost) {
  __shared__ uint32_t bits[kMaxBitmapWords];
  __shared__ int part[4];
  const int tid = threadIdx.x;
  const int words = (S + 31) >> 5;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int bh = it / groups, p = it - bh * groups;
    const int64_t r0 = (int64_t)bh * S + nb * p;
    const int64_t e = row_ptr[r0 + min(nb, S - nb * p)];   // the rows' entries are contiguous
    for (int w = tid; w < words; w += 256) bits[w] = 0u;
    __syncthreads();
    for (int64_t x = row_ptr[r0] + tid; x < e; x += 256) {
      const int c = col_idx[x];
      if (c >= 0 && c < S) atomicOr(&bits[c >> 5], 1u << (c & 31));
    }
    __syncthreads();
    int n = 0;
    for (int w = tid; w < words; w += 256) n += __popc(bits[w]);
    for (int m = 32; m >= 1; m >>= 1) n += __shfl_xor(n, m, 64);
    if ((tid & 63) == 0) part[tid >> 6] = n;
    __syncthreads();
    if (tid == 0) cost[it] = part[0] + part[1] + part[2] + part[3] + kItemOverhead;
    __syncthreads();
  }
}

// One workgroup: XCD x gets order[bounds[x] .. bounds[x+1]); an item goes to the
// XCD whose eighth of the total cost its exclusive cost prefix falls in.  Inside
// a range the long items (at least four times the mean cost) come first, then
// the rest, each class in item order (neighbouring items share key tiles, so
// they stay together; a finer sort by cost scattered them and cost L2 hits).
// No atomics: the order is deterministic.
__global__ void __launch_bounds__(1024) schedule_kernel(const int32_t* __restrict__ cost, int items,
                                                        int32_t* __restrict__ order, int32_t* __restrict__ bounds) {
  constexpr int NB = 2;             // long items, then the rest
  __shared__ int64_t psum[1024];
  __shared__ int cnt[1024][NB];      // per-chunk class counts, then their inclusive prefix over chunks
  __shared__ int lo[9];              // first item of each XCD range (lo[8] = items)
  __shared__ int plo[9][NB];         // items of each class before lo[x]
  const int t = threadIdx.x;
  const int chunk = (items + 1023) / 1024;
  const int b0 = min(items, t * chunk), b1 = min(items, b0 + chunk);
  int64_t own = 0;
  int local[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) local[b] = 0;
  for (int i = b0; i < b1; ++i) own += cost[i];
  psum[t] = own;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {   // inclusive scan of the chunk sums
    const int64_t v = t >= off ? psum[t - off] : 0;
    __syncthreads();
    psum[t] += v;
    __syncthreads();
  }
  // long items: at least four times the mean cost
  const int64_t tlong = 4 * psum[1023] / items;
  auto bucket_of = [&](int c) { return c >= tlong ? 0 : 1; };
  for (int i = b0; i < b1; ++i) ++local[bucket_of(cost[i])];
#pragma unroll
  for (int b = 0; b < NB; ++b) cnt[t][b] = local[b];
  if (t < 9) lo[t] = -1;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {   // inclusive scan of the class counts over the chunks
    int w[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) w[b] = t >= off ? cnt[t - off][b] : 0;
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NB; ++b) cnt[t][b] += w[b];
    __syncthreads();
  }
  const int64_t total = psum[1023];
  const int64_t pre0 = psum[t] - own;
  auto xcd_of = [&](int64_t pre) { return (int)min((int64_t)7, pre * 8 / total); };
  // range starts and the class counts before them
  {
    int run[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) run[b] = cnt[t][b] - local[b];
    int64_t pre = pre0;
    int xp = b0 == 0 ? -1 : (b0 < b1 ? xcd_of(pre0 - cost[b0 - 1]) : 7);
    for (int i = b0; i < b1; ++i) {
      const int c = cost[i];
      const int x = xcd_of(pre);
      for (int y = xp + 1; y <= x; ++y) {
        lo[y] = i;
#pragma unroll
        for (int b = 0; b < NB; ++b) plo[y][b] = run[b];
      }
      xp = x;
      ++run[bucket_of(c)];
      pre += c;
    }
  }
  __syncthreads();
  if (t == 0) {   // ranges left empty at the end (one item holding more than an eighth of the cost)
    for (int y = 0; y <= 8; ++y)
      if (lo[y] < 0) {
        lo[y] = items;
        for (int b = 0; b < NB; ++b) plo[y][b] = cnt[1023][b];
      }
  }
  __syncthreads();
  if (t <= 8) bounds[t] = lo[t];
  {
    int run[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) run[b] = cnt[t][b] - local[b];
    int64_t pre = pre0;
    for (int i = b0; i < b1; ++i) {
      const int c = cost[i];
      const int x = xcd_of(pre);
      const int bk = bucket_of(c);
      int pos = lo[x] + run[bk] - plo[x][bk];
      for (int b = 0; b < bk; ++b) pos += plo[x + 1][b] - plo[x][b];
      order[pos] = i;
      ++run[bk];
      pre += c;
    }
  }
}

hipError_t launch_attn_schedule(const Geom& g, const int32_t* row_ptr, const int32_t* col_idx, int32_t* cost,
                                int32_t* order, int32_t* bounds, hipStream_t s, int nb) {
  const int groups = (g.S + nb - 1) / nb;
  const int items = (int)((int64_t)g.B * g.nh * groups);
  item_cost_kernel<<<std::min(items, 4096), 256, 0, s>>>(row_ptr, col_idx, g.S, groups, nb, items, cost);
  schedule_kernel<<<1, 1024, 0, s>>>(cost, items, order, bounds);
  return hipGetLastError();
}

hipError_t launch_schedule_costs(const int32_t* cost, int items, int32_t* order, int32_t* bounds, hipStream_t s) {
  schedule_kernel<<<1, 1024, 0, s>>>(cost, items, order, bounds);
  return hipGetLastError();
}

hipError_t launch_attn_bf16(const Geom& g, const void* q, const void* k, const void* vt, void* o, void* o_lo,
                            float* lse, const int32_t* row_ptr, const int32_t* col_idx, const float* shift,
                            int32_t* counters, const int32_t* order, const int32_t* bounds, int num_cu, hipStream_t s) {
  AttnBf16Args a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.vt = (const uint16_t*)vt;
  a.o = (uint16_t*)o;
  a.o_lo = (uint16_t*)o_lo;
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.shift = shift;
  a.counters = counters;
  a.order = order;
  a.bounds = bounds;
  a.g = g;
  a.c_log2 = (float)(1.4426950408889634 / sqrt((double)g.D));
  a.magic_wp = g.layout == 1 ? 0u : (uint32_t)((1ull << 31) / (uint64_t)g.Wp + 1);
  a.pxmul = g.layout == 1 ? 64 : 8;
  a.magic_hp = (uint32_t)((1ull << 31) / (uint64_t)g.Hp + 1);
  a.pairs = (g.S + 1) / 2;
  a.items = (int32_t)((int64_t)g.B * g.nh * a.pairs);
  const int grid = ((num_cu * 2 + 7) / 8) * 8;   // two resident workgroups per CU, a multiple of 8 XCDs
  if (o_lo && shift) return hipErrorInvalidValue;   // the training variant takes unshifted masks only
  if (g.D == 64) {
    if (o_lo)
      attn_bf16_kernel<64, false, true><<<grid, 256, 0, s>>>(a);
    else if (shift)
      attn_bf16_kernel<64, true, false><<<grid, 256, 0, s>>>(a);
    else
      attn_bf16_kernel<64, false, false><<<grid, 256, 0, s>>>(a);
  } else {
    if (o_lo)
      attn_bf16_kernel<128, false, true><<<grid, 256, 0, s>>>(a);
    else if (shift)
      attn_bf16_kernel<128, true, false><<<grid, 256, 0, s>>>(a);
    else
      attn_bf16_kernel<128, false, false><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace bsa
