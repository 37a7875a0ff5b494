// Launchers of the HIP kernels (one translation unit per kernel family).
// Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "geom.h"

namespace bsa {

// Fractal flattening as a bit-exact copy of [B*nh, L, D] rows.
hipError_t launch_permute(const Geom& g, const void* x, void* y, int inverse, hipStream_t s);
// Bit-exact row copy through a device permutation table (any token order).
hipError_t launch_permute_table(const Geom& g, const int32_t* table, const void* x, void* y, int inverse,
                                hipStream_t s);
// V in the tensor's layout -> Vt [B*nh, S, D, 64] bf16: block-major, each
// block transposed to d-major with keys in MFMA operand order.
hipError_t launch_prep_vt(const Geom& g, const void* v, void* vt, hipStream_t s);
// Block means of Q and K in float64 -> qp, kp [B*nh, S, D].
hipError_t launch_pool(const Geom& g, const void* q, const void* k, double* qp, double* kp, hipStream_t s);
// Block logits z[bh, i, j] = qp_i . kp_j / sqrt(D) in float64.
hipError_t launch_block_logits(const Geom& g, const double* qp, const double* kp, double* z, hipStream_t s);
// Row softmax of z -> probs (inspection entry point).
hipError_t launch_block_softmax(const Geom& g, const double* z, double* probs, hipStream_t s);
// CDF cut + window union per row -> bitmap [rows, words] and kept counts [rows].
hipError_t launch_select(const Geom& g, const double* z, double thr, double lambda, int win_t, int win_h,
                         int win_w, uint32_t* bitmap, int32_t* counts, int words, hipStream_t s);
// SIP sampling per row (budget = counts on entry, the CDF cut's counts) -> bitmap,
// counts and (max, sum, c, top block) per row in rowstat [rows, 4].
hipError_t launch_sip(const Geom& g, const double* z, double thr, uint64_t seed, int win_t, int win_h, int win_w,
                      uint32_t* bitmap, int32_t* counts, double* rowstat, int words, hipStream_t s);
// Exclusive scan of counts -> row_ptr [rows+1]; row_ptr[rows] also copied to nnz (if not null).
// chunk_sums: ceil(rows/1024) ints of scratch.
hipError_t launch_scan(const Geom& g, const int32_t* counts, int32_t* row_ptr, int32_t* chunk_sums, int32_t* nnz,
                       hipStream_t s);
// Bitmap -> ascending col_idx at row_ptr offsets.
hipError_t launch_compact(const Geom& g, const uint32_t* bitmap, int words, const int32_t* row_ptr,
                          int32_t* col_idx, hipStream_t s);
// Compaction of a SIP bitmap, also writing each entry's logit shift log(1/pi).
hipError_t launch_compact_sip(const Geom& g, const uint32_t* bitmap, int words, const int32_t* row_ptr,
                              int32_t* col_idx, float* shift, const double* z, const double* rowstat, double thr,
                              int win_t, int win_h, int win_w, hipStream_t s);
// Block-sparse attention forward (shift: per-CSR-entry natural-log logit shift, or null).
// Work order of the bf16 attention kernel: per-item costs (cost: one int per
// item), the item order and the 9 XCD bounds (order: one int per item).
hipError_t launch_attn_schedule(const Geom& g, const int32_t* row_ptr, const int32_t* col_idx, int32_t* cost,
                                int32_t* order, int32_t* bounds, hipStream_t s);
// The same order from given per-item costs (each >= 1).
hipError_t launch_schedule_costs(const int32_t* cost, int items, int32_t* order, int32_t* bounds, hipStream_t s);
hipError_t launch_attn_bf16(const Geom& g, const void* q, const void* k, const void* vt, void* o, float* lse,
                            const int32_t* row_ptr, const int32_t* col_idx, const float* shift, int32_t* counters,
                            const int32_t* order, const int32_t* bounds, int num_cu, hipStream_t s);
hipError_t launch_attn_f32(const Geom& g, const float* q, const float* k, const float* v, float* o, float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, const float* shift, hipStream_t s);
// Backward: per-token (lse*log2e, dO.o) into ld, and the transposed mask's bitmap
// and per-key-block counts (scan and compact them to get the transposed CSR).
hipError_t launch_backward_prep(const Geom& g, const void* o, const void* dout, const float* lse, float2* ld,
                                const int32_t* row_ptr, const int32_t* col_idx, uint32_t* tbits, int words,
                                int32_t* tcounts, hipStream_t s);
// Backward: dQ over the CSR, dK/dV over the transposed CSR (qt, dot: prepared
// transposes of K, Q, dO for bf16; counters: 16 ints, zeroed).
hipError_t launch_backward(const Geom& g, const void* q, const void* k, const void* v, const void* dout,
                           const void* qt, const void* dot, const float2* ld, void* dq, void* dk,
                           void* dv, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* tcolptr,
                           const int32_t* trowidx, int32_t* counters, int32_t* cost, int32_t* order_q,
                           int32_t* order_k, int32_t* bounds, int num_cu, hipStream_t s);
// Logits of query-block means against Sk key columns (blocks or 4-token groups)
// for heads h0 .. h0+nheads-1; z holds those heads' rows only.
hipError_t launch_logits(const Geom& g, const double* qp, const double* kp, double* z, int Sk, int64_t h0,
                         int64_t nheads, hipStream_t s);
// 4-token key groups: float64 group means of k -> kg [B*nh, L/4, D].
hipError_t launch_pool_groups(const Geom& g, const void* k, double* kg, hipStream_t s);
// CDF cut + window union over the L/4 group logits of rows row0 .. row0+nrows-1
// (z: those rows, L/4 entries each) -> bitmap rows and kept counts.
hipError_t launch_group_select(const Geom& g, const double* z, int64_t row0, int64_t nrows, double thr,
                               double lambda, int win_t, int win_h, int win_w, uint32_t* bitmap, int32_t* counts,
                               int words, hipStream_t s);
int group_select_max_groups();
// V -> [B*nh, L/4, D, 4] bf16 (each group channel-major) for the gathered attention.
hipError_t launch_prep_vg(const Geom& g, const void* v, void* vg, hipStream_t s);
// Attention over a CSR of 4-token key groups (bf16 needs the prepared vg; f32 reads v).
hipError_t launch_attn_groups_bf16(const Geom& g, const void* q, const void* k, const void* vg, void* o, float* lse,
                                   const int32_t* row_ptr, const int32_t* col_idx, int32_t* counters, int32_t* cost,
                                   int32_t* order, int32_t* bounds, int num_cu, hipStream_t s);
hipError_t launch_attn_groups_f32(const Geom& g, const float* q, const float* k, const float* v, float* o,
                                  float* lse, const int32_t* row_ptr, const int32_t* col_idx, hipStream_t s);
// Zero a small device counter (a fill kernel, safe under stream capture).
hipError_t launch_zero_i32(int32_t* p, int n, hipStream_t s);

}  // namespace bsa
