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
// Screen operands of the pooled blocks (see mask_screen.hip): fp16 hi / lo of the
// power-of-two scaled centred vectors ([rows][2][D]), channel means and scale
// exponents (key blocks: one (mean, exponent) pair per block), query-block norms,
// and per head (max mean, min mean, max norm) of the key blocks as
// order-preserving 64-bit keys.
struct ScreenOps {
  _Float16* qs;
  _Float16* ks;
  double* qmu;
  double2* krec;
  double* qn;
  int32_t* qe;
  uint64_t* hstat;
};
// Resets the per-head statistics of the screen and the flagged-row count.
hipError_t launch_screen_init(const Geom& g, const ScreenOps& ops, int32_t* nflag, hipStream_t s);
// launch_pool plus the screen operands in the same pass (after launch_screen_init).
hipError_t launch_pool_screen(const Geom& g, const void* q, const void* k, double* qp, double* kp,
                              const ScreenOps& ops, hipStream_t s);
// The query half of launch_pool_screen only (qp and the query screen operands).
hipError_t launch_pool_queries_screen(const Geom& g, const void* q, double* qp, const ScreenOps& ops, hipStream_t s);
// Screened reduced map + CDF cut + window union -> bitmap rows and counts; rows it
// cannot decide are appended to flag_list (count in nflag) for the float64 path.
hipError_t launch_screen_select(const Geom& g, const ScreenOps& ops, const double* qp, const double* kp, double thr,
                                double lambda, int win_t, int win_h, int win_w, uint32_t* bitmap, int32_t* counts,
                                int words, int32_t* flag_list, int32_t* nflag, hipStream_t s);
// The float64 cut of the listed rows (float64 logits computed per row on the fly).
hipError_t launch_fallback_select(const Geom& g, const double* qp, const double* kp, double thr, double lambda,
                                  int win_t, int win_h, int win_w, uint32_t* bitmap, int32_t* counts, int words,
                                  const int32_t* flag_list, const int32_t* nflag, hipStream_t s);
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
// Work order over items of nb adjacent query blocks (2 for the bf16 forward and
// the backward): per-item costs (cost: one int per item), the item order and the 9
// XCD bounds (order: one int per item).
hipError_t launch_attn_schedule(const Geom& g, const int32_t* row_ptr, const int32_t* col_idx, int32_t* cost,
                                int32_t* order, int32_t* bounds, hipStream_t s, int nb);
// The same order from given per-item costs (each >= 1).
hipError_t launch_schedule_costs(const int32_t* cost, int items, int32_t* order, int32_t* bounds, hipStream_t s);
// o_lo non-null: the training variant (P as a bf16 pair in the PV product, O
// normalised by the float32 sum of P, O - bf16(O) written to o_lo; shift must be null).
hipError_t launch_attn_bf16(const Geom& g, const void* q, const void* k, const void* vt, void* o, void* o_lo,
                            float* lse, const int32_t* row_ptr, const int32_t* col_idx, const float* shift,
                            int32_t* counters, const int32_t* order, const int32_t* bounds, int num_cu, hipStream_t s);
hipError_t launch_attn_f32(const Geom& g, const float* q, const float* k, const float* v, float* o, float* lse,
                           const int32_t* row_ptr, const int32_t* col_idx, const float* shift, hipStream_t s);
// Backward: per-token lse*log2e into ld (.x), and the transposed mask's bitmap
// and per-key-block counts (scan and compact them to get the transposed CSR).
hipError_t launch_backward_prep(const Geom& g, const float* lse, float2* ld, const int32_t* row_ptr,
                                const int32_t* col_idx, uint32_t* tbits, int words, int32_t* tcounts, hipStream_t s);
// Backward: the row term Delta (into ld .y) and dQ over the CSR, dK/dV over the
// transposed CSR (qt, dot: prepared transposes of Q, dO for bf16; counters: 24
// ints, zeroed).
// Backward of the training pair: the row term from the forward's output instead
// of the Delta walk, Delta = dO . (o + o_lo) per token (into ld .y; bf16, D = 128).
hipError_t launch_delta_from_output(const Geom& g, const void* o, const void* o_lo, const void* dout, float2* ld,
                                   hipStream_t s);
hipError_t launch_backward(const Geom& g, const void* q, const void* k, const void* v, const void* dout,
                           float2* ld, void* dq, void* dk,
                           void* dv, const int32_t* row_ptr, const int32_t* col_idx, const int32_t* tcolptr,
                           const int32_t* trowidx, int32_t* counters, int32_t* cost, int32_t* order_q,
                           int32_t* order_k, int32_t* bounds, int num_cu, bool delta_walk, hipStream_t s);
// 4-token key groups (group_screen.hip): the screen operands of the group means
// (ops.ks in 16-group MFMA tiles, ops.krec (mean, exponent) per group, ops.hstat per
// head; after launch_screen_init).
hipError_t launch_pool_groups_screen(const Geom& g, const void* k, const ScreenOps& ops, hipStream_t s);
// Screened group map of heads h0 .. h0+nheads-1 as float32 offsets from each row's
// upper bound in log2 units: zt [nheads*S, pitch] (pitch: L/4 rounded up to a
// multiple of 32).
hipError_t launch_group_logits_screen(const Geom& g, const ScreenOps& ops, float* zt, int64_t h0, int64_t nheads,
                                      int pitch, hipStream_t s);
// CDF cut + window union of rows row0 .. row0+nrows-1 from their screened offsets
// (zt: those rows) -> bitmap rows; rows it cannot decide are appended to flag_list
// (count in nflag) for launch_group_fallback.
// Per row: the number of entries the screened cut left inside its error margin
// (cn), the mass above them and the target (cab), and the entries (cjw: up to 64
// (group id, mass) pairs per row).
struct GroupRankBufs {
  int32_t* cn;
  double2* cab;
  uint2* cjw;
};
hipError_t launch_group_screen_select(const Geom& g, const float* zt, int pitch, const ScreenOps& ops, int64_t row0,
                                      int64_t nrows, double thr, int win_t, int win_h, int win_w, uint32_t* bitmap,
                                      int words, int32_t* flag_list, int32_t* nflag, const GroupRankBufs& rb,
                                      hipStream_t s);
// Exact ranking of the entries the screened cut handed over (every row; k: the keys).
hipError_t launch_group_rank(const Geom& g, const GroupRankBufs& rb, const double* qp, const void* k,
                             uint32_t* bitmap, int words, hipStream_t s);
// Kept counts of rows from their bitmap rows (one wavefront per row).
hipError_t launch_bitmap_counts(const uint32_t* bitmap, int words, int64_t rows, int32_t* counts, hipStream_t s);
// The float64 cut of the listed rows (group_mask.hip); zscr: kGroupFallbackRows
// rows of L/4 doubles.
hipError_t launch_group_fallback(const Geom& g, const double* qp, const void* k, double* zscr, double thr,
                                 double lambda, int win_t, int win_h, int win_w, uint32_t* bitmap, int32_t* counts,
                                 int words, const int32_t* flag_list, const int32_t* nflag, hipStream_t s);
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
