// libbsa entry points: host-side validation, workspace carving and launches.
// Declarations and contracts: include/bsa.h.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>

#include "bsa.h"
#include "kernels.h"
#include "order.h"
#include "validate.h"

using namespace bsa;

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(BSA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Compute units of the current device, cached per device id.
int current_cu_count(int* out) {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(BSA_ERR_HIP, "device id out of range");
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    cache[dev] = n > 0 ? n : 1;
  }
  *out = cache[dev];
  return BSA_OK;
}

int geom_or_fail(const bsa_problem* p, Geom* g) {
  std::string msg;
  const int st = make_geom(p, g, &msg);
  if (st != BSA_OK) return fail(st, msg);
  return BSA_OK;
}

}  // namespace

extern "C" {

int bsa_version(void) { return 520; }

const char* bsa_status_str(int s) {
  switch (s) {
    case BSA_OK: return "BSA_OK";
    case BSA_ERR_INVALID_ARG: return "BSA_ERR_INVALID_ARG";
    case BSA_ERR_SHAPE: return "BSA_ERR_SHAPE";
    case BSA_ERR_DTYPE: return "BSA_ERR_DTYPE";
    case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
    case BSA_ERR_CAPACITY: return "BSA_ERR_CAPACITY";
    case BSA_ERR_WORKSPACE: return "BSA_ERR_WORKSPACE";
    case BSA_ERR_HIP: return "BSA_ERR_HIP";
    default: return "BSA_ERR_UNKNOWN";
  }
}

const char* bsa_last_error(void) { return g_last_error.c_str(); }

int bsa_query_sizes(const bsa_problem* p, int64_t* rows, int64_t* max_nnz, int64_t* mask_ws, int64_t* fwd_ws) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (rows) *rows = g.rows;
  if (max_nnz) *max_nnz = g.rows * g.S;
  if (mask_ws) *mask_ws = mask_ws_layout(g).total;
  if (fwd_ws) *fwd_ws = fwd_ws_layout(g).total;
  return BSA_OK;
}

int bsa_permute(const bsa_problem* p, const void* x, void* y, int inverse, hipStream_t stream) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (!x || !y) return fail(BSA_ERR_INVALID_ARG, "bsa_permute: null tensor pointer");
  if (!aligned(x, 16) || !aligned(y, 16)) return fail(BSA_ERR_INVALID_ARG, "bsa_permute: tensors must be 16-byte aligned");
  if (x == y) return fail(BSA_ERR_INVALID_ARG, "bsa_permute: in-place permutation is not supported");
  hipError_t e = launch_permute(g, x, y, inverse, stream);
  if (e != hipSuccess) return hip_fail(e, "permute launch");
  return BSA_OK;
}

int bsa_order_table(const bsa_problem* p, int order, int32_t* table) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (!table) return fail(BSA_ERR_INVALID_ARG, "bsa_order_table: null table");
  std::string msg;
  st = order_table(g, order, table, &msg);
  if (st != BSA_OK) return fail(st, "bsa_order_table: " + msg);
  return BSA_OK;
}

int bsa_permute_table(const bsa_problem* p, const int32_t* table, const void* x, void* y, int inverse,
                      hipStream_t stream) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (!table || !x || !y) return fail(BSA_ERR_INVALID_ARG, "bsa_permute_table: null pointer");
  if (!aligned(table, 4) || !aligned(x, 16) || !aligned(y, 16))
    return fail(BSA_ERR_INVALID_ARG, "bsa_permute_table: misaligned pointer");
  if (x == y) return fail(BSA_ERR_INVALID_ARG, "bsa_permute_table: in-place permutation is not supported");
  hipError_t e = launch_permute_table(g, table, x, y, inverse, stream);
  if (e != hipSuccess) return hip_fail(e, "permute_table launch");
  return BSA_OK;
}

int bsa_pool(const bsa_problem* p, const void* q, const void* k, double* qp, double* kp, hipStream_t stream) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !qp || !kp) return fail(BSA_ERR_INVALID_ARG, "bsa_pool: null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(qp, 8) || !aligned(kp, 8))
    return fail(BSA_ERR_INVALID_ARG, "bsa_pool: misaligned pointer");
  hipError_t e = launch_pool(g, q, k, qp, kp, stream);
  if (e != hipSuccess) return hip_fail(e, "pool launch");
  return BSA_OK;
}

int bsa_block_map(const bsa_problem* p, const double* qp, const double* kp, double* probs, hipStream_t stream) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (!qp || !kp || !probs) return fail(BSA_ERR_INVALID_ARG, "bsa_block_map: null pointer");
  if (!aligned(qp, 16) || !aligned(kp, 16) || !aligned(probs, 8))
    return fail(BSA_ERR_INVALID_ARG, "bsa_block_map: misaligned pointer");
  hipError_t e = launch_block_logits(g, qp, kp, probs, stream);
  if (e != hipSuccess) return hip_fail(e, "block logits launch");
  e = launch_block_softmax(g, probs, probs, stream);
  if (e != hipSuccess) return hip_fail(e, "block softmax launch");
  return BSA_OK;
}

int bsa_build_mask(const bsa_problem* p, const bsa_mask_params* mp, const void* q, const void* k, const bsa_csr* out,
                   void* ws, int64_t ws_bytes, hipStream_t stream) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  std::string msg;
  st = check_mask_params(g, mp, &msg);
  if (st != BSA_OK) return fail(st, msg);
  if (!q || !k || !out || !out->row_ptr || !out->col_idx)
    return fail(BSA_ERR_INVALID_ARG, "bsa_build_mask: null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(out->row_ptr, 4) || !aligned(out->col_idx, 4))
    return fail(BSA_ERR_INVALID_ARG, "bsa_build_mask: misaligned pointer");
  const bool sip = mp->mode == BSA_MASK_SIP;
  if (sip && (!out->shift || !aligned(out->shift, 4)))
    return fail(BSA_ERR_INVALID_ARG, "bsa_build_mask: SIP mode needs a 4-byte aligned shift array");
  if (out->capacity < g.rows * g.S)
    return fail(BSA_ERR_CAPACITY, "bsa_build_mask: col_idx capacity " + std::to_string(out->capacity) +
                                      " < batch*heads*S*S = " + std::to_string(g.rows * g.S));
  const MaskWs w = mask_ws_layout(g);
  if (!ws || ws_bytes < w.total)
    return fail(BSA_ERR_WORKSPACE, "bsa_build_mask: workspace needs " + std::to_string(w.total) + " bytes");
  if (!aligned(ws, 256)) return fail(BSA_ERR_WORKSPACE, "bsa_build_mask: workspace must be 256-byte aligned");
  char* base = static_cast<char*>(ws);
  double* qp = reinterpret_cast<double*>(base + w.qp);
  double* kp = reinterpret_cast<double*>(base + w.kp);
  double* z = reinterpret_cast<double*>(base + w.z);
  int32_t* counts = reinterpret_cast<int32_t*>(base + w.counts);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + w.bitmap);
  const bool win = mp->win_t >= 0;
  // Candidates for the sort: blocks within lambda of the row's max logit.  The
  // rest carry total mass < S * exp(-lambda) = 1e-17 * thr (see select_kernel).
  const double lambda = mp->thr > 0.0 ? 40.0 + std::log((double)g.S) - std::log(mp->thr) : 0.0;
  const int wt = win ? mp->win_t : -1, wh = win ? mp->win_h : -1, ww = win ? mp->win_w : -1;
  double* rowstat = reinterpret_cast<double*>(base + w.rowstat);
  hipError_t e = hipSuccess;
  if (!sip) {
    // the screened cut keeps the map on chip; rows it cannot decide take the float64 path
    ScreenOps ops;
    ops.qs = reinterpret_cast<_Float16*>(base + w.qs);
    ops.ks = reinterpret_cast<_Float16*>(base + w.ks);
    ops.qmu = reinterpret_cast<double*>(base + w.qmu);
    ops.krec = reinterpret_cast<double2*>(base + w.krec);
    ops.qn = reinterpret_cast<double*>(base + w.qn);
    ops.qe = reinterpret_cast<int32_t*>(base + w.qe);
    ops.hstat = reinterpret_cast<uint64_t*>(base + w.hstat);
    int32_t* flags = reinterpret_cast<int32_t*>(base + w.flags);
    int32_t* nflag = reinterpret_cast<int32_t*>(base + w.nflag);
    e = launch_screen_init(g, ops, nflag, stream);
    if (e == hipSuccess) e = launch_pool_screen(g, q, k, qp, kp, ops, stream);
    if (e == hipSuccess)
      e = launch_screen_select(g, ops, qp, kp, mp->thr, lambda, wt, wh, ww, bitmap, counts, w.words, flags, nflag,
                               stream);
    if (e == hipSuccess)
      e = launch_fallback_select(g, qp, kp, mp->thr, lambda, wt, wh, ww, bitmap, counts, w.words, flags, nflag,
                                 stream);
  } else {
    // SIP: the float64 map and the CDF cut without the window give each row's
    // budget, then the sampling replaces the bitmap and unions the window
    e = launch_pool(g, q, k, qp, kp, stream);
    if (e == hipSuccess) e = launch_block_logits(g, qp, kp, z, stream);
    if (e == hipSuccess) e = launch_select(g, z, mp->thr, lambda, -1, -1, -1, bitmap, counts, w.words, stream);
    if (e == hipSuccess)
      e = launch_sip(g, z, mp->thr, mp->seed, wt, wh, ww, bitmap, counts, rowstat, w.words, stream);
  }
  if (e == hipSuccess)
    e = launch_scan(g, counts, out->row_ptr, reinterpret_cast<int32_t*>(base + w.chunk_sums), out->nnz, stream);
  if (e == hipSuccess && !sip) e = launch_compact(g, bitmap, w.words, out->row_ptr, out->col_idx, stream);
  if (e == hipSuccess && sip)
    e = launch_compact_sip(g, bitmap, w.words, out->row_ptr, out->col_idx, out->shift, z, rowstat, mp->thr, wt, wh,
                           ww, stream);
  if (e != hipSuccess) return hip_fail(e, "bsa_build_mask launch");
  return BSA_OK;
}

static int check_attend_args(const bsa_problem* p, Geom* g, const void* q, const void* k, const void* v,
                             const bsa_csr* mask, const void* o, const float* lse, void* ws, int64_t ws_bytes,
                             bool whole_forward, const char* who) {
  int st = geom_or_fail(p, g);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !o || !mask || !mask->row_ptr || !mask->col_idx)
    return fail(BSA_ERR_INVALID_ARG, std::string(who) + ": null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(mask->shift, 4))
    return fail(BSA_ERR_INVALID_ARG, std::string(who) + ": misaligned pointer");
  const FwdWs w = fwd_ws_layout(*g);
  const int64_t need = whole_forward ? w.total : w.vt;   // bsa_attend: counters and work order only
  if (!ws || ws_bytes < need)
    return fail(BSA_ERR_WORKSPACE, std::string(who) + ": workspace needs " + std::to_string(need) + " bytes");
  if (!aligned(ws, 256)) return fail(BSA_ERR_WORKSPACE, std::string(who) + ": workspace must be 256-byte aligned");
  return BSA_OK;
}

static int enqueue_attend(const Geom& g, const void* q, const void* k, const void* vp, const bsa_csr* mask, void* o,
                          float* lse, char* ws, hipStream_t stream, void* o_lo = nullptr) {
  const FwdWs w = fwd_ws_layout(g);
  hipError_t e;
  if (g.dtype == BSA_BF16) {
    int ncu = 0;
    const int st = current_cu_count(&ncu);
    if (st != BSA_OK) return st;
    int32_t* counter = reinterpret_cast<int32_t*>(ws + w.counter);
    int32_t* bounds = reinterpret_cast<int32_t*>(ws + w.bounds);
    int32_t* cost = reinterpret_cast<int32_t*>(ws + w.cost);
    int32_t* order = reinterpret_cast<int32_t*>(ws + w.order);
    e = launch_zero_i32(counter, 8, stream);   // one work counter per XCD
    if (e == hipSuccess) e = launch_attn_schedule(g, mask->row_ptr, mask->col_idx, cost, order, bounds, stream, 2);
    if (e == hipSuccess)
      e = launch_attn_bf16(g, q, k, vp, o, o_lo, lse, mask->row_ptr, mask->col_idx, mask->shift, counter, order,
                           bounds, ncu, stream);
  } else {
    e = launch_attn_f32(g, (const float*)q, (const float*)k, (const float*)vp, (float*)o, lse, mask->row_ptr,
                        mask->col_idx, mask->shift, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return BSA_OK;
}

int bsa_query_attend_ws(const bsa_problem* p, int64_t* attend_ws) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (!attend_ws) return fail(BSA_ERR_INVALID_ARG, "bsa_query_attend_ws: null output");
  *attend_ws = fwd_ws_layout(g).vt;
  return BSA_OK;
}

int bsa_query_backward_ws(const bsa_problem* p, int64_t* bwd_ws) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (!bwd_ws) return fail(BSA_ERR_INVALID_ARG, "bsa_query_backward_ws: null output");
  *bwd_ws = bwd_ws_layout(g).total;
  return BSA_OK;
}

// Shared by bsa_backward (o == NULL: the Delta walk) and bsa_backward_train
// (Delta = dO . (o + o_lo) from the training forward's output pair).
static int backward_impl(const bsa_problem* p, const void* q, const void* k, const void* v, const bsa_csr* mask,
                         const void* o, const void* o_lo, const float* lse, const void* dout, void* dq, void* dk,
                         void* dv, void* ws, int64_t ws_bytes, hipStream_t stream, const char* who) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  const std::string name(who);
  if (!q || !k || !v || !lse || !dout || !dq || !dk || !dv || !mask || !mask->row_ptr || !mask->col_idx)
    return fail(BSA_ERR_INVALID_ARG, name + ": null pointer");
  const bool from_output = o != nullptr;
  if (from_output && !o_lo) return fail(BSA_ERR_INVALID_ARG, name + ": null pointer");
  const void* t16[] = {q, k, v, dout, dq, dk, dv, from_output ? o : q, from_output ? o_lo : q};
  for (const void* t : t16)
    if (!aligned(t, 16)) return fail(BSA_ERR_INVALID_ARG, name + ": tensors must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(BSA_ERR_INVALID_ARG, name + ": misaligned lse");
  if (mask->shift) return fail(BSA_ERR_UNSUPPORTED, name + ": masks with logit shifts are not supported");
  if (from_output && g.dtype != BSA_BF16)
    return fail(BSA_ERR_UNSUPPORTED, name + ": the training pair is bf16 only (float32 uses bsa_backward)");
  if (g.dtype == BSA_BF16 && g.D != 128)
    return fail(BSA_ERR_UNSUPPORTED, name + ": bf16 head_dim " + std::to_string(g.D) +
                                         " (only 128 is implemented; float32 supports 64 and 128)");
  const BwdWs w = bwd_ws_layout(g);
  if (!ws || ws_bytes < w.total)
    return fail(BSA_ERR_WORKSPACE, name + ": workspace needs " + std::to_string(w.total) + " bytes");
  if (!aligned(ws, 256)) return fail(BSA_ERR_WORKSPACE, name + ": workspace must be 256-byte aligned");
  int ncu = 0;
  if (g.dtype == BSA_BF16) {
    st = current_cu_count(&ncu);
    if (st != BSA_OK) return st;
  }
  char* base = static_cast<char*>(ws);
  float2* ld = reinterpret_cast<float2*>(base + w.delta);
  int32_t* counters = reinterpret_cast<int32_t*>(base + w.counter);
  int32_t* tcounts = reinterpret_cast<int32_t*>(base + w.tcounts);
  uint32_t* tbits = reinterpret_cast<uint32_t*>(base + w.tbitmap);
  int32_t* tcolptr = reinterpret_cast<int32_t*>(base + w.tcolptr);
  int32_t* trowidx = reinterpret_cast<int32_t*>(base + w.trowidx);
  hipError_t e = launch_backward_prep(g, lse, ld, mask->row_ptr, mask->col_idx, tbits, w.words, tcounts, stream);
  if (e == hipSuccess && from_output) e = launch_delta_from_output(g, o, o_lo, dout, ld, stream);
  if (e == hipSuccess)
    e = launch_scan(g, tcounts, tcolptr, reinterpret_cast<int32_t*>(base + w.tchunks), nullptr, stream);
  if (e == hipSuccess) e = launch_compact(g, tbits, w.words, tcolptr, trowidx, stream);
  if (e == hipSuccess) e = launch_zero_i32(counters, 24, stream);
  if (e == hipSuccess)
    e = launch_backward(g, q, k, v, dout, ld, dq, dk, dv, mask->row_ptr,
                        mask->col_idx, tcolptr, trowidx, counters, reinterpret_cast<int32_t*>(base + w.cost),
                        reinterpret_cast<int32_t*>(base + w.order_q), reinterpret_cast<int32_t*>(base + w.order_k),
                        reinterpret_cast<int32_t*>(base + w.bounds), ncu, !from_output, stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return BSA_OK;
}

int bsa_backward(const bsa_problem* p, const void* q, const void* k, const void* v, const bsa_csr* mask,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws, int64_t ws_bytes,
                 hipStream_t stream) {
  return backward_impl(p, q, k, v, mask, nullptr, nullptr, lse, dout, dq, dk, dv, ws, ws_bytes, stream,
                       "bsa_backward");
}

int bsa_backward_train(const bsa_problem* p, const void* q, const void* k, const void* v, const bsa_csr* mask,
                       const void* o, const void* o_lo, const float* lse, const void* dout, void* dq, void* dk,
                       void* dv, void* ws, int64_t ws_bytes, hipStream_t stream) {
  if (!o) return fail(BSA_ERR_INVALID_ARG, "bsa_backward_train: null pointer");
  return backward_impl(p, q, k, v, mask, o, o_lo, lse, dout, dq, dk, dv, ws, ws_bytes, stream,
                       "bsa_backward_train");
}

int bsa_prepare_v(const bsa_problem* p, const void* v, void* vt, hipStream_t stream) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (g.dtype != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "bsa_prepare_v: only bf16 uses a prepared V");
  if (!v || !vt) return fail(BSA_ERR_INVALID_ARG, "bsa_prepare_v: null pointer");
  if (!aligned(v, 16) || !aligned(vt, 16)) return fail(BSA_ERR_INVALID_ARG, "bsa_prepare_v: misaligned pointer");
  if (v == vt) return fail(BSA_ERR_INVALID_ARG, "bsa_prepare_v: v and vt must not alias");
  hipError_t e = launch_prep_vt(g, v, vt, stream);
  if (e != hipSuccess) return hip_fail(e, "prepare_v launch");
  return BSA_OK;
}

int bsa_attend(const bsa_problem* p, const void* q, const void* k, const void* vp, const bsa_csr* mask, void* o,
               float* lse, void* ws, int64_t ws_bytes, hipStream_t stream) {
  Geom g;
  int st = check_attend_args(p, &g, q, k, vp, mask, o, lse, ws, ws_bytes, false, "bsa_attend");
  if (st != BSA_OK) return st;
  return enqueue_attend(g, q, k, vp, mask, o, lse, static_cast<char*>(ws), stream);
}

int bsa_attend_train(const bsa_problem* p, const void* q, const void* k, const void* vp, const bsa_csr* mask,
                     void* o, void* o_lo, float* lse, void* ws, int64_t ws_bytes, hipStream_t stream) {
  Geom g;
  int st = check_attend_args(p, &g, q, k, vp, mask, o, lse, ws, ws_bytes, false, "bsa_attend_train");
  if (st != BSA_OK) return st;
  if (!o_lo || !lse) return fail(BSA_ERR_INVALID_ARG, "bsa_attend_train: null pointer");
  if (!aligned(o_lo, 16)) return fail(BSA_ERR_INVALID_ARG, "bsa_attend_train: misaligned pointer");
  if (g.dtype != BSA_BF16)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_train: bf16 only (the float32 path is float64-accurate already)");
  if (mask->shift) return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_train: masks with logit shifts are not supported");
  return enqueue_attend(g, q, k, vp, mask, o, lse, static_cast<char*>(ws), stream, o_lo);
}

int bsa_forward(const bsa_problem* p, const void* q, const void* k, const void* v, const bsa_csr* mask, void* o,
                float* lse, void* ws, int64_t ws_bytes, hipStream_t stream) {
  Geom g;
  int st = check_attend_args(p, &g, q, k, v, mask, o, lse, ws, ws_bytes, true, "bsa_forward");
  if (st != BSA_OK) return st;
  char* base = static_cast<char*>(ws);
  const void* vp = v;
  if (g.dtype == BSA_BF16) {
    void* vt = base + fwd_ws_layout(g).vt;
    hipError_t e = launch_prep_vt(g, v, vt, stream);
    if (e != hipSuccess) return hip_fail(e, "prepare_v launch");
    vp = vt;
  }
  return enqueue_attend(g, q, k, vp, mask, o, lse, base, stream);
}

// ---- 4-token key groups --------------------------------------------------
static int group_geom(const bsa_problem* p, int group, Geom* g) {
  int st = geom_or_fail(p, g);
  if (st != BSA_OK) return st;
  std::string msg;
  st = check_group(*g, group, &msg);
  if (st != BSA_OK) return fail(st, msg);
  return BSA_OK;
}

int bsa_query_group_sizes(const bsa_problem* p, int group, int64_t* max_nnz, int64_t* mask_ws, int64_t* fwd_ws) {
  Geom g;
  int st = group_geom(p, group, &g);
  if (st != BSA_OK) return st;
  if (max_nnz) *max_nnz = g.rows * (g.L / BSA_KEY_GROUP);
  if (mask_ws) *mask_ws = grp_mask_ws_layout(g).total;
  if (fwd_ws) *fwd_ws = grp_fwd_ws_layout(g).total;
  return BSA_OK;
}

int bsa_build_group_mask(const bsa_problem* p, int group, const bsa_mask_params* mp, const void* q, const void* k,
                         const bsa_csr* out, void* ws, int64_t ws_bytes, hipStream_t stream) {
  Geom g;
  int st = group_geom(p, group, &g);
  if (st != BSA_OK) return st;
  std::string msg;
  st = check_mask_params(g, mp, &msg);
  if (st != BSA_OK) return fail(st, msg);
  if (mp->mode != BSA_MASK_CDF) return fail(BSA_ERR_UNSUPPORTED, "bsa_build_group_mask: only BSA_MASK_CDF");
  const int64_t SG = g.L / BSA_KEY_GROUP;
  if (SG > group_select_max_groups())
    return fail(BSA_ERR_UNSUPPORTED, "bsa_build_group_mask: L/4 = " + std::to_string(SG) + " groups per head exceeds " +
                                         std::to_string(group_select_max_groups()));
  if (!q || !k || !out || !out->row_ptr || !out->col_idx)
    return fail(BSA_ERR_INVALID_ARG, "bsa_build_group_mask: null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(out->row_ptr, 4) || !aligned(out->col_idx, 4))
    return fail(BSA_ERR_INVALID_ARG, "bsa_build_group_mask: misaligned pointer");
  if (out->capacity < g.rows * SG)
    return fail(BSA_ERR_CAPACITY, "bsa_build_group_mask: col_idx capacity " + std::to_string(out->capacity) +
                                      " < batch*heads*S*(L/4) = " + std::to_string(g.rows * SG));
  const GrpMaskWs w = grp_mask_ws_layout(g);
  if (!ws || ws_bytes < w.total)
    return fail(BSA_ERR_WORKSPACE, "bsa_build_group_mask: workspace needs " + std::to_string(w.total) + " bytes");
  if (!aligned(ws, 256)) return fail(BSA_ERR_WORKSPACE, "bsa_build_group_mask: workspace must be 256-byte aligned");
  char* base = static_cast<char*>(ws);
  double* qp = reinterpret_cast<double*>(base + w.qp);
  float* zt = reinterpret_cast<float*>(base + w.zt);
  int32_t* counts = reinterpret_cast<int32_t*>(base + w.counts);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(base + w.bitmap);
  int32_t* flags = reinterpret_cast<int32_t*>(base + w.flags);
  int32_t* nflag = reinterpret_cast<int32_t*>(base + w.nflag);
  ScreenOps ops{reinterpret_cast<_Float16*>(base + w.qs), reinterpret_cast<_Float16*>(base + w.ks),
                reinterpret_cast<double*>(base + w.qmu),  reinterpret_cast<double2*>(base + w.krec),
                reinterpret_cast<double*>(base + w.qn),   reinterpret_cast<int32_t*>(base + w.qe),
                reinterpret_cast<uint64_t*>(base + w.hstat)};
  const GroupRankBufs rb{reinterpret_cast<int32_t*>(base + w.cn), reinterpret_cast<double2*>(base + w.cab),
                         reinterpret_cast<uint2*>(base + w.cjw)};
  const bool win = mp->win_t >= 0;
  // candidates: groups within lambda of the row's max logit (as in the block cut)
  const double lambda = mp->thr > 0.0 ? 40.0 + std::log((double)SG) - std::log(mp->thr) : 0.0;
  const int wt = win ? mp->win_t : -1, wh = win ? mp->win_h : -1, ww = win ? mp->win_w : -1;
  // query-block means and their screen operands, the groups' operands; then per
  // chunk of heads the screened map and the cut; the exact ranking of the entries
  // inside the cuts' margins, and the float64 cut of the rows the screen left
  hipError_t e = launch_screen_init(g, ops, nflag, stream);
  if (e == hipSuccess) e = launch_pool_queries_screen(g, q, qp, ops, stream);
  if (e == hipSuccess) e = launch_pool_groups_screen(g, k, ops, stream);
  const int64_t bh = (int64_t)g.B * g.nh;
  for (int64_t h0 = 0; h0 < bh && e == hipSuccess; h0 += w.chunk_heads) {
    const int64_t nh = std::min<int64_t>(w.chunk_heads, bh - h0);
    if (mp->thr > 0.0) e = launch_group_logits_screen(g, ops, zt, h0, nh, w.pitch, stream);
    if (e == hipSuccess)
      e = launch_group_screen_select(g, zt, w.pitch, ops, h0 * g.S, nh * g.S, mp->thr, wt, wh, ww, bitmap, w.words,
                                     flags, nflag, rb, stream);
  }
  if (e == hipSuccess && mp->thr > 0.0) e = launch_group_rank(g, rb, qp, k, bitmap, w.words, stream);
  if (e == hipSuccess && mp->thr > 0.0)
    e = launch_group_fallback(g, qp, k, reinterpret_cast<double*>(base + w.zfb), mp->thr, lambda, wt, wh, ww, bitmap,
                              counts, w.words, flags, nflag, stream);
  if (e == hipSuccess) e = launch_bitmap_counts(bitmap, w.words, g.rows, counts, stream);
  if (e == hipSuccess)
    e = launch_scan(g, counts, out->row_ptr, reinterpret_cast<int32_t*>(base + w.chunk_sums), out->nnz, stream);
  if (e == hipSuccess) {
    Geom gg = g;
    gg.S = (int32_t)SG;   // compaction walks L/4 columns per row (rows unchanged)
    e = launch_compact(gg, bitmap, w.words, out->row_ptr, out->col_idx, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "bsa_build_group_mask launch");
  return BSA_OK;
}

static int check_group_attend(const bsa_problem* p, int group, Geom* g, const void* q, const void* k, const void* v,
                              const bsa_csr* mask, const void* o, const float* lse, void* ws, int64_t ws_bytes,
                              bool whole, const char* who) {
  int st = group_geom(p, group, g);
  if (st != BSA_OK) return st;
  if (!q || !k || !v || !o || !mask || !mask->row_ptr || !mask->col_idx)
    return fail(BSA_ERR_INVALID_ARG, std::string(who) + ": null pointer");
  if (mask->shift) return fail(BSA_ERR_UNSUPPORTED, std::string(who) + ": group masks carry no logit shifts");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return fail(BSA_ERR_INVALID_ARG, std::string(who) + ": misaligned pointer");
  const GrpFwdWs w = grp_fwd_ws_layout(*g);
  const int64_t need = whole ? w.total : w.vg;
  if (!ws || ws_bytes < need)
    return fail(BSA_ERR_WORKSPACE, std::string(who) + ": workspace needs " + std::to_string(need) + " bytes");
  if (!aligned(ws, 256)) return fail(BSA_ERR_WORKSPACE, std::string(who) + ": workspace must be 256-byte aligned");
  return BSA_OK;
}

static int enqueue_attend_groups(const Geom& g, const void* q, const void* k, const void* vp, const bsa_csr* mask,
                                 void* o, float* lse, char* ws, hipStream_t stream) {
  const GrpFwdWs w = grp_fwd_ws_layout(g);
  hipError_t e;
  if (g.dtype == BSA_BF16) {
    int ncu = 0;
    const int st = current_cu_count(&ncu);
    if (st != BSA_OK) return st;
    int32_t* counter = reinterpret_cast<int32_t*>(ws + w.counter);
    e = launch_zero_i32(counter, 8, stream);
    if (e == hipSuccess)
      e = launch_attn_groups_bf16(g, q, k, vp, o, lse, mask->row_ptr, mask->col_idx, counter,
                                  reinterpret_cast<int32_t*>(ws + w.cost), reinterpret_cast<int32_t*>(ws + w.order),
                                  reinterpret_cast<int32_t*>(ws + w.bounds), ncu, stream);
  } else {
    e = launch_attn_groups_f32(g, (const float*)q, (const float*)k, (const float*)vp, (float*)o, lse, mask->row_ptr,
                               mask->col_idx, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "group attention launch");
  return BSA_OK;
}

int bsa_query_attend_groups_ws(const bsa_problem* p, int group, int64_t* attend_ws) {
  Geom g;
  int st = group_geom(p, group, &g);
  if (st != BSA_OK) return st;
  if (!attend_ws) return fail(BSA_ERR_INVALID_ARG, "bsa_query_attend_groups_ws: null output");
  *attend_ws = grp_fwd_ws_layout(g).vg;
  return BSA_OK;
}

int bsa_prepare_v_groups(const bsa_problem* p, int group, const void* v, void* vg, hipStream_t stream) {
  Geom g;
  int st = group_geom(p, group, &g);
  if (st != BSA_OK) return st;
  if (g.dtype != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "bsa_prepare_v_groups: only bf16 uses a prepared V");
  if (!v || !vg) return fail(BSA_ERR_INVALID_ARG, "bsa_prepare_v_groups: null pointer");
  if (!aligned(v, 16) || !aligned(vg, 16)) return fail(BSA_ERR_INVALID_ARG, "bsa_prepare_v_groups: misaligned pointer");
  if (v == vg) return fail(BSA_ERR_INVALID_ARG, "bsa_prepare_v_groups: v and vg must not alias");
  hipError_t e = launch_prep_vg(g, v, vg, stream);
  if (e != hipSuccess) return hip_fail(e, "prepare_v_groups launch");
  return BSA_OK;
}

int bsa_attend_groups(const bsa_problem* p, int group, const void* q, const void* k, const void* vp,
                      const bsa_csr* mask, void* o, float* lse, void* ws, int64_t ws_bytes, hipStream_t stream) {
  Geom g;
  int st = check_group_attend(p, group, &g, q, k, vp, mask, o, lse, ws, ws_bytes, false, "bsa_attend_groups");
  if (st != BSA_OK) return st;
  return enqueue_attend_groups(g, q, k, vp, mask, o, lse, static_cast<char*>(ws), stream);
}

int bsa_forward_groups(const bsa_problem* p, int group, const void* q, const void* k, const void* v,
                       const bsa_csr* mask, void* o, float* lse, void* ws, int64_t ws_bytes, hipStream_t stream) {
  Geom g;
  int st = check_group_attend(p, group, &g, q, k, v, mask, o, lse, ws, ws_bytes, true, "bsa_forward_groups");
  if (st != BSA_OK) return st;
  char* base = static_cast<char*>(ws);
  const void* vp = v;
  if (g.dtype == BSA_BF16) {
    void* vg = base + grp_fwd_ws_layout(g).vg;
    hipError_t e = launch_prep_vg(g, v, vg, stream);
    if (e != hipSuccess) return hip_fail(e, "prepare_v_groups launch");
    vp = vg;
  }
  return enqueue_attend_groups(g, q, k, vp, mask, o, lse, base, stream);
}

}  // extern "C"

// ---- attention with a static scratch buffer (no allocation) ---------------
// The work counters, XCD bounds and work order that bsa_attend keeps in its
// workspace argument live here in a file-scope device array instead.  In host
// code `g_attend_scratch` only names the symbol; its device address (one per
// GPU, each holding its own copy) comes from hipGetSymbolAddress on the first
// call on that device and is the only form passed to kernels.
namespace {

constexpr int64_t kAttendScratchBytes = int64_t(4) << 20;
__device__ __attribute__((aligned(256))) uint8_t g_attend_scratch[kAttendScratchBytes];

int attend_scratch(void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(BSA_ERR_HIP, "device id out of range");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_attend_scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(attend scratch)");
    addr[dev] = p;
  }
  *out = addr[dev];
  return BSA_OK;
}

}  // namespace

extern "C" int bsa_attend_static(const bsa_problem* p, const void* q, const void* k, const void* vp,
                                 const bsa_csr* mask, void* o, float* lse, hipStream_t stream) {
  Geom g;
  int st = geom_or_fail(p, &g);
  if (st != BSA_OK) return st;
  if (!q || !k || !vp || !o || !mask || !mask->row_ptr || !mask->col_idx)
    return fail(BSA_ERR_INVALID_ARG, "bsa_attend_static: null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(vp, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(mask->shift, 4))
    return fail(BSA_ERR_INVALID_ARG, "bsa_attend_static: misaligned pointer");
  const int64_t need = fwd_ws_layout(g).vt;
  if (need > kAttendScratchBytes)
    return fail(BSA_ERR_WORKSPACE, "bsa_attend_static: the problem needs " + std::to_string(need) +
                                       " bytes of scratch; the static scratch holds " +
                                       std::to_string(kAttendScratchBytes) + " (use bsa_attend with a workspace)");
  void* ws = nullptr;
  st = attend_scratch(&ws);
  if (st != BSA_OK) return st;
  return enqueue_attend(g, q, k, vp, mask, o, lse, static_cast<char*>(ws), stream);
}
