// Host-side validation and workspace layout for libbsa.  No HIP dependency:
// every rejection here happens before anything touches a GPU.
#include "validate.h"

#include <algorithm>
#include <cmath>
#include <cstdio>

namespace bsa {

static int fail(std::string* msg, int code, const char* fmt, long long a = 0, long long b = 0) {
  if (msg) {
    char buf[256];
    std::snprintf(buf, sizeof buf, fmt, a, b);
    *msg = buf;
  }
  return code;
}

int make_geom(const bsa_problem* p, Geom* g, std::string* msg) {
  if (!p || !g) return fail(msg, BSA_ERR_INVALID_ARG, "null problem pointer");
  if (p->dtype != BSA_F32 && p->dtype != BSA_BF16)
    return fail(msg, BSA_ERR_DTYPE, "dtype %lld is neither BSA_F32 nor BSA_BF16", p->dtype);
  if (p->layout != BSA_LAYOUT_ORIGINAL && p->layout != BSA_LAYOUT_FRACTAL)
    return fail(msg, BSA_ERR_INVALID_ARG, "layout %lld is not a valid layout", p->layout);
  if (p->batch <= 0 || p->heads <= 0 || p->T <= 0 || p->H <= 0 || p->W <= 0 ||
      p->head_dim <= 0 || p->patch <= 0 || p->block <= 0)
    return fail(msg, BSA_ERR_SHAPE, "all sizes must be positive");
  if (p->H % p->patch || p->W % p->patch)
    return fail(msg, BSA_ERR_SHAPE, "H=%lld and W=%lld must be multiples of the patch size", p->H, p->W);
  // T*H*W in two steps so that no product can overflow (each factor < 2^31)
  const long long TH = (long long)p->T * p->H;
  if (TH > (1LL << 30) || TH * p->W > (1LL << 30))
    return fail(msg, BSA_ERR_UNSUPPORTED, "T*H*W exceeds 2^30 tokens per head");
  const long long L = TH * p->W;
  if (L % p->block)
    return fail(msg, BSA_ERR_SHAPE, "L=%lld is not a multiple of the block size %lld", L, p->block);
  if (p->block != 64)
    return fail(msg, BSA_ERR_UNSUPPORTED, "block size %lld: only N = 64 is implemented", p->block);
  if (p->layout == BSA_LAYOUT_ORIGINAL && (long long)p->patch * p->patch != p->block)
    return fail(msg, BSA_ERR_UNSUPPORTED, "original layout needs P*P == N (P=%lld, N=%lld)", p->patch, p->block);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(msg, BSA_ERR_UNSUPPORTED, "head_dim %lld: only 64 and 128 are implemented", p->head_dim);
  const long long S = L / p->block;
  if (S > 4096)
    return fail(msg, BSA_ERR_UNSUPPORTED, "S=%lld blocks per head exceeds 4096", S);
  const long long bh = (long long)p->batch * p->heads;
  if (L > (1LL << 30) || bh > (1LL << 30) || bh * S * S >= (1LL << 31))
    return fail(msg, BSA_ERR_UNSUPPORTED, "batch*heads*S*S = %lld does not fit int32 CSR offsets", bh * S * S);
  g->B = p->batch; g->nh = p->heads; g->T = p->T; g->H = p->H; g->W = p->W;
  g->D = p->head_dim; g->P = p->patch; g->N = p->block;
  g->L = (int32_t)L; g->S = (int32_t)S; g->Hp = p->H / p->patch; g->Wp = p->W / p->patch;
  g->layout = p->layout; g->dtype = p->dtype; g->rows = bh * S;
  return BSA_OK;
}

int check_mask_params(const Geom& g, const bsa_mask_params* mp, std::string* msg) {
  if (!mp) return fail(msg, BSA_ERR_INVALID_ARG, "null mask params");
  if (!(mp->thr >= 0.0 && mp->thr < 1.0) || std::isnan(mp->thr))
    return fail(msg, BSA_ERR_INVALID_ARG, "thr must satisfy 0 <= thr < 1");
  if (mp->mode != BSA_MASK_CDF && mp->mode != BSA_MASK_SIP)
    return fail(msg, BSA_ERR_INVALID_ARG, "mode must be BSA_MASK_CDF or BSA_MASK_SIP");
  const int neg = (mp->win_t < 0) + (mp->win_h < 0) + (mp->win_w < 0);
  if (neg != 0 && neg != 3)
    return fail(msg, BSA_ERR_INVALID_ARG, "window extents must be all >= 0 (on) or all < 0 (off)");
  if (neg == 0 && g.P * g.P != g.N)
    return fail(msg, BSA_ERR_UNSUPPORTED, "the sliding-tile window needs N == P*P");
  return BSA_OK;
}

static int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

MaskWs mask_ws_layout(const Geom& g) {
  MaskWs w{};
  w.words = (g.S + 31) / 32;
  int64_t off = 0;
  w.qp = off; off = align256(off + g.rows * g.D * 8);
  w.kp = off; off = align256(off + g.rows * g.D * 8);
  w.z = off; off = align256(off + g.rows * (int64_t)g.S * 8);
  w.counts = off; off = align256(off + g.rows * 4);
  w.bitmap = off; off = align256(off + g.rows * (int64_t)w.words * 4);
  w.chunk_sums = off; off = align256(off + ((g.rows + 1023) / 1024) * 4);
  w.rowstat = off; off = align256(off + g.rows * 4 * 8);
  w.qs = off; off = align256(off + g.rows * 2 * g.D * 2);
  w.ks = off; off = align256(off + (int64_t)g.B * g.nh * ((g.S + 15) / 16) * 16 * 2 * g.D * 2);   // whole 16-block tiles
  w.qmu = off; off = align256(off + g.rows * 8);
  w.krec = off; off = align256(off + g.rows * 16);
  w.qn = off; off = align256(off + g.rows * 8);
  w.qe = off; off = align256(off + g.rows * 4);
  w.hstat = off; off = align256(off + (int64_t)g.B * g.nh * 3 * 8);
  w.flags = off; off = align256(off + g.rows * 4);
  w.nflag = off; off = align256(off + 4);
  w.total = off;
  return w;
}

FwdWs fwd_ws_layout(const Geom& g) {
  FwdWs w{};
  int64_t off = 0;
  w.counter = off;
  w.bounds = off + 64;
  off = align256(off + 128);
  const int64_t items = g.dtype == BSA_BF16 ? (int64_t)g.B * g.nh * ((g.S + 1) / 2) : 0;
  w.cost = off; off = align256(off + items * 4);
  w.order = off; off = align256(off + items * 4);
  w.vt = off;
  if (g.dtype == BSA_BF16) off = align256(off + (int64_t)g.B * g.nh * g.L * g.D * 2);
  w.total = off;
  return w;
}

BwdWs bwd_ws_layout(const Geom& g) {
  BwdWs w{};
  w.words = (g.S + 31) / 32;
  const int64_t tok = (int64_t)g.B * g.nh * g.L;
  int64_t off = 0;
  w.delta = off; off = align256(off + tok * 8);     // float2 per token
  w.counter = off; off = align256(off + 24 * 4);   // per-XCD item counters of the three passes
  w.bounds = off; off = align256(off + 32 * 4);   // two sets of 9 XCD bounds (at 0 and 16)
  const int64_t items = g.dtype == BSA_BF16 ? (int64_t)g.B * g.nh * ((g.S + 1) / 2) : 0;
  w.cost = off; off = align256(off + items * 4);
  w.order_q = off; off = align256(off + items * 4);
  w.order_k = off; off = align256(off + items * 4);
  w.tcounts = off; off = align256(off + g.rows * 4);
  w.tchunks = off; off = align256(off + ((g.rows + 1023) / 1024) * 4);
  w.tbitmap = off; off = align256(off + g.rows * (int64_t)w.words * 4);
  w.tcolptr = off; off = align256(off + (g.rows + 1) * 4);
  w.trowidx = off; off = align256(off + g.rows * (int64_t)g.S * 4);
  w.total = off;
  return w;
}

int check_group(const Geom& g, int group, std::string* msg) {
  if (group != BSA_KEY_GROUP)
    return fail(msg, BSA_ERR_UNSUPPORTED, "key group size %lld: only %lld is implemented", group, BSA_KEY_GROUP);
  if (g.dtype == BSA_BF16 && g.D != 128)
    return fail(msg, BSA_ERR_UNSUPPORTED, "bf16 key-group attention: head_dim %lld (only 128 is implemented)", g.D);
  const long long SG = g.L / BSA_KEY_GROUP;
  if (g.rows * SG >= (1LL << 31))
    return fail(msg, BSA_ERR_UNSUPPORTED,
                "batch*heads*S*(L/4) = %lld does not fit int32 CSR offsets (split the call by heads)", g.rows * SG);
  return BSA_OK;
}

GrpMaskWs grp_mask_ws_layout(const Geom& g) {
  GrpMaskWs w{};
  const int64_t SG = g.L / BSA_KEY_GROUP;
  const int64_t bh = (int64_t)g.B * g.nh;
  w.pitch = (int32_t)((SG + 31) / 32 * 32);
  const int64_t per_head = (int64_t)g.S * w.pitch * 4;      // one head's screened group logits
  const int64_t budget = int64_t(1) << 31;                  // at most ~2 GiB of them at a time
  w.chunk_heads = std::max<int64_t>(1, std::min<int64_t>(bh, budget / per_head));
  w.words = (int32_t)((SG + 31) / 32);
  int64_t off = 0;
  w.qp = off; off = align256(off + g.rows * g.D * 8);
  w.zt = off; off = align256(off + w.chunk_heads * per_head);
  w.qs = off; off = align256(off + g.rows * 2 * g.D * 2);
  w.ks = off; off = align256(off + bh * ((SG + 15) / 16) * 16 * 2 * g.D * 2);   // whole 16-group tiles
  w.qmu = off; off = align256(off + g.rows * 8);
  w.krec = off; off = align256(off + bh * SG * 16);
  w.qn = off; off = align256(off + g.rows * 8);
  w.qe = off; off = align256(off + g.rows * 4);
  w.hstat = off; off = align256(off + bh * 3 * 8);
  w.flags = off; off = align256(off + g.rows * 4);
  w.nflag = off; off = align256(off + 4);
  w.zfb = off; off = align256(off + (int64_t)kGroupFallbackRows * SG * 8);
  w.cn = off; off = align256(off + g.rows * 4);
  w.cab = off; off = align256(off + g.rows * 16);
  w.cjw = off; off = align256(off + g.rows * 64 * 8);
  w.counts = off; off = align256(off + g.rows * 4);
  w.bitmap = off; off = align256(off + g.rows * (int64_t)w.words * 4);
  w.chunk_sums = off; off = align256(off + ((g.rows + 1023) / 1024) * 4);
  w.total = off;
  return w;
}

GrpFwdWs grp_fwd_ws_layout(const Geom& g) {
  GrpFwdWs w{};
  int64_t off = 0;
  w.counter = off;
  w.bounds = off + 64;
  off = align256(off + 128);
  const int64_t items = g.dtype == BSA_BF16 ? g.rows : 0;
  w.cost = off; off = align256(off + items * 4);
  w.order = off; off = align256(off + items * 4);
  w.vg = off;
  if (g.dtype == BSA_BF16) off = align256(off + (int64_t)g.B * g.nh * g.L * g.D * 2);
  w.total = off;
  return w;
}

}  // namespace bsa
