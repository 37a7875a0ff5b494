// Host-only checks of libbsa's argument validation, workspace layouts and token
// order tables, built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py (plain g++, no GPU code).  Exits non-zero and
// prints the failing check on the first mismatch.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <string>
#include <vector>

#include "order.h"
#include "validate.h"

using namespace bsa;

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static bsa_problem prob(int B, int nh, int T, int H, int W, int D, int P = 8, int N = 64, int dtype = BSA_BF16,
                        int layout = BSA_LAYOUT_ORIGINAL) {
  bsa_problem p;
  p.batch = B; p.heads = nh; p.T = T; p.H = H; p.W = W; p.head_dim = D;
  p.patch = P; p.block = N; p.dtype = dtype; p.layout = layout;
  return p;
}

static int geom(const bsa_problem& p, Geom* g) {
  std::string msg;
  const int st = make_geom(&p, g, &msg);
  CHECK((st == BSA_OK) == msg.empty());
  return st;
}

// every region of a layout is 256-byte aligned, in increasing order, and inside the total
static void check_offsets(const std::vector<int64_t>& offs, int64_t total) {
  int64_t prev = 0;
  for (int64_t o : offs) {
    CHECK(o % 256 == 0);
    CHECK(o >= prev);
    CHECK(o <= total);
    prev = o;
  }
  CHECK(total % 256 == 0);
}

static void valid_problems() {
  const int shapes[][5] = {{1, 4, 4, 16, 16}, {1, 8, 8, 32, 32}, {1, 40, 21, 32, 48}, {2, 24, 33, 48, 80},
                           {1, 2, 2, 16, 8}, {1, 2, 3, 8, 24}, {1, 1, 16, 128, 128}};
  for (const auto& s : shapes) {
    for (int dtype : {BSA_F32, BSA_BF16}) {
      Geom g;
      bsa_problem p = prob(s[0], s[1], s[2], s[3], s[4], 128, 8, 64, dtype);
      CHECK(geom(p, &g) == BSA_OK);
      CHECK(g.L == s[2] * s[3] * s[4]);
      CHECK(g.S * 64 == g.L);
      CHECK(g.rows == (int64_t)s[0] * s[1] * g.S);
      const MaskWs m = mask_ws_layout(g);
      check_offsets({m.qp, m.kp, m.z, m.counts, m.bitmap, m.chunk_sums, m.rowstat, m.qs, m.ks, m.qmu, m.krec, m.qn,
                     m.qe, m.hstat, m.flags, m.nflag},
                    m.total);
      CHECK(m.words == (g.S + 31) / 32);
      const FwdWs f = fwd_ws_layout(g);
      check_offsets({f.counter, f.cost, f.order, f.vt}, f.total);
      const BwdWs b = bwd_ws_layout(g);
      check_offsets({b.delta, b.counter, b.bounds, b.cost, b.order_q, b.order_k, b.tcounts, b.tchunks, b.tbitmap,
                     b.tcolptr, b.trowidx}, b.total);
      CHECK(b.counter + 24 * 4 <= b.bounds);
      std::string msg;
      if (check_group(g, BSA_KEY_GROUP, &msg) == BSA_OK) {
        const GrpMaskWs gm = grp_mask_ws_layout(g);
        check_offsets({gm.qp, gm.zt, gm.qs, gm.ks, gm.qmu, gm.krec, gm.qn, gm.qe, gm.hstat, gm.flags, gm.nflag,
                       gm.zfb, gm.cn, gm.cab, gm.cjw, gm.counts, gm.bitmap, gm.chunk_sums}, gm.total);
        CHECK(gm.pitch % 32 == 0 && gm.pitch >= g.L / BSA_KEY_GROUP);
        CHECK(gm.chunk_heads >= 1);
        const GrpFwdWs gf = grp_fwd_ws_layout(g);
        check_offsets({gf.counter, gf.cost, gf.order, gf.vg}, gf.total);
      }
      bsa_mask_params mp{0.1, -1, -1, -1, BSA_MASK_CDF, 0};
      CHECK(check_mask_params(g, &mp, &msg) == BSA_OK);
      mp.win_t = mp.win_h = mp.win_w = 1;
      CHECK(check_mask_params(g, &mp, &msg) == BSA_OK);
    }
  }
}

static void rejected_problems() {
  Geom g;
  std::string msg;
  CHECK(make_geom(nullptr, &g, &msg) == BSA_ERR_INVALID_ARG);
  bsa_problem p = prob(1, 8, 8, 32, 32, 128);
  p.dtype = 7;
  CHECK(geom(p, &g) == BSA_ERR_DTYPE);
  p = prob(1, 8, 8, 32, 32, 128);
  p.layout = 2;
  CHECK(geom(p, &g) == BSA_ERR_INVALID_ARG);
  CHECK(geom(prob(0, 8, 8, 32, 32, 128), &g) == BSA_ERR_SHAPE);
  CHECK(geom(prob(1, 8, 8, -32, 32, 128), &g) == BSA_ERR_SHAPE);
  CHECK(geom(prob(1, 8, 8, 36, 32, 128), &g) == BSA_ERR_SHAPE);                 // H % P
  CHECK(geom(prob(1, 8, 1, 8, 24, 128, 8, 128), &g) == BSA_ERR_SHAPE);          // L % N
  CHECK(geom(prob(1, 8, 2, 16, 16, 128, 8, 128), &g) == BSA_ERR_UNSUPPORTED);   // N != 64
  CHECK(geom(prob(1, 8, 8, 32, 32, 128, 4, 64), &g) == BSA_ERR_UNSUPPORTED);    // original layout, P*P != N
  CHECK(geom(prob(1, 8, 8, 32, 32, 96), &g) == BSA_ERR_UNSUPPORTED);            // head_dim
  CHECK(geom(prob(1, 8, 8, 32, 32, 96, 8, 64, BSA_F32), &g) == BSA_ERR_UNSUPPORTED);
  CHECK(geom(prob(1, 1, 17, 128, 128, 128), &g) == BSA_ERR_UNSUPPORTED);        // S > 4096
  CHECK(geom(prob(200, 1000, 33, 48, 80, 128), &g) == BSA_ERR_UNSUPPORTED);     // int32 CSR offsets
  CHECK(geom(prob(2147483647, 2147483647, 1, 8, 8, 128), &g) == BSA_ERR_UNSUPPORTED);
  CHECK(geom(prob(1, 1, 2147483647, 2147483640, 2147483640, 128), &g) != BSA_OK);
  CHECK(geom(prob(1, 8, 8, 32, 32, 128), &g) == BSA_OK);
  const double bad_thr[] = {-0.1, 1.0, 1.5, std::numeric_limits<double>::quiet_NaN(),
                            std::numeric_limits<double>::infinity()};
  for (double t : bad_thr) {
    bsa_mask_params mp{t, -1, -1, -1, BSA_MASK_CDF, 0};
    CHECK(check_mask_params(g, &mp, &msg) == BSA_ERR_INVALID_ARG);
  }
  bsa_mask_params mp{0.1, 1, -1, 1, BSA_MASK_CDF, 0};
  CHECK(check_mask_params(g, &mp, &msg) == BSA_ERR_INVALID_ARG);   // mixed window signs
  mp = {0.1, -1, -1, -1, 9, 0};
  CHECK(check_mask_params(g, &mp, &msg) == BSA_ERR_INVALID_ARG);   // mode
  CHECK(check_mask_params(g, nullptr, &msg) == BSA_ERR_INVALID_ARG);
  Geom gf;
  CHECK(geom(prob(1, 8, 2, 32, 32, 128, 4, 64, BSA_BF16, BSA_LAYOUT_FRACTAL), &gf) == BSA_OK);
  mp = {0.1, 1, 1, 1, BSA_MASK_CDF, 0};
  CHECK(check_mask_params(gf, &mp, &msg) == BSA_ERR_UNSUPPORTED);  // window needs N == P*P
  CHECK(check_group(g, 8, &msg) == BSA_ERR_UNSUPPORTED);
}

static void order_tables() {
  const int grids[][4] = {{4, 16, 16, 8}, {3, 24, 40, 8}, {8, 32, 32, 4}, {4, 8, 8, 4}, {2, 16, 8, 8}, {5, 8, 24, 8}};
  for (const auto& gr : grids) {
    Geom g;
    CHECK(geom(prob(1, 1, gr[0], gr[1], gr[2], 128, gr[3], 64, BSA_BF16, BSA_LAYOUT_FRACTAL), &g) == BSA_OK);
    for (int order : {BSA_ORDER_FRACTAL, BSA_ORDER_TILE_MAJOR, BSA_ORDER_HILBERT}) {
      std::vector<int32_t> table((size_t)g.L, -1);
      std::string msg;
      const int st = order_table(g, order, table.data(), &msg);
      if (order == BSA_ORDER_TILE_MAJOR && g.T % (g.N / (g.P * g.P)) != 0) {
        CHECK(st == BSA_ERR_SHAPE);
        continue;
      }
      if (order == BSA_ORDER_FRACTAL && g.P * g.P != g.N) continue;
      CHECK(st == BSA_OK);
      std::vector<int> seen((size_t)g.L, 0);
      for (int32_t v : table) {
        CHECK(v >= 0 && v < g.L);
        if (v >= 0 && v < g.L) ++seen[(size_t)v];
      }
      for (int c : seen) CHECK(c == 1);
    }
    std::string msg;
    std::vector<int32_t> table((size_t)g.L);
    CHECK(order_table(g, 5, table.data(), &msg) == BSA_ERR_INVALID_ARG);
  }
}

int main() {
  valid_problems();
  rejected_problems();
  order_tables();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks ok\n");
  return 0;
}
