// Host-side argument checks and workspace layout (plain C++, no HIP calls).
#pragma once
#include <stdint.h>
#include <string>

#include "bsa.h"
#include "geom.h"

namespace bsa {

// Fills g from p; returns a bsa status and a message on failure.
int make_geom(const bsa_problem* p, Geom* g, std::string* msg);
int check_mask_params(const Geom& g, const bsa_mask_params* mp, std::string* msg);

struct MaskWs {       // byte offsets into the mask workspace
  int64_t qp, kp, z, counts, bitmap, chunk_sums, rowstat, total;   // rowstat: SIP (max, sum, c, top) per row
  // screened cut: fp16 operands, means, norms, exponents, per-head stats, the list of
  // rows left to the float64 path and its length
  int64_t qs, ks, qmu, krec, qn, qe, hstat, flags, nflag;
  int32_t words;      // 32-bit words per bitmap row
};
struct FwdWs {         // work counters and XCD bounds, per-item costs and order (bf16), prepared V (bf16)
  int64_t counter, bounds, cost, order, vt, total;
};
struct BwdWs {        // transposed mask, per-token (lse*log2e, Delta), work counters and orders
  int64_t delta, counter, bounds, cost, order_q, order_k, tcounts, tchunks, tbitmap, tcolptr, trowidx, total;
  int32_t words;
};
// Workgroups of the key-group mask's float64 path, each with one float64 scratch row.
constexpr int kGroupFallbackRows = 256;
struct GrpMaskWs {     // key-group mask: query-block means, the screen operands, a head chunk of
                       // screened logits, the rows left to the float64 path and its scratch rows, bits
  int64_t qp, zt, qs, ks, qmu, krec, qn, qe, hstat, flags, nflag, zfb, cn, cab, cjw, counts, bitmap,
      chunk_sums, total;
  int64_t chunk_heads;  // heads whose group logits are computed together
  int32_t pitch;        // floats per screened row (L/4 rounded up to 32)
  int32_t words;        // 32-bit words per bitmap row (L/4 bits)
};
struct GrpFwdWs {      // work counters and XCD bounds, per-row cost and order (bf16), prepared V (bf16)
  int64_t counter, bounds, cost, order, vg, total;
};
// Checks the key-group size and the limits of the group path.
int check_group(const Geom& g, int group, std::string* msg);
GrpMaskWs grp_mask_ws_layout(const Geom& g);
GrpFwdWs grp_fwd_ws_layout(const Geom& g);
BwdWs bwd_ws_layout(const Geom& g);
MaskWs mask_ws_layout(const Geom& g);
FwdWs fwd_ws_layout(const Geom& g);

}  // namespace bsa
