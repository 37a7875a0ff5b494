/*
 * bsa.h -- C ABI of libbsa: content-adaptive block-sparse self-attention over
 * 3D video tokens on AMD Instinct MI355X (gfx950).
 *
 * The operation is the NABLA pipeline ("Resumen Tecnico: NABLA - Atencion de
 * Bloque Adaptativa al Vecindario para la Generacion Eficiente de Video",
 * gist.science/es/paper/2507.13546, section "Metodologia: NABLA"):
 *   1. fractal flattening of the T x H x W tokens (item 1),
 *   2. average pooling of Q and K into N-token blocks, a softmax map over the
 *      pooled blocks and a per-row CDF cut at mass 1 - thr (item 2, bullets
 *      "Submuestreo", "Atencion Reducida", "Umbralizacion CDF"),
 *   3. optional union with a static sliding-tile window (item 3),
 *   4. attention computed only on the kept N x N tiles (item 2, "Expansion").
 * The CDF mask is emitted as a CSR list of key blocks per query block, the
 * "skip list" form that the CalibAtt page ("Accelerating Text-to-Video
 * Generation with Calibrated Sparse Attention", gist.science/es/paper/2603.05503,
 * "Fase de Inferencia") feeds to its sparse kernel; any CSR, from any source,
 * can be passed to bsa_forward.
 *
 * Conventions shared by every call
 *   - Tensors Q, K, V, O are dense [batch, heads, L, head_dim], row-major,
 *     L = T*H*W, in the problem's dtype.  With layout BSA_LAYOUT_ORIGINAL the
 *     tokens are in (t, h, w) row-major order; with BSA_LAYOUT_FRACTAL they are
 *     already in fractal order.
 *   - Fractal order: position f = ((t*Hp + y/P)*Wp + x/P)*P*P + (y%P)*P + (x%P),
 *     Hp = H/P, Wp = W/P: frames outermost, P x P patches row-major inside a
 *     frame, tokens row-major inside a patch.  Block i = fractal tokens
 *     [i*N, (i+1)*N); S = L/N blocks per head.
 *   - CSR row r = (b*heads + h)*S + i lists the kept key blocks of query block i
 *     of head (b, h), ascending, as block ids in fractal order.
 *   - Every pointer argument except the problem/params structs and the
 *     workspace size is a DEVICE pointer unless stated otherwise; the caller
 *     owns all memory.  The library allocates nothing and keeps no state
 *     besides cached device properties; calls are reentrant.
 *   - Calls validate on the host, enqueue kernels on `stream` and return
 *     without synchronising.  Errors detected on the host return a status
 *     before anything is enqueued; a failed launch returns BSA_ERR_HIP.
 *     Asynchronous device faults surface at the caller's next synchronisation.
 *     No C++ exception crosses this interface.  bsa_last_error() returns a
 *     thread-local message describing the last non-OK status.
 *
 * Supported shapes (else BSA_ERR_SHAPE / BSA_ERR_UNSUPPORTED):
 *   N == 64; H % P == 0, W % P == 0, L % N == 0; layout ORIGINAL needs P*P == N;
 *   head_dim in {64, 128} (bf16 backward and bf16 key-group attention: 128 only); S <= 4096;
 *   batch*heads*S*S < 2^31 (int32 CSR offsets).
 */
#ifndef BSA_H
#define BSA_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1,   /* null pointer, bad enum, thr outside [0, 1) */
  BSA_ERR_SHAPE = 2,         /* sizes that do not tile (L % N, H % P, ...) */
  BSA_ERR_DTYPE = 3,         /* dtype not BSA_F32 / BSA_BF16 */
  BSA_ERR_UNSUPPORTED = 4,   /* valid but not implemented (head_dim, N, S) */
  BSA_ERR_CAPACITY = 5,      /* CSR col_idx capacity below batch*heads*S*S */
  BSA_ERR_WORKSPACE = 6,     /* workspace null or smaller than bsa_query_sizes says */
  BSA_ERR_HIP = 7            /* a HIP runtime call or kernel launch failed */
};

enum { BSA_F32 = 0, BSA_BF16 = 1 };
enum { BSA_LAYOUT_ORIGINAL = 0, BSA_LAYOUT_FRACTAL = 1 };

/* Problem description (host struct). */
typedef struct bsa_problem {
  int32_t batch, heads;      /* B, nh */
  int32_t T, H, W;           /* token grid; L = T*H*W */
  int32_t head_dim;          /* D */
  int32_t patch;             /* P, fractal patch side */
  int32_t block;             /* N, tokens per block */
  int32_t dtype;             /* BSA_F32 or BSA_BF16 */
  int32_t layout;            /* BSA_LAYOUT_ORIGINAL or BSA_LAYOUT_FRACTAL */
} bsa_problem;

/* Mask parameters (host struct).  thr in [0, 1): per row keep the shortest
 * prefix of key blocks, ordered by reduced-map probability descending (ties by
 * block index ascending), whose mass reaches 1 - thr; thr == 0 keeps every
 * block.  The sliding-tile window is enabled when win_t, win_h and win_w are
 * all >= 0: query tile (t, y, x) then also keeps every key tile (t', y', x')
 * with |t-t'| <= win_t, |y-y'| <= win_h, |x-x'| <= win_w (clipped, no wrap);
 * it needs N == P*P.  All three < 0 disables it; mixed signs are an error.
 *
 * mode BSA_MASK_SIP replaces the cut by sampling with inclusion-probability
 * weights (the SIP resource of the AB-Attention page, "AB-Attention acelera la
 * generacion de video hasta 2,23x y omite el 92% de la atencion",
 * news.hamidun.com/es/news/14960, section "Los tres recursos de AB-Attention"):
 * row i always takes its top block (largest reduced-map probability A_ij,
 * lowest j on ties) and samples every other block j independently with
 * probability
 *   pi_ij = min(1, c_i * A_ij),  c_i such that 1 + sum_{j != top} pi_ij = k_i,
 * where the budget k_i is the number of blocks the CDF cut above keeps for that
 * row (so the blocks with c_i * A_ij >= 1 are always taken too, and no row is
 * empty).  The Bernoulli draw uses u = (w >> 11) * 2^-53, w = word 0 of
 * Philox4x64-10 (Salmon et al., SC 2011) at counter (row, block, 0, 0) and key
 * (seed, 0); the block is taken iff u < pi.  Each taken block carries the
 * Horvitz-Thompson logit shift log(1 / pi) in the CSR's shift array, which
 * makes the attention numerator and normaliser unbiased.  Window blocks are
 * unioned afterwards with shift 0; thr == 0 keeps every block with shift 0. */
enum { BSA_MASK_CDF = 0, BSA_MASK_SIP = 1 };
typedef struct bsa_mask_params {
  double thr;
  int32_t win_t, win_h, win_w;
  int32_t mode;              /* BSA_MASK_CDF or BSA_MASK_SIP */
  uint64_t seed;             /* Philox key word 0 (BSA_MASK_SIP only) */
} bsa_mask_params;

/* CSR block mask (host struct holding device pointers). */
typedef struct bsa_csr {
  int32_t* row_ptr;          /* device, [rows + 1], row_ptr[0] = 0 */
  int32_t* col_idx;          /* device, [capacity] */
  int64_t capacity;          /* elements available in col_idx (and shift) */
  int32_t* nnz;              /* device scalar receiving row_ptr[rows]; may be NULL */
  float* shift;              /* device, [capacity], aligned with col_idx: natural-log
                                shift added to every logit of that tile.  Written by
                                bsa_build_mask in BSA_MASK_SIP mode (required there;
                                with BSA_MASK_CDF it is left untouched); read by
                                bsa_forward / bsa_attend when not NULL. */
} bsa_csr;

/* Sizes for a problem (all outputs are host pointers; any may be NULL).
 * rows = batch*heads*S; max_nnz = rows*S (the col_idx capacity bsa_build_mask
 * requires); mask_ws / fwd_ws = workspace bytes for bsa_build_mask /
 * bsa_forward.  Pure host computation; needs no GPU. */
int bsa_query_sizes(const bsa_problem* p, int64_t* rows, int64_t* max_nnz,
                    int64_t* mask_ws, int64_t* fwd_ws);

/* Fractal flattening (NABLA page, Metodologia item 1) as a bit-exact copy:
 * inverse == 0 maps original (t, h, w) order to fractal order, inverse != 0
 * maps back.  x, y: [batch, heads, L, head_dim] of p->dtype; must not overlap.
 * p->layout is ignored. */
int bsa_permute(const bsa_problem* p, const void* x, void* y, int inverse, hipStream_t stream);

/* Alternative token orders (drop-in variants of the fractal flattening).  A
 * caller permutes Q, K, V with bsa_permute_table into any of these orders and
 * runs the rest of the path with layout BSA_LAYOUT_FRACTAL, which means "block
 * i = positions [i*N, (i+1)*N) of the given order"; O comes back in that order
 * (bsa_permute_table with inverse != 0 restores (t, h, w) order).  The sliding-
 * tile window assumes the fractal order's block geometry and is meaningless in
 * the other orders.
 *   BSA_ORDER_FRACTAL    the NABLA fractal order (the same permutation as
 *                        bsa_permute);
 *   BSA_ORDER_TILE_MAJOR tiles of (N/P^2) x P x P tokens spanning N/P^2 frames
 *                        (tile-major layout of the TRA page, "Atencion de
 *                        Radio de Tokens", gist.science/es/paper/2608.02504,
 *                        "El Pipeline de TRA", item 3), tiles and
 *                        tokens row-major in (t, y, x); needs T % (N/P^2) == 0;
 *                        equals the fractal order when N == P*P;
 *   BSA_ORDER_HILBERT    increasing index along the 3D Hilbert curve of the
 *                        smallest 2^b cube holding the grid, axes (t, y, x),
 *                        Skilling's transpose form (DFSAttn page,
 *                        gist.science/es/paper/2605.23445, section 1).
 * bsa_order_table fills the HOST array table[L] with the original (t, h, w)
 * row-major index of the token at each position (pure host computation).
 * bsa_permute_table copies rows bit-exactly: inverse == 0 gives
 * y[b,h,f,:] = x[b,h,table[f],:], inverse != 0 the reverse scatter.  table is a
 * DEVICE array of L int32 that must be a permutation of [0, L) (entries are
 * clamped into range, so a malformed table yields wrong rows but no fault);
 * x, y must not overlap. */
enum { BSA_ORDER_FRACTAL = 0, BSA_ORDER_TILE_MAJOR = 1, BSA_ORDER_HILBERT = 2 };
int bsa_order_table(const bsa_problem* p, int order, int32_t* table);
int bsa_permute_table(const bsa_problem* p, const int32_t* table, const void* x, void* y, int inverse,
                      hipStream_t stream);

/* Block average pooling (Metodologia item 2, "Submuestreo"): qp[b,h,i,:] is the
 * mean of Q over the N tokens of fractal block i, likewise kp for K; outputs
 * are float64 [batch, heads, S, head_dim].  Inputs in p->layout order.  The
 * sums are accumulated in float64 (exact for bf16 inputs). */
int bsa_pool(const bsa_problem* p, const void* q, const void* k, double* qp, double* kp,
             hipStream_t stream);

/* Reduced map (Metodologia item 2, "Atencion Reducida"): probs[b,h,i,j] =
 * softmax_j(qp_i . kp_j / sqrt(head_dim)) in float64, from the outputs of
 * bsa_pool.  probs: [batch, heads, S, S] float64.  An inspection entry point:
 * bsa_build_mask never materialises this array. */
int bsa_block_map(const bsa_problem* p, const double* qp, const double* kp, double* probs,
                  hipStream_t stream);

/* Whole mask stage: pooling, reduced map, CDF cut (or SIP sampling, see
 * bsa_mask_params), optional window union and CSR compaction (Metodologia
 * items 2 and 3).  q, k in p->layout order.  out->row_ptr receives rows+1
 * offsets, out->col_idx the ascending kept block ids, out->nnz (if not NULL)
 * the total, and in SIP mode out->shift the per-entry logit shifts.  ws: device workspace of at least
 * mask_ws bytes (bsa_query_sizes), 256-byte aligned; its contents on entry do
 * not matter and are clobbered. */
int bsa_build_mask(const bsa_problem* p, const bsa_mask_params* mp, const void* q, const void* k,
                   const bsa_csr* out, void* ws, int64_t ws_bytes, hipStream_t stream);

/* Block-sparse attention forward (Metodologia item 2, "Expansion"): every query
 * token of block i attends, with scale 1/sqrt(head_dim), to all tokens of the
 * key blocks listed in CSR row i of its head and to nothing else:
 *   o_n = sum_k softmax_k(q_n . k_k / sqrt(D) + s_k) v_k,  lse_n = log sum_k exp(q_n . k_k / sqrt(D) + s_k),
 * where s_k is the shift of the CSR entry of k's block (0 when mask->shift is
 * NULL).  q, k, v, o: [batch, heads, L, head_dim] in p->layout order (o written
 * in the same order as q); lse: float32 [batch, heads, L] in the same token
 * order, or NULL.  mask->row_ptr / col_idx (/ shift) as produced by
 * bsa_build_mask (capacity and nnz are not read).  Every CSR row must be non-empty with ids in [0, S).
 * ws: device workspace of at least fwd_ws bytes, 256-byte aligned. */
int bsa_forward(const bsa_problem* p, const void* q, const void* k, const void* v,
                const bsa_csr* mask, void* o, float* lse, void* ws, int64_t ws_bytes,
                hipStream_t stream);

/* The two halves of bsa_forward, for callers that time or reuse them separately.
 * bsa_prepare_v (bf16 only; f32 returns BSA_ERR_UNSUPPORTED) writes V in the
 * attention kernel's layout: fractal block order, each 64-token block stored
 * transposed (head_dim rows of 64 keys), keys inside every group of 16 in the
 * order 0-3, 8-11, 4-7, 12-15.  vt: device buffer of batch*heads*L*head_dim
 * bf16 elements (the size of V), 16-byte aligned.
 * bsa_attend runs the attention kernel; `vp` is the output of bsa_prepare_v for
 * bf16, or the V tensor itself (p->layout order) for f32.  ws: at least
 * attend_ws bytes (bsa_query_attend_ws), 256-byte aligned; contents on entry do
 * not matter (it holds the work counters and, for bf16, the work order: each
 * item's cost, its position in the order and the per-XCD bounds; 8 bytes per
 * query-block pair plus 256).  bsa_query_attend_ws is a pure host computation;
 * null output -> BSA_ERR_INVALID_ARG. */
int bsa_prepare_v(const bsa_problem* p, const void* v, void* vt, hipStream_t stream);
int bsa_query_attend_ws(const bsa_problem* p, int64_t* attend_ws);
int bsa_attend(const bsa_problem* p, const void* q, const void* k, const void* vp, const bsa_csr* mask,
               void* o, float* lse, void* ws, int64_t ws_bytes, hipStream_t stream);

/* bsa_attend without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, semantics and kernels as bsa_attend,
 * except that the work counters and work order live in a static scratch array
 * of the library, 4 MiB per GPU (held from the library's first use on a device
 * until the process ends).  The call allocates nothing: problems whose order
 * needs more (bsa_query_attend_ws > 4 MiB, i.e. more than about 524,000 bf16
 * query-block pairs batch*heads*ceil(S/2)) are rejected with BSA_ERR_WORKSPACE
 * before anything is enqueued.  Every call on one GPU shares that GPU's
 * scratch: calls that overlap in time on one GPU (different streams, or
 * threads) race and must be serialised by the caller; each call clears the
 * counters it needs with a fill kernel on `stream`, and the scratch keeps the
 * last call's contents afterwards. */
int bsa_attend_static(const bsa_problem* p, const void* q, const void* k, const void* vp, const bsa_csr* mask,
                      void* o, float* lse, hipStream_t stream);

/* Backward of the block-sparse attention (the gradient of sum(O * dO) with
 * respect to Q, K and V, for training with the mask, NABLA page, Metodologia
 * item 2 "Expansion"): with P = softmax over each query's kept keys of
 * q.k / sqrt(D),
 *   dV_k = sum_n P[n,k] dO_n,   dP[n,k] = dO_n . v_k,
 *   dZ[n,k] = P[n,k] (dP[n,k] - Delta_n),   Delta_n = sum_k P[n,k] dP[n,k],
 *   dQ_n = sum_k dZ[n,k] k_k / sqrt(D),   dK_k = sum_n dZ[n,k] q_n / sqrt(D).
 * The row term Delta_n is computed by the call from P and dP themselves (a
 * first walk over the kept tiles), not from a stored output, so that the dZ of
 * one query sum to zero in the arithmetic the kernels use; the forward's output
 * is therefore not an argument.
 * q, k, v, dout, dq, dk, dv: [batch, heads, L, head_dim] in p->layout order;
 * lse: float32 [batch, heads, L] as returned by bsa_forward for the same mask
 * (required).  mask: the forward's CSR; per-entry shifts are not supported here
 * (BSA_ERR_UNSUPPORTED when mask->shift is not NULL).  Every output element is
 * written (key blocks no query keeps get zero dK, dV); the result is
 * deterministic (no atomics on the gradients: dQ is summed per query block, dK
 * and dV per key block over the transposed mask, which the call builds in its
 * workspace).  ws: at least bwd_ws bytes (bsa_query_backward_ws), 256-byte
 * aligned, contents on entry irrelevant. */
int bsa_query_backward_ws(const bsa_problem* p, int64_t* bwd_ws);
int bsa_backward(const bsa_problem* p, const void* q, const void* k, const void* v, const bsa_csr* mask,
                 const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws, int64_t ws_bytes,
                 hipStream_t stream);

/* The training pair (bf16, head_dim 128 for the backward; NABLA page,
 * Metodologia item 2 "Expansion", the method trained with the mask): a forward
 * that also returns the low part of its output, and a backward that takes the
 * row term from that output instead of recomputing it over the kept tiles.
 * bsa_attend_train: bsa_attend's arguments and work order, plus o_lo (same
 * shape and order as o, 16-byte aligned, required) and lse (required).  The PV
 * product takes P as a pair of bf16 terms (the rounded value and its rounding
 * residual), O = sum P v / sum P is normalised by the float32 sum of P, and
 * o = bf16(O), o_lo = bf16(O - o): o + o_lo holds O to ~2^-16 relative.  The
 * lse equals bsa_attend's; o differs from bsa_attend's in the last bf16 place
 * (bsa_attend divides by the sum of the rounded weights).  float32 problems and
 * masks with shifts -> BSA_ERR_UNSUPPORTED.
 * bsa_backward_train: bsa_backward's arguments, contract and workspace
 * (bsa_query_backward_ws), plus o and o_lo from bsa_attend_train on the same
 * mask (required, 16-byte aligned); Delta_n = dO_n . (o_n + o_lo_n).  Its error
 * against sum P dP / sum P is ~2^-16 of |dO||O|, far below what the dQ sum
 * amplifies into a visible error even when all keys share a large common
 * component; bsa_backward's walk over the kept tiles is skipped.  float32
 * problems -> BSA_ERR_UNSUPPORTED. */
int bsa_attend_train(const bsa_problem* p, const void* q, const void* k, const void* vp, const bsa_csr* mask,
                     void* o, void* o_lo, float* lse, void* ws, int64_t ws_bytes, hipStream_t stream);
int bsa_backward_train(const bsa_problem* p, const void* q, const void* k, const void* v, const bsa_csr* mask,
                       const void* o, const void* o_lo, const float* lse, const void* dout, void* dq, void* dk,
                       void* dv, void* ws, int64_t ws_bytes, hipStream_t stream);

/* ---- 4-token key groups ---------------------------------------------
 * Fine-grained key selection gathered into full tiles (AB-Attention page,
 * news.hamidun.com/es/news/14960, "Los tres recursos de AB-Attention", third
 * resource): keys and values are selected in groups of BSA_KEY_GROUP = 4
 * consecutive fractal-order tokens, and the attention kernel gathers every 16
 * kept groups of a row into one 64-key tile by index (no token is reordered or
 * copied).  Query blocks stay N = 64 tokens, so CSR rows are the same rows
 * r = (b*heads + h)*S + i as above, but col_idx holds GROUP ids g in [0, L/4)
 * (group g = fractal tokens [4g, 4g+4)), ascending.
 * Selection (reading of the page in the NABLA setting): the reduced map taken
 * at group granularity, A[i, g] = softmax_g(Qp_i . Kg_g / sqrt(D)) with Qp the
 * 64-token query-block means and Kg the 4-token key-group means, cut per row
 * exactly as bsa_build_mask cuts the block map (CDF at 1 - thr, same ordering,
 * tie and thr == 0 rules); a window keeps every group of each window block.
 * Limits (else BSA_ERR_UNSUPPORTED): group == BSA_KEY_GROUP;
 * batch*heads*S*(L/4) < 2^31 (int32 CSR offsets: larger problems are split by
 * heads, every (batch, head) being independent); L/4 <= 32768 for the mask
 * (one row of the group map is cut inside one workgroup's LDS); mode
 * BSA_MASK_CDF only. */
#define BSA_KEY_GROUP 4

/* max_nnz: col_idx capacity bsa_build_group_mask needs (rows * L/4); mask_ws:
 * its workspace bytes; fwd_ws: bsa_forward_groups' workspace bytes (a prepared
 * V for bf16 plus work counters). */
int bsa_query_group_sizes(const bsa_problem* p, int group, int64_t* max_nnz, int64_t* mask_ws, int64_t* fwd_ws);

/* Group mask: pooling of Q into blocks and K into groups (float64), the group
 * map in float64 (computed a chunk of heads at a time inside ws), the CDF cut
 * and window union per row, CSR compaction.  q, k in p->layout order; out as for
 * bsa_build_mask with capacity >= max_nnz (out->shift unused).  ws: at least
 * mask_ws bytes, 256-byte aligned, clobbered. */
int bsa_build_group_mask(const bsa_problem* p, int group, const bsa_mask_params* mp, const void* q, const void* k,
                         const bsa_csr* out, void* ws, int64_t ws_bytes, hipStream_t stream);

/* Attention over the kept groups: query token n of block i attends, with scale
 * 1/sqrt(head_dim), to the tokens of the groups in CSR row i and to nothing else
 * (o, lse as in bsa_forward; an empty row gives o = 0 and lse = -inf).  mask:
 * group CSR (ids in [0, L/4), ascending; mask->shift must be NULL).  ws: at least
 * fwd_ws bytes (bsa_query_group_sizes), 256-byte aligned.
 * bsa_prepare_v_groups (bf16 only) writes V as [batch, heads, L/4, head_dim, 4]:
 * each group's 4 tokens stored channel-major (vg: the size of V, 16-byte
 * aligned); bsa_attend_groups then runs the attention on it (f32: pass V itself)
 * with ws of at least attend_ws bytes (bsa_query_attend_groups_ws: the work
 * counters and, for bf16, each row's cost, its position in the work order and the
 * per-XCD bounds, 8 bytes per row plus 256; pure host computation, null output ->
 * BSA_ERR_INVALID_ARG), 256-byte aligned, contents on entry irrelevant. */
int bsa_forward_groups(const bsa_problem* p, int group, const void* q, const void* k, const void* v,
                       const bsa_csr* mask, void* o, float* lse, void* ws, int64_t ws_bytes, hipStream_t stream);
int bsa_prepare_v_groups(const bsa_problem* p, int group, const void* v, void* vg, hipStream_t stream);
int bsa_query_attend_groups_ws(const bsa_problem* p, int group, int64_t* attend_ws);
int bsa_attend_groups(const bsa_problem* p, int group, const void* q, const void* k, const void* vp,
                      const bsa_csr* mask, void* o, float* lse, void* ws, int64_t ws_bytes, hipStream_t stream);

/* Status code -> static string. */
const char* bsa_status_str(int status);
/* Thread-local description of the last non-OK status returned on this thread. */
const char* bsa_last_error(void);
/* ABI version (major*10000 + minor*100 + patch): 200 adds the SIP mask mode and CSR shifts,
 * token-order tables and the backward pass; 300 adds the 4-token key-group path; 400 adds
 * bsa_query_attend_ws and bsa_query_attend_groups_ws (the attention workspaces hold the work
 * order); 500 drops the forward output from bsa_backward (the row term is recomputed); 510
 * adds bsa_attend_static; 520 adds the training pair bsa_attend_train / bsa_backward_train. */
int bsa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
