"""Fine-grained key selection: small key/value groups gathered into full tiles, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "AB-Attention acelera la generacion de video hasta 2,23x y omite el 92%
de la atencion" (news.hamidun.com/es/news/14960), section "Los tres recursos de
AB-Attention", third resource: the key/value blocks are only 4 tokens long, and
the kernel gathers the chosen blocks by index into full matrix-core tiles
without reordering or copying tokens; going from 128-token to 4-token blocks
raises the attention mass the ideal selection keeps at the same tile budget.

Readings taken where the page is silent (also listed with the design notes):
  G1  a key group is G consecutive tokens of the fractal order (G = 4 on the
      page; G divides the query block size N).  Group g of a head covers tokens
      gG .. gG+G-1; query blocks stay N tokens.
  G2  the score of group g for query block i is the NABLA reduced map taken at
      group granularity: A[i, g] = softmax_g(Qp_i . Kg_g / sqrt(D)) over all L/G
      groups of the head, with Qp the N-token query-block means and Kg the
      G-token key-group means.  (AB-Attention scores its 4-token blocks with its
      own clustering selector, which is out of scope; the reduced map is the
      score this path already has.)
  G3  the selection is the NABLA CDF cut (cdf_keep: order by probability
      descending then index ascending, keep the shortest prefix reaching
      1 - thr, thr = 0 keeps all) on that map; with the sliding-tile window, every
      group of a window block is kept as well (union after the cut).
  G4  query block i attends to the tokens of its kept groups (all or nothing per
      group); a kernel may gather them 16 groups (64 keys) per tile in ascending
      group order, the last tile of a row padded with keys that take no part.
  With G = N the groups are the blocks and everything reduces to the NABLA path
  exactly (pinned).
"""
import math

import numpy as np

from .nabla import cdf_keep, csr_from_keep, fractal_positions, pool_blocks, reduced_map, sta_window


def group_window(T: int, Hp: int, Wp: int, win, per_block: int) -> np.ndarray:
    """Sliding-tile window at group granularity (reading G3): query block i keeps
    group g iff g's block g // per_block is in i's window.  Returns bool [S, S*per_block]."""
    return np.repeat(sta_window(T, Hp, Wp, win), per_block, axis=1)


def head_group_mask(qf: np.ndarray, kf: np.ndarray, N: int, G: int, thr: float, window_mask=None):
    """Group mask of one (batch, head): qf, kf [L, D] in fractal order (readings G1-G3).
    Returns dict(keep [S, L/G], cexcl [S, L/G], A [S, L/G], cdf_keep [S, L/G])."""
    if N % G:
        raise ValueError("the group size must divide the block size")
    Qp = pool_blocks(qf, N)
    Kg = pool_blocks(kf, G)
    A = reduced_map(Qp, Kg)
    keep_cdf, cexcl = cdf_keep(A, thr)
    keep = keep_cdf | window_mask if window_mask is not None else keep_cdf
    return {"keep": keep, "cexcl": cexcl, "A": A, "cdf_keep": keep_cdf}


def build_group_mask(q: np.ndarray, k: np.ndarray, T: int, H: int, W: int, P: int, N: int, G: int,
                     thr: float, window=None, layout: str = "original", details: bool = False):
    """Whole group-mask stage.  q, k: [B, nh, L, D] (original token order unless
    layout == "fractal").  Returns dict with the CSR (row_ptr, col_idx = group ids,
    ascending) over rows r = (b*nh + h)*S + i, and with details=True also
    keep/cexcl/A/cdf_keep [B, nh, S, L/G]."""
    B, nh, L, D = q.shape
    S, SG = L // N, L // G
    wmask = None
    if window is not None:
        if N != P * P:
            raise ValueError("the sliding-tile window needs N == P*P")
        wmask = group_window(T, H // P, W // P, window, N // G)
    keep = np.zeros((B, nh, S, SG), dtype=bool)
    extra = {}
    if details:
        extra = {"cexcl": np.zeros((B, nh, S, SG)), "A": np.zeros((B, nh, S, SG)),
                 "cdf_keep": np.zeros((B, nh, S, SG), dtype=bool)}
    src = fractal_positions(T, H, W, P) if layout == "original" else None
    for b in range(B):
        for h in range(nh):
            qf = q[b, h] if src is None else q[b, h][src]
            kf = k[b, h] if src is None else k[b, h][src]
            m = head_group_mask(qf, kf, N, G, thr, wmask)
            keep[b, h] = m["keep"]
            for key in extra:
                extra[key][b, h] = m[key]
    row_ptr, col_idx = csr_from_keep(keep.reshape(B * nh * S, SG))
    out = {"row_ptr": row_ptr, "col_idx": col_idx, "keep": keep}
    out.update(extra)
    return out


def expand_block_csr(row_ptr, col_idx, per_block: int):
    """A block CSR as a group CSR: kept block j becomes groups j*per_block ..
    (j+1)*per_block - 1 (row_ptr scaled, col_idx expanded, still ascending)."""
    row_ptr = np.asarray(row_ptr, np.int64)
    cols = np.asarray(col_idx, np.int64)
    groups = (cols[:, None] * per_block + np.arange(per_block)[None, :]).reshape(-1)
    return row_ptr * per_block, groups.astype(np.int32)


def group_attention(qf, kf, vf, row_ptr, col_idx, N: int, G: int, rows=None):
    """Attention of each query block over the tokens of its kept groups (reading G4),
    float64.  qf, kf, vf: [B, nh, L, D] fractal order; CSR rows r = (b*nh + h)*S + i
    with group ids in col_idx.  Query token n of block i:
        O_n = sum_k softmax_k(q_n . k_k / sqrt(D)) v_k over k in the kept groups' tokens,
        LSE_n = log sum_k exp(q_n . k_k / sqrt(D)).
    `rows` restricts the computation to a subset of rows (others stay NaN); an
    empty row gives O = 0 and LSE = -inf.  Returns (O [B, nh, L, Dv], LSE [B, nh, L])."""
    B, nh, L, D = qf.shape
    S = L // N
    O = np.full((B, nh, L, vf.shape[-1]), np.nan)
    LSE = np.full((B, nh, L), np.nan)
    scale = 1.0 / math.sqrt(D)
    rows = range(B * nh * S) if rows is None else rows
    for r in rows:
        bh, i = divmod(int(r), S)
        b, h = divmod(bh, nh)
        groups = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)
        if groups.size == 0:                       # an empty row attends to nothing
            O[b, h, i * N:(i + 1) * N] = 0.0
            LSE[b, h, i * N:(i + 1) * N] = -np.inf
            continue
        keys = (groups[:, None] * G + np.arange(G)[None, :]).reshape(-1)
        q = np.asarray(qf[b, h, i * N:(i + 1) * N], np.float64)
        kk = np.asarray(kf[b, h, keys], np.float64)
        vv = np.asarray(vf[b, h, keys], np.float64)
        z = (q @ kk.T) * scale
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        s = e.sum(axis=1, keepdims=True)
        O[b, h, i * N:(i + 1) * N] = (e @ vv) / s
        LSE[b, h, i * N:(i + 1) * N] = (m + np.log(s))[:, 0]
    return O, LSE
