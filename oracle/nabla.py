"""Plain float64 CPU oracle of the NABLA block-sparse attention pipeline.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Resumen Tecnico: NABLA - Atencion de Bloque Adaptativa al Vecindario
para la Generacion Eficiente de Video", gist.science/es/paper/2507.13546,
section "Metodologia: NABLA":
  item 1  "Reordenamiento de Tokens (Aplanamiento Fractal)"      -> fractal_positions, permute
  item 2  "Construccion de Mascara Adaptativa":
            bullet "Submuestreo"        (block average pooling)  -> pool_blocks
            bullet "Atencion Reducida"  (map over pooled blocks) -> reduced_map
            bullet "Umbralizacion CDF"  (per-row CDF cut)        -> cdf_keep
            bullet "Expansion"          (tile-level mask)        -> block_sparse_attention
  item 3  "Integracion Hibrida con STA" (M = M_nabla OR M_STA)  -> sta_window, head_mask

Readings taken where the page is silent (each is also listed with the design notes):
  R1  fractal order is one level: frames outermost, P x P patches row-major
      inside a frame, tokens row-major inside a patch.
  R2  a block is N consecutive tokens of the fractal order (N = P*P in every
      workload, so a block is exactly one patch of one frame).
  R3  the reduced map is softmax over all key blocks of Qp.Kp / sqrt(D),
      D = head dim, non-causal.
  R4  the CDF cut keeps the smallest prefix of the row sorted by probability
      descending whose mass reaches (>=) 1 - thr; ties are ordered by block
      index ascending; thr = 0 keeps every block; at least one block is kept.
  R5  the sliding-tile window is +-w tiles in (t, patch-row, patch-col),
      clipped at the borders, and is unioned after the CDF cut.
  R6  expansion is all-or-nothing per N x N tile: a query token of block i
      attends to every token of every kept key block and to nothing else.
  R7  attention scale is 1/sqrt(D).
"""
import math

import numpy as np


# --------------------------------------------------------------------------
# item 1: fractal flattening
# --------------------------------------------------------------------------
def fractal_positions(T: int, H: int, W: int, P: int) -> np.ndarray:
    """src[f] = original (t, h, w) row-major index of the token placed at fractal
    position f.  NABLA page, Metodologia item 1: the tokens of every P x P spatial
    patch become one contiguous run and time stays ordered (reading R1)."""
    if H % P or W % P:
        raise ValueError("H and W must be multiples of P")
    t, py, px, y, x = np.meshgrid(np.arange(T), np.arange(H // P), np.arange(W // P),
                                  np.arange(P), np.arange(P), indexing="ij")
    src = (t * H + py * P + y) * W + (px * P + x)
    return src.reshape(-1).astype(np.int64)


def permute(x: np.ndarray, T: int, H: int, W: int, P: int) -> np.ndarray:
    """Original order -> fractal order along axis -2 ([..., L, D])."""
    return np.ascontiguousarray(x[..., fractal_positions(T, H, W, P), :])


def inverse_permute(y: np.ndarray, T: int, H: int, W: int, P: int) -> np.ndarray:
    """Fractal order -> original order along axis -2."""
    out = np.empty_like(y)
    out[..., fractal_positions(T, H, W, P), :] = y
    return out


def tile_coords(i, T: int, Hp: int, Wp: int):
    """Block id (fractal order, N = P*P) -> (t, patch row, patch col)."""
    i = np.asarray(i)
    return i // (Hp * Wp), (i // Wp) % Hp, i % Wp


# --------------------------------------------------------------------------
# item 2: adaptive mask
# --------------------------------------------------------------------------
def pool_blocks(xf: np.ndarray, N: int) -> np.ndarray:
    """Average of every N consecutive fractal-order tokens ("Submuestreo", reading R2).
    xf: [..., L, D]; returns [..., L/N, D] float64."""
    L, D = xf.shape[-2], xf.shape[-1]
    if L % N:
        raise ValueError("L must be a multiple of N")
    x = np.asarray(xf, dtype=np.float64).reshape(xf.shape[:-2] + (L // N, N, D))
    return x.mean(axis=-2)


def reduced_map(Qp: np.ndarray, Kp: np.ndarray) -> np.ndarray:
    """Full attention map over the pooled blocks ("Atencion Reducida", reading R3):
    A[i, j] = softmax_j(Qp_i . Kp_j / sqrt(D)).  Qp, Kp: [S, D]; returns [S, S]."""
    D = Qp.shape[-1]
    Z = (np.asarray(Qp, np.float64) @ np.asarray(Kp, np.float64).T) / math.sqrt(D)
    Z = Z - Z.max(axis=-1, keepdims=True)
    E = np.exp(Z)
    return E / E.sum(axis=-1, keepdims=True)


def cdf_keep(A: np.ndarray, thr: float):
    """Per-row CDF threshold ("Umbralizacion CDF", reading R4).

    A: [S_rows, S] probabilities.  Each row is ordered by (probability descending,
    block index ascending); c_k is the exclusive prefix sum of that ordering; the
    block at position k is kept iff thr == 0, or k == 0, or c_k < 1 - thr.  That is
    the shortest prefix whose inclusive mass reaches 1 - thr.

    Returns (keep bool [rows, S], cexcl float64 [rows, S]) where cexcl[r, j] is the
    exclusive prefix mass in front of block j in row r's ordering."""
    A = np.asarray(A, dtype=np.float64)
    R, S = A.shape
    order = np.argsort(-A, axis=1, kind="stable")          # stable: equal p -> index ascending
    ps = np.take_along_axis(A, order, axis=1)
    c = np.zeros_like(ps)                                   # exclusive prefix, left to right
    c[:, 1:] = np.cumsum(ps, axis=1)[:, :-1]
    pos = np.arange(S)[None, :]
    keep_pos = (thr == 0) | (pos == 0) | (c < 1.0 - thr)
    keep = np.zeros((R, S), dtype=bool)
    cexcl = np.zeros((R, S), dtype=np.float64)
    np.put_along_axis(keep, order, keep_pos, axis=1)
    np.put_along_axis(cexcl, order, c, axis=1)
    return keep, cexcl


# --------------------------------------------------------------------------
# item 3: hybrid with sliding-tile attention
# --------------------------------------------------------------------------
def sta_window(T: int, Hp: int, Wp: int, win) -> np.ndarray:
    """Static sliding-tile window over tiles (reading R5): query tile (t, y, x) sees
    key tile (t', y', x') iff |t-t'| <= wt, |y-y'| <= wh and |x-x'| <= ww.
    Returns bool [S, S], S = T*Hp*Wp."""
    wt, wh, ww = win
    S = T * Hp * Wp
    t, y, x = tile_coords(np.arange(S), T, Hp, Wp)
    return ((np.abs(t[:, None] - t[None, :]) <= wt)
            & (np.abs(y[:, None] - y[None, :]) <= wh)
            & (np.abs(x[:, None] - x[None, :]) <= ww))


def csr_from_keep(keep: np.ndarray):
    """Block mask [rows, S] -> CSR (row_ptr int64 [rows+1], col_idx int32, columns ascending)."""
    keep = np.asarray(keep, dtype=bool)
    counts = keep.sum(axis=1)
    row_ptr = np.zeros(keep.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.nonzero(keep)[1].astype(np.int32)          # row-major scan: ascending per row
    return row_ptr, col_idx


def head_mask(qf: np.ndarray, kf: np.ndarray, N: int, thr: float, window_mask=None):
    """Mask of one (batch, head): qf, kf [L, D] in fractal order.
    Returns dict(keep [S,S] bool, cexcl [S,S], A [S,S], cdf_keep [S,S])."""
    Qp = pool_blocks(qf, N)
    Kp = pool_blocks(kf, N)
    A = reduced_map(Qp, Kp)
    keep_cdf, cexcl = cdf_keep(A, thr)
    keep = keep_cdf | window_mask if window_mask is not None else keep_cdf
    return {"keep": keep, "cexcl": cexcl, "A": A, "cdf_keep": keep_cdf}


def build_mask(q: np.ndarray, k: np.ndarray, T: int, H: int, W: int, P: int, N: int,
               thr: float, window=None, layout: str = "original", details: bool = False):
    """Whole mask stage.  q, k: [B, nh, L, D] (original token order unless
    layout == "fractal").  Returns dict with CSR (row_ptr, col_idx) over rows
    r = (b*nh + h)*S + i, and with details=True also keep/cexcl/A [B, nh, S, S]."""
    B, nh, L, D = q.shape
    S = L // N
    wmask = None
    if window is not None:
        if N != P * P:
            raise ValueError("the sliding-tile window needs N == P*P")
        wmask = sta_window(T, H // P, W // P, window)
    keep = np.zeros((B, nh, S, S), dtype=bool)
    extra = {}
    if details:
        extra = {"cexcl": np.zeros((B, nh, S, S)), "A": np.zeros((B, nh, S, S)),
                 "cdf_keep": np.zeros((B, nh, S, S), dtype=bool)}
    src = fractal_positions(T, H, W, P) if layout == "original" else None
    for b in range(B):
        for h in range(nh):
            qf = q[b, h] if src is None else q[b, h][src]
            kf = k[b, h] if src is None else k[b, h][src]
            m = head_mask(qf, kf, N, thr, wmask)
            keep[b, h] = m["keep"]
            if details:
                for key in extra:
                    extra[key][b, h] = m[key]
    row_ptr, col_idx = csr_from_keep(keep.reshape(B * nh * S, S))
    out = {"row_ptr": row_ptr, "col_idx": col_idx, "keep": keep}
    out.update(extra)
    return out


# --------------------------------------------------------------------------
# block-sparse attention over the kept tiles ("Expansion", reading R6)
# --------------------------------------------------------------------------
def block_sparse_attention(qf, kf, vf, row_ptr, col_idx, N: int, rows=None):
    """Attention restricted to kept N x N tiles, float64.

    qf, kf, vf: [B, nh, L, D] in fractal order; CSR rows r = (b*nh + h)*S + i.
    Query token n of block i attends to the union of the kept key blocks' tokens:
        O_n = sum_k softmax_k(q_n . k_k / sqrt(D)) v_k,   LSE_n = log sum_k exp(q_n . k_k / sqrt(D)).
    `rows` restricts the computation to a subset of CSR rows (others stay NaN).
    Returns (O [B, nh, L, D] float64, LSE [B, nh, L] float64)."""
    B, nh, L, D = qf.shape
    S = L // N
    O = np.full((B, nh, L, vf.shape[-1]), np.nan)
    LSE = np.full((B, nh, L), np.nan)
    scale = 1.0 / math.sqrt(D)
    rows = range(B * nh * S) if rows is None else rows
    for r in rows:
        bh, i = divmod(int(r), S)
        b, h = divmod(bh, nh)
        cols = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)
        keys = (cols[:, None] * N + np.arange(N)[None, :]).reshape(-1)
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


def dense_attention(q, k, v):
    """Textbook softmax attention, float64: softmax(q k^T / sqrt(D)) v over all keys.
    q, k, v: [..., L, D].  Returns (O, LSE)."""
    D = q.shape[-1]
    z = (np.asarray(q, np.float64) @ np.swapaxes(np.asarray(k, np.float64), -1, -2)) / math.sqrt(D)
    m = z.max(axis=-1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=-1, keepdims=True)
    return (e @ np.asarray(v, np.float64)) / s, (m + np.log(s))[..., 0]


def attention_pipeline(q, k, v, T, H, W, P, N, thr, window=None):
    """All five steps on original-order inputs: permute, mask, block-sparse
    attention, inverse permute.  Returns (O original order, LSE original order, mask)."""
    src = fractal_positions(T, H, W, P)
    qf, kf, vf = q[..., src, :], k[..., src, :], v[..., src, :]
    mask = build_mask(qf, kf, T, H, W, P, N, thr, window, layout="fractal")
    Of, LSEf = block_sparse_attention(qf, kf, vf, mask["row_ptr"], mask["col_idx"], N)
    O = np.empty_like(Of)
    O[..., src, :] = Of
    LSE = np.empty_like(LSEf)
    LSE[..., src] = LSEf
    return O, LSE, mask


# --------------------------------------------------------------------------
# backward of the block-sparse attention (the training use of the mask)
# --------------------------------------------------------------------------
def block_sparse_attention_backward(qf, kf, vf, row_ptr, col_idx, dO, N: int, rows=None, O=None):
    """Gradients of sum(O * dO) for the attention above, float64, written out from
    the chain rule of softmax attention (the NABLA page's method is trained with
    this mask, Metodologia item 2 "Expansion"; the gradient of the kept-tile
    attention is the dense one restricted to the kept tiles):
        P = softmax(Z),  Z = q k^T / sqrt(D)           (over the kept keys only)
        dV_k += sum_n P[n,k] dO_n
        dP[n,k] = dO_n . v_k
        dZ[n,k] = P[n,k] (dP[n,k] - sum_k' P[n,k'] dP[n,k'])
        dQ_n = sum_k dZ[n,k] k_k / sqrt(D),   dK_k += sum_n dZ[n,k] q_n / sqrt(D).
    qf, kf, vf, dO: [B, nh, L, D] in fractal order; CSR as in block_sparse_attention.
    sum_k' P[n,k'] dP[n,k'] equals dO_n . o_n for the exact output o; when the
    forward's output O (fractal order) is given, the row term is taken as
    dO_n . O_n from it -- the form a kernel that stores O and not P uses -- so a
    rounded O enters the gradient exactly as it does there.
    Returns (dQ, dK, dV) [B, nh, L, D] float64; `rows` restricts the query blocks
    whose contributions are summed (the full gradient needs every row)."""
    B, nh, L, D = qf.shape
    S = L // N
    dQ = np.zeros((B, nh, L, D))
    dK = np.zeros((B, nh, L, D))
    dV = np.zeros((B, nh, L, vf.shape[-1]))
    scale = 1.0 / math.sqrt(D)
    rows = range(B * nh * S) if rows is None else rows
    for r in rows:
        bh, i = divmod(int(r), S)
        b, h = divmod(bh, nh)
        cols = np.asarray(col_idx[row_ptr[r]:row_ptr[r + 1]], dtype=np.int64)
        keys = (cols[:, None] * N + np.arange(N)[None, :]).reshape(-1)
        qs = slice(i * N, (i + 1) * N)
        q = np.asarray(qf[b, h, qs], np.float64)
        kk = np.asarray(kf[b, h, keys], np.float64)
        vv = np.asarray(vf[b, h, keys], np.float64)
        do = np.asarray(dO[b, h, qs], np.float64)
        z = (q @ kk.T) * scale
        e = np.exp(z - z.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dp = do @ vv.T
        if O is None:
            delta = (p * dp).sum(axis=1, keepdims=True)
        else:
            delta = (do * np.asarray(O[b, h, qs], np.float64)).sum(axis=1, keepdims=True)
        dz = p * (dp - delta)
        dQ[b, h, qs] = dz @ kk * scale
        np.add.at(dK[b, h], keys, dz.T @ q * scale)
        np.add.at(dV[b, h], keys, p.T @ do)
    return dQ, dK, dV
