"""Sampled block selection with inclusion-probability weights (SIP), float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "AB-Attention acelera la generacion de video hasta 2,23x y omite el 92%
de la atencion" (news.hamidun.com/es/news/14960), section "Los tres recursos de
AB-Attention", second resource (SIP): a key block enters the sample with a
probability proportional to its score, the most important blocks are always
taken and every other one has a nonzero chance; a sampled block is weighted by
the inverse of its inclusion probability (the Horvitz-Thompson estimator), which
makes both the attention numerator and the softmax normaliser unbiased, and the
weighting is applied as a shift of that block's logits inside an otherwise
ordinary softmax attention.

Readings taken where the page is silent (also listed with the design notes):
  S1  the score of key block j for query block i is the reduced-map probability
      A[i, j] of the NABLA pipeline (the same map the CDF cut uses).
  S2  "proportional to its score, the most important always taken" is the
      capped proportional design: the row's top block (largest A, lowest index
      on ties) is always taken (pi = 1), which also keeps every row non-empty;
      every other block gets pi_j = min(1, c * A[i, j]) with c chosen so that
      the probabilities of all blocks sum to the row's budget k (so blocks with
      c * A >= 1 are always taken too).
  S3  the budget k of a row is the number of blocks the CDF cut keeps for that
      row (SIP spends the same number of tiles as the cut it replaces, in
      expectation); thr = 0 keeps every block with pi = 1.
  S4  the draw is one independent Bernoulli trial per (row, block) -- Poisson
      sampling, for which the Horvitz-Thompson weights 1 / pi are exactly the
      unbiasing ones -- with the uniform variate of Philox4x64-10 (Salmon et al.,
      "Parallel random numbers: as easy as 1, 2, 3", SC 2011): the block at
      counter (row, floor(block / 4), 0, 0) and key (seed, 0) gives four words,
      one per block of four consecutive blocks, u = (word_(block mod 4) >> 11)
      * 2^-53, and the block is taken iff u < pi.
  S5  blocks of the sliding-tile window are always present and carry no weight
      (pi = 1); the window is unioned after the sampling.
  S6  the weight enters attention as the additive logit shift log(1 / pi) on
      every logit of the sampled tile.
"""
import math

import numpy as np

_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157      # Philox4x64 multipliers
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B      # Weyl key increments
_MASK = (1 << 64) - 1


def _mul_hilo(a: np.ndarray, m: int):
    """64x64 -> 128-bit product of uint64 array a and constant m, as (hi, lo) uint64."""
    a = a.astype(np.uint64)
    a_lo, a_hi = a & np.uint64(0xFFFFFFFF), a >> np.uint64(32)
    m_lo, m_hi = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    ll = a_lo * m_lo
    lh = a_lo * m_hi
    hl = a_hi * m_lo
    hh = a_hi * m_hi
    mid = (ll >> np.uint64(32)) + (lh & np.uint64(0xFFFFFFFF)) + (hl & np.uint64(0xFFFFFFFF))
    lo = (ll & np.uint64(0xFFFFFFFF)) | (mid << np.uint64(32))
    hi = hh + (lh >> np.uint64(32)) + (hl >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10(ctr: np.ndarray, key) -> np.ndarray:
    """Philox4x64 with 10 rounds (Salmon et al. 2011).  ctr: uint64 [..., 4];
    key: two uint64 words.  Each round multiplies words 0 and 2 by the two
    constants and mixes the high halves with words 1, 3 and the key; the key is
    bumped by the Weyl constants between rounds.  Returns uint64 [..., 4]."""
    c = [np.asarray(ctr, np.uint64)[..., x].copy() for x in range(4)]
    k0, k1 = int(key[0]) & _MASK, int(key[1]) & _MASK
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = _mul_hilo(c[0], _M0)
            hi1, lo1 = _mul_hilo(c[2], _M1)
            c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
            k0, k1 = (k0 + _W0) & _MASK, (k1 + _W1) & _MASK
    return np.stack(c, axis=-1)


def uniforms(rows: np.ndarray, S: int, seed: int) -> np.ndarray:
    """u[r, j] in [0, 1) for the given CSR rows and every block j (reading S4):
    word j mod 4 of the generator block at counter (r, floor(j / 4))."""
    rows = np.asarray(rows, np.uint64)
    nq = (S + 3) // 4
    ctr = np.zeros((len(rows), nq, 4), np.uint64)
    ctr[..., 0] = rows[:, None]
    ctr[..., 1] = np.arange(nq, dtype=np.uint64)[None, :]
    words = philox4x64_10(ctr, (seed, 0)).reshape(len(rows), 4 * nq)[:, :S]
    return (words >> np.uint64(11)).astype(np.float64) * 2.0 ** -53


def inclusion_probabilities(a: np.ndarray, k: int) -> np.ndarray:
    """Inclusion probabilities of one row with budget k >= 1 (reading S2): the top
    block gets 1; the others get min(1, c * a_j) summing to k - 1.  a: one row of
    nonnegative scores.  Written out from the definition: with the other scores
    sorted in descending order, the first t are capped at 1 and the rest share
    k - 1 - t in proportion to their score, for the smallest t at which no
    uncapped block would exceed 1."""
    a = np.asarray(a, np.float64)
    top = int(np.argmax(a))                      # first maximum: lowest index on ties
    pi = np.zeros(len(a))
    pi[top] = 1.0
    others = np.delete(np.arange(len(a)), top)
    b = a[others]
    kk = k - 1
    if kk <= 0:
        return pi
    positive = int(np.count_nonzero(b > 0))
    if kk >= positive:
        pi[others] = (b > 0).astype(np.float64)
        return pi
    s = np.sort(b)[::-1]
    for t in range(kk):
        c = (kk - t) / s[t:].sum()
        if c * s[t] < 1.0:
            break
    # Falling through means the mass after the first kk - 1 others is below the
    # rounding unit of their sum: then c * s[kk - 1] rounds to 1, the first kk
    # others are all taken and the rest keep their vanishing probabilities.
    pi[others] = np.minimum(1.0, c * b)
    return pi


def sip_row(a: np.ndarray, k: int, u: np.ndarray, thr: float):
    """Sample one row: (taken mask, pi).  thr == 0 takes every block (reading S3)."""
    if thr == 0.0:
        return np.ones(len(a), bool), np.ones(len(a))
    pi = inclusion_probabilities(a, k)
    return u < pi, pi


def build_sip_mask(A: np.ndarray, cdf_counts: np.ndarray, u: np.ndarray, thr: float, window_mask=None):
    """SIP mask of one head.  A: [S, S] reduced map; cdf_counts: [S] budget per row
    (the CDF cut's kept count, reading S3); u: [S, S] uniforms; window_mask: [S, S]
    or None.  Returns (keep [S, S] bool, shift [S, S] float64 = log(1/pi) on sampled
    non-window blocks, 0 elsewhere)."""
    S = A.shape[0]
    keep = np.zeros((S, S), bool)
    shift = np.zeros((S, S))
    for i in range(S):
        taken, pi = sip_row(A[i], int(cdf_counts[i]), u[i], thr)
        keep[i] = taken
        shift[i, taken] = -np.log(pi[taken])
    if window_mask is not None:
        keep |= window_mask
        shift[window_mask] = 0.0
    return keep, shift


def shifted_block_sparse_attention(qf, kf, vf, row_ptr, col_idx, shift, N: int, rows=None):
    """Block-sparse attention whose tile (i, j) logits get + shift[entry] (reading S6),
    float64.  Same conventions as nabla.block_sparse_attention; `shift` is aligned
    with col_idx.  Returns (O, LSE)."""
    B, nh, L, D = qf.shape
    S = L // N
    O = np.full((B, nh, L, vf.shape[-1]), np.nan)
    LSE = np.full((B, nh, L), np.nan)
    scale = 1.0 / math.sqrt(D)
    rows = range(B * nh * S) if rows is None else rows
    for r in rows:
        bh, i = divmod(int(r), S)
        b, h = divmod(bh, nh)
        lo, hi = int(row_ptr[r]), int(row_ptr[r + 1])
        cols = np.asarray(col_idx[lo:hi], dtype=np.int64)
        keys = (cols[:, None] * N + np.arange(N)[None, :]).reshape(-1)
        sh = np.repeat(np.asarray(shift[lo:hi], np.float64), N)
        q = np.asarray(qf[b, h, i * N:(i + 1) * N], np.float64)
        kk = np.asarray(kf[b, h, keys], np.float64)
        vv = np.asarray(vf[b, h, keys], np.float64)
        z = (q @ kk.T) * scale + sh[None, :]
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        s = e.sum(axis=1, keepdims=True)
        O[b, h, i * N:(i + 1) * N] = (e @ vv) / s
        LSE[b, h, i * N:(i + 1) * N] = (m + np.log(s))[:, 0]
    return O, LSE
