"""Pins for the SIP part of the oracle (oracle/sip.py) against facts that do not
come from the oracle itself: numpy's own Philox4x64-10 generator, a bisection
solve of the capped proportional design, closed forms, and Monte-Carlo
unbiasedness of the Horvitz-Thompson numerator and normaliser (the property the
AB-Attention page states for SIP, section "Los tres recursos de AB-Attention")."""
import math

import numpy as np
import pytest

from oracle import sip
from oracle.nabla import cdf_keep, reduced_map, pool_blocks


# ------------------------------------------------------------------ Philox4x64-10
@pytest.mark.parametrize("key,state", [
    ((0, 0), (0, 0, 0, 0)),
    ((123, 456), (0, 0, 0, 0)),
    ((2**64 - 1, 7), (41, 9, 3, 1)),
    ((0xDEADBEEF, 0), (2**64 - 1, 3, 0, 0)),       # carry into word 1
])
def test_philox_matches_numpy(key, state):
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(state, dtype=np.uint64))
    ref = g.random_raw(8).reshape(2, 4)
    # numpy advances its 256-bit counter before producing each block of four words
    c = list(state)
    ctrs = []
    for _ in range(2):
        c[0] = (c[0] + 1) % 2**64
        if c[0] == 0:
            c[1] = (c[1] + 1) % 2**64
        ctrs.append(list(c))
    got = sip.philox4x64_10(np.array(ctrs, dtype=np.uint64), key)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("row,seed", [(1, 7), (5, 123456789), (300, 2**63 + 5)])
def test_uniforms_are_numpys_philox_words(row, seed):
    """Reading S4: u[r, j] is word j mod 4 of the Philox4x64-10 block at counter
    (r, floor(j / 4), 0, 0), key (seed, 0) -- checked against numpy's own Philox
    (numpy advances its counter before producing a block, so its state is set
    one below the wanted counter)."""
    S = 37
    u = sip.uniforms(np.array([row]), S, seed)[0]
    for q in range((S + 3) // 4):
        gen = np.random.Philox(key=np.array([seed, 0], dtype=np.uint64),
                               counter=np.array([row - 1, q, 0, 0], dtype=np.uint64))
        words = gen.random_raw(4)
        for w in range(4):
            j = 4 * q + w
            if j < S:
                assert u[j] == float(int(words[w]) >> 11) * 2.0 ** -53


def test_uniforms_range_and_mean():
    u = sip.uniforms(np.arange(300), 400, seed=99)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / u.size)
    assert not np.array_equal(u, sip.uniforms(np.arange(300), 400, seed=100))


# ------------------------------------------------------------------ inclusion probabilities
def _bisect_pi(a, k):
    """Independent solve: the top block at 1, then bisection on c of
    1 + sum_{j != top} min(1, c a_j) = k."""
    top = int(np.argmax(a))
    rest = np.delete(a, top)
    lo, hi = 0.0, 1.0
    while np.minimum(1.0, hi * rest).sum() < k - 1:
        hi *= 2
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.minimum(1.0, mid * rest).sum() < k - 1:
            lo = mid
        else:
            hi = mid
    return np.insert(np.minimum(1.0, hi * rest), top, 1.0)


@pytest.mark.parametrize("seed", range(6))
def test_inclusion_probabilities_solve_the_design(seed):
    rng = np.random.default_rng(seed)
    S = 50
    a = rng.exponential(size=S) ** 3          # heavy-tailed: several capped blocks
    a /= a.sum()
    for k in (1, 2, 3, 10, 25, 49):
        pi = sip.inclusion_probabilities(a, k)
        assert abs(pi.sum() - k) < 1e-12
        assert pi.min() >= 0 and pi.max() <= 1.0
        assert pi[np.argmax(a)] == 1.0
        if k > 1:
            assert np.allclose(pi, _bisect_pi(a, k), rtol=0, atol=1e-12)
        capped = pi == 1.0
        if capped.any() and (~capped).any():
            assert a[capped].min() >= a[~capped].max()
        free = ~capped
        if free.any():
            ratio = pi[free] / a[free]
            assert np.allclose(ratio, ratio[0], rtol=1e-12)


def test_inclusion_probabilities_closed_forms():
    # uniform scores: the top block (lowest index on the tie) plus (k-1)/(S-1) each
    pi = sip.inclusion_probabilities(np.full(16, 1 / 16), 4)
    assert pi[0] == 1.0 and np.allclose(pi[1:], 3 / 15)
    assert np.allclose(sip.inclusion_probabilities(np.array([0.9, 0.05, 0.05]), 2), [1.0, 0.5, 0.5])
    assert np.array_equal(sip.inclusion_probabilities(np.array([0.2, 0.5, 0.3]), 1), [0.0, 1.0, 0.0])
    # budget at or above the number of positive scores: every positive block, with certainty
    assert np.array_equal(sip.inclusion_probabilities(np.array([0.5, 0.5, 0.0]), 2), [1.0, 1.0, 0.0])
    # the page's example weight: inclusion probability 25 % counts four times
    pi = sip.inclusion_probabilities(np.full(9, 1 / 9), 3)
    assert np.allclose(1 / pi[1:], 4.0)


# ------------------------------------------------------------------ Horvitz-Thompson unbiasedness
def _small_head(seed=0, S=12, N=4, D=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S * N, D))
    k = rng.standard_normal((S * N, D)) + 0.7 * np.sin(np.arange(S * N))[:, None]
    v = rng.standard_normal((S * N, D))
    return q, k, v


def test_ht_estimates_are_unbiased_and_plain_sums_are_not():
    S, N, D = 12, 4, 8
    q, k, v = _small_head(S=S, N=N, D=D)
    A = reduced_map(pool_blocks(q, N), pool_blocks(k, N))
    keep_cdf, _ = cdf_keep(A, 0.3)
    budget = keep_cdf.sum(1)
    z = q @ k.T / math.sqrt(D)
    e = np.exp(z - z.max())
    i = 5                                          # one query block; its N queries
    rows_q = slice(i * N, (i + 1) * N)
    blk_num = np.stack([(e[rows_q, j * N:(j + 1) * N] @ v[j * N:(j + 1) * N]) for j in range(S)])  # [S, N, D]
    blk_den = np.stack([e[rows_q, j * N:(j + 1) * N].sum(1) for j in range(S)])                     # [S, N]
    true_num, true_den = blk_num.sum(0), blk_den.sum(0)
    pi = sip.inclusion_probabilities(A[i], int(budget[i]))
    assert 0 < pi.min() and pi.max() <= 1 and (pi < 1).any()
    M = 3000
    taken, w = [], []
    for s in range(M):                              # the whole mask builder, one seed per draw
        keep, shift = sip.build_sip_mask(A, budget, sip.uniforms(np.arange(S), S, seed=s), 0.3)
        taken.append(keep[i])
        w.append(np.where(keep[i], np.exp(shift[i]), 0.0))   # exp(log(1/pi)): Horvitz-Thompson weight
    taken, w = np.array(taken), np.array(w)
    assert np.allclose(w[taken], np.broadcast_to(1 / pi, taken.shape)[taken], rtol=1e-12)
    ht_num = np.einsum("ms,snd->mnd", w, blk_num)
    ht_den = w @ blk_den
    plain_num = np.einsum("ms,snd->mnd", taken.astype(float), blk_num)
    for est, true in ((ht_num, true_num), (ht_den, true_den)):
        se = est.std(0) / math.sqrt(M)
        assert np.all(np.abs(est.mean(0) - true) <= 5 * se + 1e-12)
    se = plain_num.std(0) / math.sqrt(M)
    assert np.any(np.abs(plain_num.mean(0) - true_num) > 5 * se)     # the check has power
    # expected sample size equals the budget
    cnt = taken.sum(1)
    assert abs(cnt.mean() - budget[i]) <= 5 * cnt.std() / math.sqrt(M)


def test_logit_shift_equals_ht_ratio():
    """Attention with log(1/pi) added to a sampled tile's logits is the ratio of the HT
    numerator to the HT normaliser for that sample (reading S6)."""
    S, N, D = 12, 4, 8
    q, k, v = _small_head(seed=3, S=S, N=N, D=D)
    A = reduced_map(pool_blocks(q, N), pool_blocks(k, N))
    keep_cdf, _ = cdf_keep(A, 0.2)
    u = sip.uniforms(np.arange(S), S, seed=17)
    keep, shift = sip.build_sip_mask(A, keep_cdf.sum(1), u, 0.2)
    row_ptr = np.concatenate([[0], np.cumsum(keep.sum(1))])
    cols = np.concatenate([np.nonzero(keep[r])[0] for r in range(S)])
    sh = np.concatenate([shift[r, keep[r]] for r in range(S)])
    O, LSE = sip.shifted_block_sparse_attention(q[None, None], k[None, None], v[None, None], row_ptr, cols, sh, N)
    z = q @ k.T / math.sqrt(D)
    for r in range(S):
        w = np.zeros(S)
        w[keep[r]] = np.exp(shift[r, keep[r]])      # = 1/pi
        wt = np.repeat(w, N)
        rq = slice(r * N, (r + 1) * N)
        num = (np.exp(z[rq]) * wt) @ v
        den = (np.exp(z[rq]) * wt).sum(1)
        assert np.allclose(O[0, 0, rq], num / den[:, None], rtol=1e-12, atol=1e-12)
        assert np.allclose(LSE[0, 0, rq], np.log(den), rtol=1e-12, atol=1e-12)


def test_sip_window_and_thr_zero():
    S = 16
    rng = np.random.default_rng(4)
    A = rng.dirichlet(np.ones(S), size=S)
    u = sip.uniforms(np.arange(S), S, seed=5)
    win = np.eye(S, dtype=bool) | np.eye(S, k=1, dtype=bool)
    keep, shift = sip.build_sip_mask(A, np.full(S, 4), u, 0.1, window_mask=win)
    assert np.all(keep[win]) and np.all(shift[win] == 0)
    assert np.all(shift[~keep] == 0) and np.all(shift >= 0)
    keep0, shift0 = sip.build_sip_mask(A, np.full(S, 4), u, 0.0)
    assert keep0.all() and not shift0.any()
