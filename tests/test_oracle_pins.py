"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-derived cases (tests/golden, each cited), closed forms, invariants, brute
force on tiny inputs and independent library routines (scipy, torch SDPA).

Each group is chosen so that a plausible slip in the oracle (a transposed axis,
a dropped scale, a strict-vs-non-strict comparison, a wrong tie-break, an
off-by-one prefix) fails at least one test.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
from workloads import get_config, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


# ---------------------------------------------------------------- a1: fractal order
@pytest.mark.parametrize("row", list(_rows("fractal_hand_cases.txt")))
def test_fractal_hand_cases(row):
    T, H, W, P, n, f = map(int, row)
    src = oracle.fractal_positions(T, H, W, P)
    assert src[f] == n


@pytest.mark.parametrize("T,H,W,P", [(4, 16, 16, 8), (3, 24, 40, 8), (2, 12, 8, 4), (5, 8, 8, 8), (1, 6, 9, 3)])
def test_fractal_is_bijection_and_inverse(T, H, W, P):
    L = T * H * W
    src = oracle.fractal_positions(T, H, W, P)
    assert np.array_equal(np.sort(src), np.arange(L))
    x = np.random.default_rng(0).standard_normal((2, L, 3))
    y = oracle.permute(x, T, H, W, P)
    assert np.array_equal(oracle.inverse_permute(y, T, H, W, P), x)


@pytest.mark.parametrize("T,H,W,P", [(4, 16, 16, 8), (3, 24, 40, 8), (2, 12, 8, 4)])
def test_fractal_patch_contiguity(T, H, W, P):
    """Invariants stated by the page: each run of P*P fractal positions is exactly
    one P x P patch of one frame, frames appear in order, and inside a frame the
    patches are visited row-major (reading R1)."""
    src = oracle.fractal_positions(T, H, W, P)
    t = src // (H * W)
    y = (src // W) % H
    x = src % W
    prev = (-1, -1, -1)
    for b in range(len(src) // (P * P)):
        sl = slice(b * P * P, (b + 1) * P * P)
        tb, yb, xb = t[sl], y[sl], x[sl]
        assert len(set(tb)) == 1
        y0, x0 = yb.min(), xb.min()
        assert y0 % P == 0 and x0 % P == 0
        cells = set(zip(yb - y0, xb - x0))
        assert cells == {(a, c) for a in range(P) for c in range(P)}
        # row-major inside the patch
        assert list(zip(yb - y0, xb - x0)) == [(a, c) for a in range(P) for c in range(P)]
        key = (tb[0], y0 // P, x0 // P)
        assert key > prev
        prev = key


# ---------------------------------------------------------------- a2: pooling
def test_pool_closed_form_token_index():
    """Value = original token index n = (t*H + y)*W + x is affine in (t, y, x), so the
    mean over patch (t, py, px) is (t*H + py*P + (P-1)/2)*W + px*P + (P-1)/2."""
    T, H, W, P = 3, 16, 24, 8
    L = T * H * W
    x = np.repeat(np.arange(L, dtype=np.float64)[:, None], 2, axis=1)
    pooled = oracle.pool_blocks(oracle.permute(x, T, H, W, P), P * P)
    Hp, Wp = H // P, W // P
    i = 0
    for t in range(T):
        for py in range(Hp):
            for px in range(Wp):
                expect = (t * H + py * P + (P - 1) / 2) * W + px * P + (P - 1) / 2
                assert pooled[i, 0] == expect and pooled[i, 1] == expect
                i += 1


def test_pool_constant_and_linear():
    rng = np.random.default_rng(1)
    c = np.full((2, 256, 5), 3.25)
    assert np.all(oracle.pool_blocks(c, 64) == 3.25)
    a, b = rng.standard_normal((2, 256, 5)), rng.standard_normal((2, 256, 5))
    lhs = oracle.pool_blocks(2.0 * a - 0.5 * b, 64)
    rhs = 2.0 * oracle.pool_blocks(a, 64) - 0.5 * oracle.pool_blocks(b, 64)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-14)


def test_pool_brute_force_loop():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((128, 3))
    p = oracle.pool_blocks(x, 32)
    for i in range(4):
        for d in range(3):
            assert math.isclose(p[i, d], math.fsum(x[i * 32 + m, d] for m in range(32)) / 32,
                                rel_tol=0, abs_tol=1e-15)


# ---------------------------------------------------------------- a3: reduced map
def test_map_two_block_closed_form_pins_scale():
    """D = 64 so sqrt(D) = 8: logits 8*ln3*u/u / 8 = ln 3 and 0 -> probabilities 3/4, 1/4.
    Dropping the 1/sqrt(D) scale or using 1/D gives different numbers."""
    D, u = 64, 0.37
    Qp = np.zeros((1, D)); Qp[0, 0] = u
    Kp = np.zeros((2, D)); Kp[0, 0] = 8.0 * math.log(3.0) / u
    A = oracle.reduced_map(Qp, Kp)
    assert abs(A[0, 0] - 0.75) < 1e-15 and abs(A[0, 1] - 0.25) < 1e-15


def test_map_brute_force_and_library():
    rng = np.random.default_rng(3)
    S, D = 16, 8
    Qp, Kp = rng.standard_normal((S, D)) * 3, rng.standard_normal((S, D)) * 3
    A = oracle.reduced_map(Qp, Kp)
    for i in range(S):
        z = [math.fsum(Qp[i, d] * Kp[j, d] for d in range(D)) / math.sqrt(D) for j in range(S)]
        zm = max(z)
        e = [math.exp(v - zm) for v in z]
        s = math.fsum(e)
        for j in range(S):
            assert abs(A[i, j] - e[j] / s) < 1e-14
    ref = scipy.special.softmax(Qp @ Kp.T / math.sqrt(D), axis=1)
    assert np.allclose(A, ref, rtol=1e-13, atol=1e-16)
    assert np.allclose(A.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_map_row_shift_invariance_and_query_direction():
    """Adding a common vector to every Kp row adds a per-row constant to the logits:
    the map must not change.  Swapping Qp and Kp transposes the logits, which changes
    a non-symmetric map (catches a transposed product)."""
    rng = np.random.default_rng(4)
    Qp, Kp = rng.standard_normal((12, 16)), rng.standard_normal((12, 16))
    c = rng.standard_normal(16) * 5
    assert np.allclose(oracle.reduced_map(Qp, Kp), oracle.reduced_map(Qp, Kp + c), atol=1e-13)
    A = oracle.reduced_map(Qp, Kp)
    assert not np.allclose(A, oracle.reduced_map(Kp, Qp))
    # row i must depend only on Qp[i]
    Qp2 = Qp.copy(); Qp2[3] *= -2
    A2 = oracle.reduced_map(Qp2, Kp)
    assert np.array_equal(np.delete(A, 3, 0), np.delete(A2, 3, 0))


# ---------------------------------------------------------------- a4: CDF threshold
@pytest.mark.parametrize("row", list(_rows("uniform_kept_counts.txt")))
def test_cdf_uniform_closed_form(row):
    S, thr, K = int(row[0]), float(row[1]), int(row[2])
    D = 8
    rng = np.random.default_rng(5)
    Qp = rng.standard_normal((S, D))
    Kp = np.tile(rng.standard_normal((1, D)), (S, 1))        # identical key blocks -> uniform rows
    A = oracle.reduced_map(Qp, Kp)
    assert np.all(A == A[:, :1])                              # exactly uniform (bit-equal)
    keep, _ = oracle.cdf_keep(A, thr)
    expect = np.zeros(S, dtype=bool); expect[:K] = True      # ties -> lowest indices first
    for r in range(S):
        assert np.array_equal(keep[r], expect), (r, keep[r].sum(), K)


def test_cdf_one_hot_row():
    A = np.full((1, 10), 0.01 / 9); A[0, 6] = 0.99
    keep, c = oracle.cdf_keep(A, 0.05)
    assert keep.sum() == 1 and keep[0, 6]
    assert c[0, 6] == 0.0


def test_cdf_brute_force_over_subsets():
    """For S <= 10, the kept set must have the minimum cardinality among subsets with
    mass >= 1-thr, and among those it must be the one of largest mass (the top-K set,
    unique for distinct probabilities)."""
    rng = np.random.default_rng(6)
    for trial in range(60):
        S = int(rng.integers(2, 11))
        p = rng.gamma(0.6, size=S); p /= p.sum()
        thr = float(rng.choice([0.02, 0.1, 0.2, 0.35, 0.5, 0.8]))
        keep, _ = oracle.cdf_keep(p[None, :], thr)
        kept = set(np.nonzero(keep[0])[0].tolist())
        best = None
        for k in range(1, S + 1):
            sets = [set(c) for c in itertools.combinations(range(S), k)
                    if math.fsum(p[list(c)]) >= 1 - thr]
            if sets:
                best = sets
                break
        assert len(kept) == k
        assert kept in best
        masses = [math.fsum(p[sorted(b)]) for b in best]
        assert kept == best[int(np.argmax(masses))]


def test_cdf_thr_zero_keeps_underflowed_blocks():
    Qp = np.array([[100.0, 0.0]])
    Kp = np.array([[100.0, 0.0], [-100.0, 0.0], [0.0, 1.0]])   # logits 7071, -7071, 0 -> exp underflows
    A = oracle.reduced_map(Qp, Kp)
    assert A[0, 1] == 0.0 and A[0, 2] == 0.0
    keep, _ = oracle.cdf_keep(A, 0.0)
    assert keep.all()
    keep, _ = oracle.cdf_keep(A, 1e-9)
    assert keep[0].tolist() == [True, False, False]


def test_cdf_monotone_in_thr_and_nonempty():
    rng = np.random.default_rng(7)
    A = scipy.special.softmax(rng.standard_normal((50, 40)) * 3, axis=1)
    prev = None
    for thr in [0.0, 0.01, 0.05, 0.1, 0.3, 0.6, 0.9, 0.999]:
        keep, c = oracle.cdf_keep(A, thr)
        assert keep.sum(axis=1).min() >= 1
        if prev is not None:
            assert np.all(prev | ~keep)      # kept(thr2) subset of kept(thr1) for thr1 < thr2
        prev = keep
        # mass of the kept set reaches 1-thr, and dropping its smallest block falls short
        mass = (A * keep).sum(axis=1)
        assert np.all(mass >= 1 - thr - 1e-12)
        smallest = np.where(keep, A, np.inf).min(axis=1)
        if thr > 0:
            assert np.all((mass - smallest < 1 - thr + 1e-12) | (keep.sum(axis=1) == 1))


def test_cdf_exclusive_prefix_values():
    A = np.array([[0.1, 0.4, 0.2, 0.3]])
    keep, c = oracle.cdf_keep(A, 0.25)
    # order: 1 (0.4), 3 (0.3), 2 (0.2), 0 (0.1); exclusive prefix 0, .4, .7, .9
    assert np.allclose(c[0], [0.9, 0.0, 0.7, 0.4], atol=1e-15)
    assert keep[0].tolist() == [False, True, True, True]      # .7 < .75 keeps block 2; .9 >= .75 drops 0


# ---------------------------------------------------------------- STA window
@pytest.mark.parametrize("row", list(_rows("sta_pair_counts.txt")))
def test_sta_pair_count_closed_form(row):
    T, Hp, Wp, wt, wh, ww, count = map(int, row)
    m = oracle.sta_window(T, Hp, Wp, (wt, wh, ww))
    assert int(m.sum()) == count
    assert np.array_equal(m, m.T)
    assert np.all(np.diag(m))


def test_sta_neighbours_of_one_tile():
    T, Hp, Wp = 4, 3, 5
    m = oracle.sta_window(T, Hp, Wp, (1, 1, 1))
    i = (2 * Hp + 0) * Wp + 4           # tile (t=2, y=0, x=4): corner in y and x
    js = set(np.nonzero(m[i])[0].tolist())
    expect = {(t * Hp + y) * Wp + x for t in (1, 2, 3) for y in (0, 1) for x in (3, 4)}
    assert js == expect


def test_mask_union_with_window():
    cfg = get_config(0)
    d = make_inputs(cfg)
    m0 = oracle.build_mask(d["q"], d["k"], cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block, cfg.thr, None, details=True)
    m1 = oracle.build_mask(d["q"], d["k"], cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block, cfg.thr, (1, 1, 1), details=True)
    win = oracle.sta_window(cfg.T, cfg.H // cfg.patch, cfg.W // cfg.patch, (1, 1, 1))
    assert np.array_equal(m1["keep"], m0["keep"] | win[None, None])


# ---------------------------------------------------------------- a5: attention
def _small_problem(seed=8, B=1, nh=2, T=2, H=16, W=16, D=16):
    rng = np.random.default_rng(seed)
    L = T * H * W
    q, k, v = (rng.standard_normal((B, nh, L, D)) for _ in range(3))
    return q, k, v, T, H, W


def test_thr_zero_is_dense_attention_vs_torch_sdpa():
    torch = pytest.importorskip("torch")
    q, k, v, T, H, W = _small_problem()
    O, LSE, mask = oracle.attention_pipeline(q, k, v, T, H, W, 8, 64, 0.0)
    S = T * H * W // 64
    assert mask["row_ptr"][-1] == q.shape[0] * q.shape[1] * S * S
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v)).numpy()
    assert np.abs(O - ref).max() < 1e-12
    Od, LSEd = oracle.dense_attention(q, k, v)
    assert np.abs(O - Od).max() < 1e-12
    z = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(q.shape[-1])
    assert np.abs(LSE - scipy.special.logsumexp(z, axis=-1)).max() < 1e-12


def test_single_block_sequence_is_dense():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 3, 64, 32)) * 2 for _ in range(3))
    for thr in (0.0, 0.1, 0.9):
        O, _, mask = oracle.attention_pipeline(q, k, v, 1, 8, 8, 8, 64, thr)
        Od, _ = oracle.dense_attention(q, k, v)
        assert np.abs(O - Od).max() < 1e-12


def test_convex_combination_and_dropped_keys_ignored():
    q, k, v, T, H, W = _small_problem(seed=10, T=2, H=16, W=24)
    N = 64
    qf, kf, vf = (oracle.permute(x, T, H, W, 8) for x in (q, k, v))
    m = oracle.build_mask(qf, kf, T, H, W, 8, N, 0.3, layout="fractal")
    rp, ci = m["row_ptr"], m["col_idx"]
    O, _ = oracle.block_sparse_attention(qf, kf, vf, rp, ci, N)
    S = qf.shape[2] // N
    nh = qf.shape[1]
    for r in range(nh * S):
        h, i = divmod(r, S)
        keys = (ci[rp[r]:rp[r + 1]][:, None] * N + np.arange(N)).ravel()
        lo, hi = vf[0, h, keys].min(axis=0), vf[0, h, keys].max(axis=0)
        o = O[0, h, i * N:(i + 1) * N]
        assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)
    ones = np.ones_like(vf)
    O1, _ = oracle.block_sparse_attention(qf, kf, ones, rp, ci, N)
    assert np.abs(O1 - 1).max() < 1e-12
    # replace every dropped key/value tile with garbage: nothing changes
    keep = m["keep"].reshape(nh * S, S)
    kf2, vf2 = kf.copy(), vf.copy()
    for r in range(nh * S):
        h, i = divmod(r, S)
    dropped_everywhere = ~keep.reshape(nh, S, S).any(axis=1)     # key blocks no query keeps
    for h in range(nh):
        for j in np.nonzero(dropped_everywhere[h])[0]:
            kf2[0, h, j * N:(j + 1) * N] = 1e3
            vf2[0, h, j * N:(j + 1) * N] = -1e6
    O2, _ = oracle.block_sparse_attention(qf, kf2, vf2, rp, ci, N)
    assert np.array_equal(O, O2)


def test_attention_weights_are_softmax_over_kept_keys():
    """Using V = identity over the kept keys exposes the weights; they must equal the
    softmax over exactly the kept keys (scipy) and be zero elsewhere."""
    rng = np.random.default_rng(11)
    N, S, D = 64, 3, 8
    L = N * S
    qf = rng.standard_normal((1, 1, L, D)); kf = rng.standard_normal((1, 1, L, D))
    vf = np.eye(L)[None, None]
    rp = np.array([0, 1, 3, 4]); ci = np.array([2, 0, 2, 1], dtype=np.int32)
    O, LSE = oracle.block_sparse_attention(qf, kf, vf, rp, ci, N)
    for r, cols in enumerate([[2], [0, 2], [1]]):
        keys = np.concatenate([np.arange(c * N, (c + 1) * N) for c in cols])
        z = qf[0, 0, r * N:(r + 1) * N] @ kf[0, 0, keys].T / math.sqrt(D)
        w = scipy.special.softmax(z, axis=1)
        got = O[0, 0, r * N:(r + 1) * N]
        assert np.abs(got[:, keys] - w).max() < 1e-14
        others = np.setdiff1d(np.arange(L), keys)
        assert np.all(got[:, others] == 0)
        assert np.abs(LSE[0, 0, r * N:(r + 1) * N] - scipy.special.logsumexp(z, axis=1)).max() < 1e-12


def test_attention_invariant_to_column_order():
    q, k, v, T, H, W = _small_problem(seed=12)
    N = 64
    m = oracle.build_mask(q, k, T, H, W, 8, N, 0.2, layout="fractal")
    rp, ci = m["row_ptr"], m["col_idx"].copy()
    O, _ = oracle.block_sparse_attention(q, k, v, rp, ci, N)
    ci2 = ci.copy()
    for r in range(len(rp) - 1):
        ci2[rp[r]:rp[r + 1]] = ci2[rp[r]:rp[r + 1]][::-1]
    O2, _ = oracle.block_sparse_attention(q, k, v, rp, ci2, N)
    assert np.abs(O - O2).max() < 1e-13


def test_head_mask_uses_fractal_blocks():
    """Pipeline on original-order inputs equals the fractal-layout mask on permuted inputs,
    and differs from (mis)pooling raw original-order runs when the content is local."""
    cfg = get_config(0)
    d = make_inputs(cfg)
    T, H, W, P, N = cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block
    m_orig = oracle.build_mask(d["q"], d["k"], T, H, W, P, N, cfg.thr)
    qf, kf = oracle.permute(d["q"], T, H, W, P), oracle.permute(d["k"], T, H, W, P)
    m_frac = oracle.build_mask(qf, kf, T, H, W, P, N, cfg.thr, layout="fractal")
    assert np.array_equal(m_orig["row_ptr"], m_frac["row_ptr"])
    assert np.array_equal(m_orig["col_idx"], m_frac["col_idx"])
    m_raw = oracle.build_mask(d["q"], d["k"], T, H, W, P, N, cfg.thr, layout="fractal")
    assert not np.array_equal(m_orig["keep"], m_raw["keep"])


def test_cdf_tie_break_inside_a_large_tie_group():
    """S = 240 blocks on four probability levels in shuffled positions; the cut falls
    inside a tie group, so exactly the lowest-index members of that group are kept
    (reading R4: ties ordered by block index ascending)."""
    rng = np.random.default_rng(13)
    S = 240
    levels = np.repeat([8.0, 4.0, 2.0, 1.0], S // 4)          # 60 blocks per level
    p = levels[rng.permutation(S)]
    p = p / p.sum()                                           # total 900 units -> 1
    # level masses are 480, 240, 120 and 60 out of 900.  thr = 0.25 needs 675/900: all
    # 60 blocks of level 8 (480) plus 195 units of level 4, i.e. ceil(48.75) = 49 blocks.
    keep, _ = oracle.cdf_keep(p[None, :], 0.25)
    lvl4 = np.nonzero(p == p.max() / 2)[0]                    # ascending indices
    assert keep[0][p == p.max()].all()
    assert keep[0][p < p.max() / 2].sum() == 0
    assert np.array_equal(np.nonzero(keep[0] & (p == p.max() / 2))[0], lvl4[:49])
