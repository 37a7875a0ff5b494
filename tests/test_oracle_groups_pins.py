"""Pins for oracle/groups.py (4-token key groups, AB-Attention page, third resource):
the group path must reduce exactly to the NABLA block path when a group is a whole
block, a block CSR expanded to groups must give block attention, group attention
must equal torch float64 attention under a token-level mask built here from the
group list, and group means must be linear (the mean of a block's group logits is
the block logit)."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import groups


def _inputs(seed, B=1, nh=2, T=2, H=16, W=16, D=16, amp=2.0):
    rng = np.random.default_rng(seed)
    L = T * H * W
    q, k, v = (rng.standard_normal((B, nh, L, D)) for _ in range(3))
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    pos = amp * np.sin(np.pi * (t / T + y / H + x / W)).reshape(-1)
    return q + pos[None, None, :, None], k + pos[None, None, :, None], v


@pytest.mark.parametrize("thr,window", [(0.1, None), (0.3, (1, 1, 1)), (0.0, None)])
def test_groups_of_a_whole_block_are_the_block_path(thr, window):
    T, H, W, P, N = 2, 16, 16, 8, 64
    q, k, v = _inputs(1, T=T, H=H, W=W)
    bm = oracle.build_mask(q, k, T, H, W, P, N, thr, window, details=True)
    gm = groups.build_group_mask(q, k, T, H, W, P, N, N, thr, window, details=True)
    assert np.array_equal(gm["row_ptr"], bm["row_ptr"]) and np.array_equal(gm["col_idx"], bm["col_idx"])
    assert np.allclose(gm["A"], bm["A"], rtol=0, atol=1e-15)
    src = oracle.fractal_positions(T, H, W, P)
    qf, kf, vf = (x[:, :, src] for x in (q, k, v))
    Ob, Lb = oracle.block_sparse_attention(qf, kf, vf, bm["row_ptr"], bm["col_idx"], N)
    Og, Lg = groups.group_attention(qf, kf, vf, gm["row_ptr"], gm["col_idx"], N, N)
    assert np.array_equal(Ob, Og) and np.array_equal(Lb, Lg)


def test_expanded_block_csr_gives_block_attention():
    T, H, W, P, N, G = 2, 16, 16, 8, 64, 4
    q, k, v = _inputs(2, T=T, H=H, W=W)
    src = oracle.fractal_positions(T, H, W, P)
    qf, kf, vf = (x[:, :, src] for x in (q, k, v))
    bm = oracle.build_mask(q, k, T, H, W, P, N, 0.2)
    rp, ci = groups.expand_block_csr(bm["row_ptr"], bm["col_idx"], N // G)
    assert np.all(np.diff(rp) == (N // G) * np.diff(bm["row_ptr"]))
    Ob, Lb = oracle.block_sparse_attention(qf, kf, vf, bm["row_ptr"], bm["col_idx"], N)
    Og, Lg = groups.group_attention(qf, kf, vf, rp, ci, N, G)
    assert np.allclose(Ob, Og, rtol=0, atol=1e-12) and np.allclose(Lb, Lg, rtol=0, atol=1e-12)


def test_group_attention_matches_masked_torch_attention():
    """Random group lists (including a row with a single group): torch float64
    softmax attention with -inf on every token outside the row's groups."""
    rng = np.random.default_rng(3)
    B, nh, L, D, N, G = 1, 2, 256, 16, 64, 4
    S, SG = L // N, L // G
    q, k, v = (rng.standard_normal((B, nh, L, D)) for _ in range(3))
    keep = rng.random((B * nh * S, SG)) < 0.3
    keep[0] = False
    keep[0, 17] = True
    keep[:, 0] |= ~keep.any(axis=1)
    rp, ci = oracle.csr_from_keep(keep)
    O, LSE = groups.group_attention(q, k, v, rp, ci, N, G)
    allowed = torch.zeros(B, nh, L, L, dtype=torch.bool)
    for r in range(B * nh * S):
        bh, i = divmod(r, S)
        for gid in ci[rp[r]:rp[r + 1]]:
            allowed.view(B * nh, L, L)[bh, i * N:(i + 1) * N, gid * G:(gid + 1) * G] = True
    tq, tk, tv = (torch.tensor(x) for x in (q, k, v))
    z = tq @ tk.transpose(-1, -2) / math.sqrt(D)
    z = z.masked_fill(~allowed, -math.inf)
    ref = torch.softmax(z, dim=-1) @ tv
    assert np.allclose(O, ref.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(LSE, torch.logsumexp(z, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_empty_row_gives_zero_output():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 1, 128, 8)) for _ in range(3))
    rp = np.array([0, 0, 3])
    ci = np.array([1, 5, 30], np.int32)
    O, LSE = groups.group_attention(q, k, v, rp, ci, 64, 4)
    assert np.all(O[0, 0, :64] == 0) and np.all(np.isneginf(LSE[0, 0, :64]))
    assert np.all(np.isfinite(O[0, 0, 64:]))


def test_group_logits_average_to_block_logits():
    """Kp_j = mean of its groups' Kg, so the block logit is the mean of the group
    logits; in log-probabilities the row normalisers cancel in differences."""
    T, H, W, P, N, G = 2, 16, 16, 8, 64, 4
    q, k, _ = _inputs(5, T=T, H=H, W=W, amp=1.0)
    bm = oracle.build_mask(q, k, T, H, W, P, N, 0.1, details=True)
    gm = groups.build_group_mask(q, k, T, H, W, P, N, G, 0.1, details=True)
    lb = np.log(bm["A"])                                           # [B, nh, S, S]
    lg = np.log(gm["A"]).reshape(lb.shape + (N // G,)).mean(-1)    # mean over each block's groups
    db = lb - lb[..., :1]
    dg = lg - lg[..., :1]
    assert np.allclose(db, dg, rtol=0, atol=1e-9)


def test_thr_zero_keeps_every_group_and_is_dense():
    T, H, W, P, N, G = 2, 8, 16, 8, 64, 4
    q, k, v = _inputs(6, T=T, H=H, W=W)
    gm = groups.build_group_mask(q, k, T, H, W, P, N, G, 0.0, layout="original")
    L = T * H * W
    assert gm["keep"].all() and gm["row_ptr"][-1] == q.shape[0] * q.shape[1] * (L // N) * (L // G)
    src = oracle.fractal_positions(T, H, W, P)
    qf, kf, vf = (x[:, :, src] for x in (q, k, v))
    O, LSE = groups.group_attention(qf, kf, vf, gm["row_ptr"], gm["col_idx"], N, G)
    Od, Ld = oracle.dense_attention(qf, kf, vf)
    assert np.allclose(O, Od, rtol=0, atol=1e-12) and np.allclose(LSE, Ld, rtol=0, atol=1e-12)


def test_window_keeps_whole_blocks_of_groups():
    T, H, W, P, N, G = 3, 16, 16, 8, 64, 4
    q, k, _ = _inputs(7, T=T, H=H, W=W)
    gm = groups.build_group_mask(q, k, T, H, W, P, N, G, 0.5, window=(1, 0, 0), details=True)
    w = groups.group_window(T, H // P, W // P, (1, 0, 0), N // G)
    assert np.all(gm["keep"] >= w[None, None]) and np.array_equal(gm["keep"], gm["cdf_keep"] | w[None, None])
    # the window at group level is the block window repeated over each block's groups
    bw = oracle.sta_window(T, H // P, W // P, (1, 0, 0))
    assert np.array_equal(w.reshape(bw.shape + (N // G,)).all(-1), bw)
    assert np.array_equal(w.reshape(bw.shape + (N // G,)).any(-1), bw)


def test_finer_groups_keep_fewer_keys_for_the_same_mass():
    """On the page's premise (finer blocks retain more mass per tile): with the
    same threshold, the group cut reaches 1 - thr of the (group-level) map with
    no more keys than the block cut needs on the block map, on local inputs."""
    T, H, W, P, N, G = 2, 16, 16, 8, 64, 4
    q, k, _ = _inputs(8, T=T, H=H, W=W, amp=3.0)
    bm = oracle.build_mask(q, k, T, H, W, P, N, 0.2)
    gm = groups.build_group_mask(q, k, T, H, W, P, N, G, 0.2)
    assert gm["row_ptr"][-1] * G <= bm["row_ptr"][-1] * N
