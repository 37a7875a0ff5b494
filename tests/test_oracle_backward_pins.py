"""Pins for oracle.block_sparse_attention_backward: central finite differences of
the oracle's own forward on tiny sparse problems (the gradient is the derivative
of what the forward computes), and torch autograd of textbook softmax attention
in float64 when every tile is kept."""
import math

import numpy as np
import pytest
import torch

import oracle


def _sparse_problem(seed, S=4, N=4, D=4, B=1, nh=2, density=0.5):
    rng = np.random.default_rng(seed)
    L = S * N
    q, k, v, do = (rng.standard_normal((B, nh, L, D)) for _ in range(4))
    keep = rng.random((B * nh * S, S)) < density
    keep[np.arange(B * nh * S), rng.integers(0, S, B * nh * S)] = True      # no empty row
    row_ptr, col_idx = oracle.csr_from_keep(keep)
    return q, k, v, do, row_ptr, col_idx, N


def _loss(q, k, v, do, row_ptr, col_idx, N):
    O, _ = oracle.block_sparse_attention(q, k, v, row_ptr, col_idx, N)
    return float((O * do).sum())


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_backward_matches_finite_differences(seed):
    q, k, v, do, rp, ci, N = _sparse_problem(seed)
    dQ, dK, dV = oracle.block_sparse_attention_backward(q, k, v, rp, ci, do, N)
    h = 1e-6
    rng = np.random.default_rng(100 + seed)
    for name, x, g in (("q", q, dQ), ("k", k, dK), ("v", v, dV)):
        for _ in range(12):
            idx = tuple(rng.integers(0, s) for s in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            fp = _loss(*(xp if n == name else args[n] for n in "qkv"), do, rp, ci, N)
            fm = _loss(*(xm if n == name else args[n] for n in "qkv"), do, rp, ci, N)
            num = (fp - fm) / (2 * h)
            assert abs(num - g[idx]) <= 1e-6 * max(1.0, abs(num)), (name, idx, num, g[idx])


def test_dropped_tiles_get_no_gradient():
    q, k, v, do, rp, ci, N = _sparse_problem(5, S=6, density=0.3)
    _, dK, dV = oracle.block_sparse_attention_backward(q, k, v, rp, ci, do, N)
    keep = np.zeros((len(rp) - 1, 6), bool)
    for r in range(len(rp) - 1):
        keep[r, ci[rp[r]:rp[r + 1]]] = True
    B, nh, L, D = q.shape
    used = keep.reshape(B, nh, 6, 6).any(axis=2)           # key blocks some query block keeps
    for b in range(B):
        for h in range(nh):
            for j in range(6):
                if not used[b, h, j]:
                    assert not dK[b, h, j * N:(j + 1) * N].any() and not dV[b, h, j * N:(j + 1) * N].any()


def test_dense_mask_matches_torch_autograd():
    rng = np.random.default_rng(7)
    B, nh, S, N, D = 1, 2, 3, 4, 8
    L = S * N
    q, k, v, do = (rng.standard_normal((B, nh, L, D)) for _ in range(4))
    rp, ci = oracle.csr_from_keep(np.ones((B * nh * S, S), bool))
    dQ, dK, dV = oracle.block_sparse_attention_backward(q, k, v, rp, ci, do, N)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    p = torch.softmax(tq @ tk.transpose(-1, -2) / math.sqrt(D), dim=-1)
    (p @ tv * torch.tensor(do)).sum().backward()
    for mine, ref in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        assert np.allclose(mine, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_row_term_from_the_exact_output_changes_nothing():
    q, k, v, do, rp, ci, N = _sparse_problem(11)
    O, _ = oracle.block_sparse_attention(q, k, v, rp, ci, N)
    a = oracle.block_sparse_attention_backward(q, k, v, rp, ci, do, N)
    b = oracle.block_sparse_attention_backward(q, k, v, rp, ci, do, N, O=O)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-12)
    # a perturbed output moves dQ and dK but never dV
    c = oracle.block_sparse_attention_backward(q, k, v, rp, ci, do, N, O=O * 1.01)
    assert not np.allclose(a[0], c[0]) and np.array_equal(a[2], c[2])
