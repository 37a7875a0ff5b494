"""GPU parity of the backward pass (dQ, dK, dV) against the float64 oracle
(oracle.block_sparse_attention_backward) on the GPU's own mask.

Like any kernel that stores O rather than P, the backward forms the row term
Delta_n = dO_n . o_n from the forward's output, so the oracle is given the same
(rounded) O; with the exact O the two forms agree (pinned on the CPU).
Tolerances, derived from the arithmetic: float32 tensors go through float64
kernels, so the error is the float32 rounding of the lse the kernels read back
(P's relative error is 2^-24 |lse|): max-abs (1e-5 + 2^-23 max|lse|) of the
gradient's scale.  bf16 tensors take the forward's bar (mean-relative 5e-3,
max-abs 2e-2) relative to the gradient's scale (max |reference|): dV and dK
round P and dZ to bf16 once (2^-9 per term, no cancellation, ~2e-3 measured on
the CPU by rounding the oracle's own P and dZ), and dQ, whose dZ terms of one
query sum to zero, carries dZ as a hi + lo pair of bf16 values."""
import numpy as np
import pytest
import torch

import oracle
from parity import to_device, to_host_f64
from workloads import bf16_bits_to_f32, bf16_round, get_config, make_inputs
from workloads.configs import Config

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_fractal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa.lib()


def grid_of(cfg):
    return bsa.VideoGrid(cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block)


def small_cfg(dtype="bf16", B=1, nh=2, T=3, H=24, W=40, D=128, thr=0.1, amp=3.0, seed=7):
    return Config(99, "edge", dtype, B, nh, T, H, W, D, 8, 64, thr, None, amp, seed=seed)


def dout_for(cfg, seed=123):
    rng = np.random.default_rng(seed)
    d = rng.standard_normal((cfg.batch, cfg.heads, cfg.L, cfg.head_dim)).astype(np.float32)
    return bf16_bits_to_f32(bf16_round(d)) if cfg.dtype == "bf16" else d


def to_dev(x: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def grad_errors(got, ref, dtype, name, lse_max=0.0):
    """Returns (ok, message) for one gradient tensor."""
    scale = max(1.0, float(np.abs(ref).max()))
    err = np.abs(got - ref)
    bad = ~np.isfinite(got)
    if bad.any():
        return False, f"{name}: {int(bad.sum())} non-finite values, first at {np.argwhere(bad)[:4].tolist()}"
    mean_rel = err.mean() / max(np.abs(ref).mean(), 1e-30)
    msg = f"{name}: max_abs {err.max():.3e} mean_rel {mean_rel:.3e} (scale {scale:.3e})"
    if dtype == "f32":
        return err.max() <= (1e-5 + 2.0 ** -23 * lse_max) * scale, msg
    return mean_rel <= 5e-3 and err.max() <= 2e-2 * scale, msg


def run_case(cfg, inputs, row_ptr=None, col_idx=None, thr=None):
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    g = grid_of(cfg)
    if row_ptr is None:
        mask = bsa.build_mask(q, k, g, cfg.thr if thr is None else thr, cfg.window)
    else:
        mask = bsa.mask_from_csr(torch.from_numpy(row_ptr.astype(np.int32)).cuda(),
                                 torch.from_numpy(col_idx.astype(np.int32)).cuda(), cfg.S)
    o, lse = bsa.forward(q, k, v, mask, g, return_lse=True)
    do_np = dout_for(cfg)
    dq, dk, dv = bsa.backward(q, k, v, mask, g, o, lse, to_dev(do_np, cfg.dtype))
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    qf, kf, vf, dof = (x[:, :, src] for x in (inputs["q"], inputs["k"], inputs["v"], do_np))
    of = to_host_f64(o)[:, :, src]
    rdq, rdk, rdv = oracle.block_sparse_attention_backward(qf, kf, vf, rp, ci, dof, cfg.block, O=of)
    lse_max = float(lse.abs().max())
    res = []
    for name, got, ref in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv)):
        ref_o = np.empty_like(ref)
        ref_o[:, :, src] = ref
        res.append(grad_errors(to_host_f64(got), ref_o, cfg.dtype, name, lse_max))
    msg = "; ".join(m for _, m in res)
    print(msg)
    assert all(ok for ok, _ in res), msg
    return msg


@pytest.mark.parametrize("ci", [0, 1])
def test_backward_matches_oracle(ci):
    cfg = get_config(ci)
    run_case(cfg, make_inputs(cfg))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_backward_odd_blocks_and_unused_keys(dtype, D):
    """S = 15 (the last pair of query and key blocks is half empty) and a hand-made
    CSR in which key blocks 3 and 11 are kept by no row: their dK, dV must be 0."""
    cfg = small_cfg(dtype=dtype, D=D, T=1, H=24, W=40, seed=9)
    assert cfg.S == 15
    rng = np.random.default_rng(4)
    allowed = np.array([j for j in range(15) if j not in (3, 11)])
    keep = np.zeros((cfg.rows, 15), bool)
    for r in range(cfg.rows):
        keep[r, rng.choice(allowed, size=rng.integers(1, 6), replace=False)] = True
    rp, ci = oracle.csr_from_keep(keep)
    run_case(cfg, make_inputs(cfg), rp, ci)


def test_backward_dense_mask_bf16():
    cfg = small_cfg(nh=2, T=2, H=16, W=32, thr=0.0, seed=31)
    run_case(cfg, make_inputs(cfg), thr=0.0)


def test_backward_fullsize_sampled():
    """The Wan2.1-scale workload (40 heads, 21 x 32 x 48 tokens) at full size, as the
    benchmark's backward leg runs it: dQ on sampled query blocks (the oracle needs
    only that row's keys) and dK, dV on sampled key blocks (the oracle sums exactly
    the rows whose CSR keeps the block), on three heads."""
    cfg = get_config(2)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    for n in ("q_bits", "k_bits", "v_bits"):
        inputs.pop(n)
    mask = bsa.build_mask(q, k, g, cfg.thr, cfg.window)
    o, lse = bsa.forward(q, k, v, mask, g, return_lse=True)
    do_np = dout_for(cfg)
    dq, dk, dv = bsa.backward(q, k, v, mask, g, o, lse, to_dev(do_np, cfg.dtype))
    torch.cuda.synchronize()
    S = cfg.S
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    o_h = to_host_f64(o)
    grads = [to_host_f64(x) for x in (dq, dk, dv)]
    rng = np.random.default_rng(8)
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for h in (0, 17, 39):
        r0 = h * S
        lo, hi = int(rp[r0]), int(rp[r0 + S])
        ci = mask.col_idx[lo:hi].cpu().numpy()
        prp = rp[r0:r0 + S + 1] - lo
        qf, kf, vf, dof = (x[0:1, h:h + 1][:, :, src] for x in (inputs["q"], inputs["k"], inputs["v"], do_np))
        of = o_h[0:1, h:h + 1][:, :, src]
        qrows = sorted(rng.choice(S, 8, replace=False).tolist())
        rdq, _, _ = oracle.block_sparse_attention_backward(qf, kf, vf, prp, ci, dof, 64, rows=qrows, O=of)
        for i in qrows:
            tok = src[i * 64:(i + 1) * 64]
            got["dq"].append(grads[0][0, h, tok])
            ref["dq"].append(rdq[0, 0, i * 64:(i + 1) * 64])
        rows_of = np.repeat(np.arange(S), np.diff(prp))
        for j in rng.choice(S, 4, replace=False):
            krows = sorted(set(rows_of[ci == j].tolist()))
            if not krows:
                continue
            _, rdk, rdv = oracle.block_sparse_attention_backward(qf, kf, vf, prp, ci, dof, 64, rows=krows, O=of)
            tok = src[j * 64:(j + 1) * 64]
            got["dk"].append(grads[1][0, h, tok])
            ref["dk"].append(rdk[0, 0, j * 64:(j + 1) * 64])
            got["dv"].append(grads[2][0, h, tok])
            ref["dv"].append(rdv[0, 0, j * 64:(j + 1) * 64])
    res = [grad_errors(np.stack(got[n]), np.stack(ref[n]), cfg.dtype, n) for n in ("dq", "dk", "dv")]
    msg = "; ".join(m for _, m in res)
    print(msg)
    assert all(ok for ok, _ in res), msg
