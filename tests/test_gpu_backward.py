"""GPU parity of the backward pass (dQ, dK, dV) against the exact float64
gradient of the oracle (oracle.block_sparse_attention_backward with no stored
output: the row term is sum_k P dP from the exact P), on the GPU's own mask.

The kernels recompute the row term from their own P and dP as well, so nothing
of the forward's rounded output enters the gradient.  Tolerances, derived from
the arithmetic: float32 tensors go through float64 kernels, so the error is the
float32 rounding of the lse the kernels read back (P's relative error is
2^-24 |lse|): max-abs (1e-5 + 2^-23 max|lse|) of the gradient's scale.  bf16
tensors take the forward's bar (mean-relative 5e-3, max-abs 2e-2) relative to
the gradient's scale (max |reference|): dV and dK round P and dZ to bf16 once
(2^-9 per term, no cancellation, ~2e-3 measured on the CPU by rounding the
oracle's own P and dZ), and dQ, whose dZ terms of one query sum to zero,
carries dZ as a hi + lo pair of bf16 values.

The training pair (attend_train + backward_train, mode "train") takes the row
term from the forward's output pair o + o_lo instead; its error against the
kernels' own sum P dP / sum P is ~2^-16 |dO||O|, so the same bars apply.  The
pair's output is checked on its own: o within the forward's bf16 bar, o + o_lo
ten times tighter (mean-relative 5e-4, max-abs 2e-3: P enters the PV product as a
bf16 pair, 2^-17, so what remains is the float32 rounding of the logits), and
lse bit-identical to attend's (same float32 sum in the same order)."""
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


def dout_for(cfg, seed=123, batch=None):
    rng = np.random.default_rng(seed)
    d = rng.standard_normal((cfg.batch if batch is None else batch, cfg.heads, cfg.L, cfg.head_dim)).astype(np.float32)
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


def run_case(cfg, inputs, row_ptr=None, col_idx=None, thr=None, mode="walk"):
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    g = grid_of(cfg)
    if row_ptr is None:
        mask = bsa.build_mask(q, k, g, cfg.thr if thr is None else thr, cfg.window)
    else:
        mask = bsa.mask_from_csr(torch.from_numpy(row_ptr.astype(np.int32)).cuda(),
                                 torch.from_numpy(col_idx.astype(np.int32)).cuda(), cfg.S)
    do_np = dout_for(cfg)
    if mode == "train":
        o, o_lo, lse = bsa.attend_train(q, k, bsa.prepare_v(v, g), mask, g)
        dq, dk, dv = bsa.backward_train(q, k, v, mask, g, o, o_lo, lse, to_dev(do_np, cfg.dtype))
    else:
        _, lse = bsa.forward(q, k, v, mask, g, return_lse=True)
        dq, dk, dv = bsa.backward(q, k, v, mask, g, lse, to_dev(do_np, cfg.dtype))
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    qf, kf, vf, dof = (x[:, :, src] for x in (inputs["q"], inputs["k"], inputs["v"], do_np))
    rdq, rdk, rdv = oracle.block_sparse_attention_backward(qf, kf, vf, rp, ci, dof, cfg.block)
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


@pytest.mark.parametrize("ci,mode", [(0, "walk"), (1, "walk"), (1, "train")])
def test_backward_matches_oracle(ci, mode):
    cfg = get_config(ci)
    run_case(cfg, make_inputs(cfg), mode=mode)


@pytest.mark.parametrize("dtype,D,mode", [("bf16", 128, "walk"), ("bf16", 128, "train"), ("f32", 64, "walk")])
def test_backward_odd_blocks_and_unused_keys(dtype, D, mode):
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
    run_case(cfg, make_inputs(cfg), rp, ci, mode=mode)


@pytest.mark.parametrize("mode", ["walk", "train"])
def test_backward_dense_mask_bf16(mode):
    cfg = small_cfg(nh=2, T=2, H=16, W=32, thr=0.0, seed=31)
    run_case(cfg, make_inputs(cfg), thr=0.0, mode=mode)


@pytest.mark.parametrize("mode", ["walk", "train"])
def test_backward_strong_common_key_component(mode):
    """Local heads with the HunyuanVideo-scale positional amplitude (4): every key
    carries a large common component, the case in which a row term that does not
    match the kernel's own P would leak into dQ."""
    cfg = Config(98, "edge", "bf16", 1, 2, 4, 48, 80, 128, 8, 64, 0.05, None, 4.0, seed=17)
    run_case(cfg, make_inputs(cfg), mode=mode)


@pytest.mark.parametrize("dtype,D,mode", [("bf16", 128, "walk"), ("bf16", 128, "train"), ("f32", 64, "walk")])
def test_backward_fractal_layout_matches_original(dtype, D, mode):
    """The whole path in fractal token order (inputs permuted, layout="fractal",
    gradients permuted back) gives gradients bit-identical to the original order's:
    the kernels change only their addressing with the layout."""
    cfg = small_cfg(dtype=dtype, nh=2, T=3, H=16, W=24, D=D, thr=0.2, seed=21)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    dout = to_dev(dout_for(cfg), cfg.dtype)

    def grads(layout):
        x = [q, k, v, dout]
        if layout == "fractal":
            x = [bsa.permute(t, g) for t in x]
        qq, kk, vv, dd = x
        mask = bsa.build_mask(qq, kk, g, cfg.thr, layout=layout)
        if mode == "train":
            o, o_lo, lse = bsa.attend_train(qq, kk, bsa.prepare_v(vv, g, layout=layout), mask, g, layout=layout)
            out = bsa.backward_train(qq, kk, vv, mask, g, o, o_lo, lse, dd, layout=layout)
        else:
            _, lse = bsa.forward(qq, kk, vv, mask, g, layout=layout, return_lse=True)
            out = bsa.backward(qq, kk, vv, mask, g, lse, dd, layout=layout)
        if layout == "fractal":
            out = [bsa.permute(t, g, inverse=True) for t in out]
        torch.cuda.synchronize()
        return [t.cpu() for t in out]

    a, b = grads("original"), grads("fractal")
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        assert torch.equal(x, y), name


@pytest.mark.parametrize("name,cfg", [("small-bf16", get_config(1)),
                                      ("ragged-S15", small_cfg(T=1, H=24, W=40, seed=9)),
                                      ("common-key", Config(98, "edge", "bf16", 1, 2, 4, 48, 80, 128, 8, 64, 0.05,
                                                            None, 4.0, seed=17))],
                         ids=["small-bf16", "ragged-S15", "common-key"])
def test_attend_train_output_pair(name, cfg):
    """attend_train: o within the forward's bf16 bar, o + o_lo ten times tighter,
    lse bit-identical to attend's on the same mask."""
    inputs = make_inputs(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    g = grid_of(cfg)
    mask = bsa.build_mask(q, k, g, cfg.thr, cfg.window)
    vt = bsa.prepare_v(v, g)
    o, o_lo, lse = bsa.attend_train(q, k, vt, mask, g)
    _, lse_ref = bsa.attend(q, k, vt, mask, g, return_lse=True)
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    qf, kf, vf = (inputs[n][:, :, src] for n in "qkv")
    O, _ = oracle.block_sparse_attention(qf, kf, vf, rp, ci, cfg.block)
    ref = np.empty_like(O)
    ref[:, :, src] = O
    hi = to_host_f64(o)
    pair = hi + to_host_f64(o_lo)
    e_hi, e_pair = np.abs(hi - ref), np.abs(pair - ref)
    mr_hi = e_hi.mean() / np.abs(ref).mean()
    mr_pair = e_pair.mean() / np.abs(ref).mean()
    print(f"{name}: o max_abs {e_hi.max():.3e} mean_rel {mr_hi:.3e}; o+o_lo max_abs {e_pair.max():.3e} "
          f"mean_rel {mr_pair:.3e}")
    assert np.array_equal(lse.cpu().numpy(), lse_ref.cpu().numpy())
    assert e_hi.max() <= 2e-2 and mr_hi <= 5e-3
    assert e_pair.max() <= 2e-3 and mr_pair <= 5e-4


@pytest.mark.parametrize("ci,dq_heads,dkv_heads,mode", [(2, (0, 17, 39), (0, 17, 39), "walk"),
                                                        (4, (0, 20), (0, 16), "walk"), (4, (0, 20), (0, 16), "train")])
def test_backward_fullsize_sampled(ci, dq_heads, dkv_heads, mode):
    """Full-size workloads as the benchmark's backward leg runs them: the Wan2.1-scale
    one (40 heads, 21 x 32 x 48 tokens) and one batch item of the HunyuanVideo-scale
    hybrid one (24 heads, 33 x 48 x 80 tokens, sliding-tile window; local heads 0-16,
    diffuse 17-23).  dQ on sampled query blocks (the oracle needs only that row's
    keys) and dK, dV on sampled key blocks (the oracle sums exactly the rows whose
    CSR keeps the block), against the exact gradient.  dQ covers a local and a
    diffuse head; dK, dV cover local heads only at the HunyuanVideo scale, where a
    diffuse head's key block is kept by ~1800 rows of ~1900 blocks each (minutes of
    oracle time per block)."""
    cfg = get_config(ci)
    inputs = make_inputs(cfg, batch=1)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    for n in ("q_bits", "k_bits", "v_bits"):
        inputs.pop(n)
    mask = bsa.build_mask(q, k, g, cfg.thr, cfg.window)
    do_np = dout_for(cfg, batch=1)
    if mode == "train":
        o, o_lo, lse = bsa.attend_train(q, k, bsa.prepare_v(v, g), mask, g)
        dq, dk, dv = bsa.backward_train(q, k, v, mask, g, o, o_lo, lse, to_dev(do_np, cfg.dtype))
        del o, o_lo
    else:
        _, lse = bsa.forward(q, k, v, mask, g, return_lse=True)
        dq, dk, dv = bsa.backward(q, k, v, mask, g, lse, to_dev(do_np, cfg.dtype))
    torch.cuda.synchronize()
    del q, k, v, lse
    S = cfg.S
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    rng = np.random.default_rng(8)
    got = {"dq": [], "dk": [], "dv": []}
    ref = {"dq": [], "dk": [], "dv": []}
    for h in sorted(set(dq_heads) | set(dkv_heads)):
        r0 = h * S
        lo, hi = int(rp[r0]), int(rp[r0 + S])
        ci_ = mask.col_idx[lo:hi].cpu().numpy()
        prp = rp[r0:r0 + S + 1] - lo
        qf, kf, vf, dof = (x[0:1, h:h + 1][:, :, src] for x in (inputs["q"], inputs["k"], inputs["v"], do_np))
        gh = [to_host_f64(x[0, h]) for x in (dq, dk, dv)]
        if h in dq_heads:
            qrows = sorted(rng.choice(S, 8 if ci == 2 else 4, replace=False).tolist())
            rdq, _, _ = oracle.block_sparse_attention_backward(qf, kf, vf, prp, ci_, dof, 64, rows=qrows)
            for i in qrows:
                tok = src[i * 64:(i + 1) * 64]
                got["dq"].append(gh[0][tok])
                ref["dq"].append(rdq[0, 0, i * 64:(i + 1) * 64])
        if h in dkv_heads:
            rows_of = np.repeat(np.arange(S), np.diff(prp))
            for j in rng.choice(S, 4, replace=False):
                krows = sorted(set(rows_of[ci_ == j].tolist()))
                if not krows:
                    continue
                _, rdk, rdv = oracle.block_sparse_attention_backward(qf, kf, vf, prp, ci_, dof, 64, rows=krows)
                tok = src[j * 64:(j + 1) * 64]
                got["dk"].append(gh[1][tok])
                ref["dk"].append(rdk[0, 0, j * 64:(j + 1) * 64])
                got["dv"].append(gh[2][tok])
                ref["dv"].append(rdv[0, 0, j * 64:(j + 1) * 64])
        print(f"head {h} compared", flush=True)
    res = [grad_errors(np.stack(got[n]), np.stack(ref[n]), cfg.dtype, n) for n in ("dq", "dk", "dv")]
    msg = "; ".join(m for _, m in res)
    print(msg)
    assert all(ok for ok, _ in res), msg
