"""GPU parity of the 4-token key-group path (AB-Attention page, third resource)
against oracle/groups.py: the group CSR equals the oracle's outside the 1e-4
band; attention over the GPU's group CSR (and over hand-made ragged CSRs, where
rows end mid-tile and some waves have no keys) matches the oracle within the
bf16 / f32 tolerances; full-size Wan2.1-scale and HunyuanVideo-scale (one batch
item: the group CSR of both needs more than int32 offsets) masks are compared
on whole heads, attention on a seeded sample of rows."""
import numpy as np
import pytest
import torch

import oracle
from oracle import groups
from parity import compare_masks, compare_outputs, to_device, to_host_f64
from workloads import get_config, make_inputs
from workloads.configs import Config

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_fractal_amd")
G = 4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa.lib()


def grid_of(cfg):
    return bsa.VideoGrid(cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block)


def small(dtype="bf16", nh=2, T=4, H=32, W=32, D=128, thr=0.2, window=None, amp=3.0, seed=11):
    return Config(97, "groups", dtype, 1, nh, T, H, W, D, 8, 64, thr, window, amp, seed=seed)


def check_attention(cfg, inputs, o, lse, rp, ci):
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    qf, kf, vf = (inputs[n][:, :, src] for n in "qkv")
    O, LSE = groups.group_attention(qf, kf, vf, rp, ci, 64, G)
    O_orig = np.empty_like(O)
    O_orig[:, :, src] = O
    L_orig = np.empty_like(LSE)
    L_orig[:, :, src] = LSE
    ma, mr = compare_outputs(to_host_f64(o), O_orig, cfg.dtype)
    got = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L_orig)
    assert np.array_equal(np.isfinite(got), fin)
    lse_err = np.abs(got[fin] - L_orig[fin])
    assert np.all(lse_err <= (1e-5 if cfg.dtype == "f32" else 2e-3) + 2 * 2.0 ** -24 * np.abs(L_orig[fin]))
    return ma, mr


CASES = {
    "bf16-local": small(),
    "bf16-window-odd": small(T=3, H=24, W=40, thr=0.1, window=(1, 1, 1), seed=12),
    "bf16-diffuse": small(amp=0.0, thr=0.05, seed=13),
    "bf16-one-patch-column": small(T=3, H=16, W=8, thr=0.1, seed=15),
    "bf16-one-patch-row": small(T=2, H=8, W=24, thr=0.1, seed=16),
    "f32-cfg0": get_config(0),
    "f32-window": small(dtype="f32", D=64, T=2, H=16, W=24, thr=0.3, window=(0, 1, 1), amp=1.0, seed=14),
}


@pytest.mark.parametrize("name", list(CASES))
def test_group_mask_and_attention_match_oracle(name):
    cfg = CASES[name]
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    mask = bsa.build_group_mask(q, k, g, cfg.thr, cfg.window)
    o, lse = bsa.forward_groups(q, k, v, mask, g, return_lse=True)
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    assert int(mask.nnz()) == rp[-1]
    ref = groups.build_group_mask(inputs["q"], inputs["k"], cfg.T, cfg.H, cfg.W, cfg.patch, 64, G, cfg.thr,
                                  cfg.window, details=True)
    n_mis, n_band = compare_masks(rp, ci, ref, cfg.thr, cfg.L // G)
    ma, mr = check_attention(cfg, inputs, o, lse, rp, ci)
    print(f"{name}: groups kept {rp[-1]} of {cfg.rows * cfg.L // G}, mismatches={n_mis} band={n_band} "
          f"max_abs={ma:.2e} mean_rel={mr:.2e}")


def _group_mask_vs_oracle(cfg, inputs):
    g = grid_of(cfg)
    q, k = (to_device(inputs, n, cfg.dtype) for n in "qk")
    mask = bsa.build_group_mask(q, k, g, cfg.thr, cfg.window)
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    ref = groups.build_group_mask(inputs["q"], inputs["k"], cfg.T, cfg.H, cfg.W, cfg.patch, 64, G, cfg.thr,
                                  cfg.window, details=True)
    return rp, compare_masks(rp, ci, ref, cfg.thr, cfg.L // G)


def _with_bf16(inputs, name, x):
    from workloads import bf16_bits_to_f32, bf16_round
    bits = bf16_round(x)
    inputs[name + "_bits"], inputs[name] = bits, bf16_bits_to_f32(bits)


@pytest.mark.parametrize("frames,dtype,D", [(4, "bf16", 128), (2, "bf16", 128), (2, "f32", 64)],
                         ids=["every-row-float64", "half-the-rows-float64", "f32-d64-half-the-rows-float64"])
def test_group_mask_rows_beyond_the_screen(frames, dtype, D):
    """Queries of the first `frames` frames scaled by 96: the screened group logits of
    their rows cannot be trusted to the band, so those rows are cut from float64
    logits (the group means formed from the keys in the input's own type); the CSR
    must match the oracle's, alone and mixed with screened rows."""
    cfg = small(dtype=dtype, D=D, T=4, H=24, W=40, thr=0.1, window=(1, 1, 1), amp=0.0, seed=52)
    inputs = make_inputs(cfg)
    x = inputs["q"].copy()
    x[:, :, : frames * cfg.H * cfg.W] *= 96.0
    if dtype == "bf16":
        _with_bf16(inputs, "q", x)
    else:
        inputs["q"] = x
    rp, (n_mis, n_band) = _group_mask_vs_oracle(cfg, inputs)
    print(f"groups, frames scaled {frames}: nnz={rp[-1]} mismatches={n_mis} band={n_band}")


def test_group_mask_exact_ties():
    """Every key equal: all group logits of a row tie, the screen's margin holds the
    whole row (more entries than it ranks exactly), so every row goes to the float64
    path, which keeps the lowest group indices first."""
    cfg = small(nh=2, T=2, H=16, W=32, thr=0.3, seed=53)
    inputs = make_inputs(cfg)
    _with_bf16(inputs, "k", np.repeat(inputs["k"][:, :, :1], cfg.L, axis=2))
    rp, (n_mis, n_band) = _group_mask_vs_oracle(cfg, inputs)
    assert n_mis == 0
    print(f"groups, all keys equal: nnz={rp[-1]} of {cfg.rows * cfg.L // G}")


def test_thr_zero_keeps_every_group_and_is_dense():
    cfg = small(nh=1, T=2, H=16, W=32, thr=0.0, seed=15)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    mask = bsa.build_group_mask(q, k, g, 0.0)
    o = bsa.forward_groups(q, k, v, mask, g)
    torch.cuda.synchronize()
    assert mask.nnz() == cfg.rows * (cfg.L // G)
    Od, _ = oracle.dense_attention(inputs["q"], inputs["k"], inputs["v"])
    compare_outputs(to_host_f64(o), Od, "bf16")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("f32", 128)])
def test_ragged_hand_made_group_lists(dtype, D):
    """Rows of 1..70 groups (partial last tiles, tiles whose second half is empty),
    one empty row (o = 0, lse = -inf) and groups from anywhere in the head."""
    cfg = small(dtype=dtype, D=D, nh=2, T=2, H=24, W=32, seed=16)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    SG = cfg.L // G
    rng = np.random.default_rng(5)
    keep = np.zeros((cfg.rows, SG), bool)
    sizes = rng.integers(1, 71, cfg.rows)
    sizes[:8] = [1, 3, 8, 9, 15, 16, 17, 33]
    for r in range(cfg.rows):
        keep[r, rng.choice(SG, size=sizes[r], replace=False)] = True
    keep[5] = False                                     # an empty row
    rp, ci = oracle.csr_from_keep(keep)
    q, k, v = (to_device(inputs, n, dtype) for n in "qkv")
    mask = bsa.mask_from_csr(torch.from_numpy(rp.astype(np.int32)).cuda(), torch.from_numpy(ci).cuda(), SG)
    o, lse = bsa.forward_groups(q, k, v, mask, g, return_lse=True)
    torch.cuda.synchronize()
    check_attention(cfg, inputs, o, lse, rp, ci)


def test_expanded_block_mask_gives_block_attention():
    """A block CSR expanded to its groups: the gathered-group kernel and the block
    kernel both match the block oracle on it."""
    cfg = small(seed=17)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    bmask = bsa.build_mask(q, k, g, cfg.thr)
    torch.cuda.synchronize()
    brp = bmask.row_ptr.cpu().numpy().astype(np.int64)
    bci = bmask.col_idx[: int(brp[-1])].cpu().numpy()
    rp, ci = groups.expand_block_csr(brp, bci, 64 // G)
    gmask = bsa.mask_from_csr(torch.from_numpy(rp.astype(np.int32)).cuda(), torch.from_numpy(ci).cuda(),
                              cfg.L // G)
    og, lg = bsa.forward_groups(q, k, v, gmask, g, return_lse=True)
    ob = bsa.forward(q, k, v, bmask, g)
    torch.cuda.synchronize()
    check_attention(cfg, inputs, og, lg, rp, ci)
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    O, _ = oracle.block_sparse_attention(*(inputs[n][:, :, src] for n in "qkv"), brp, bci, 64)
    O_orig = np.empty_like(O)
    O_orig[:, :, src] = O
    compare_outputs(to_host_f64(ob), O_orig, "bf16")


def _head_ref(inputs, cfg, b, h, src):
    wmask = None
    if cfg.window is not None:
        wmask = groups.group_window(cfg.T, cfg.H // cfg.patch, cfg.W // cfg.patch, cfg.window, 64 // G)
    return groups.head_group_mask(inputs["q"][b, h][src], inputs["k"][b, h][src], 64, G, cfg.thr, wmask)


@pytest.mark.parametrize("ci,heads,n_rows", [(2, (0, 21, 39), 24), (4, (0, 20), 16)])
def test_fullsize_group_mask_and_sampled_attention(ci, heads, n_rows):
    cfg = get_config(ci)
    B = 1
    inputs = make_inputs(cfg, batch=B)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    for n in ("q_bits", "k_bits", "v_bits"):
        inputs.pop(n)
    mask = bsa.build_group_mask(q, k, g, cfg.thr, cfg.window)
    o, lse = bsa.forward_groups(q, k, v, mask, g, return_lse=True)
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    SG = cfg.L // G
    S = cfg.S
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    rng = np.random.default_rng(cfg.seed)
    o_h = to_host_f64(o)
    lse_h = lse.cpu().numpy().astype(np.float64)
    tot_mis = tot_band = 0
    for h in heads:
        r0 = h * S
        lo, hi = int(rp[r0]), int(rp[r0 + S])
        ci_h = mask.col_idx[lo:hi].cpu().numpy()
        ref = _head_ref(inputs, cfg, 0, h, src)
        n_mis, n_band = compare_masks(rp[r0:r0 + S + 1] - lo, ci_h, ref, cfg.thr, SG)
        tot_mis += n_mis
        tot_band += n_band
        del ref
        # sampled rows of this head: oracle attention on the GPU's groups
        rows = sorted(set(rng.choice(S, n_rows // len(heads), replace=False).tolist()) | {0, S - 1})
        qf, kf, vf = (inputs[n][0:1, h:h + 1][:, :, src] for n in "qkv")
        prp = rp[r0:r0 + S + 1] - lo
        O, LSE = groups.group_attention(qf, kf, vf, prp, ci_h, 64, G, rows=rows)
        for i in rows:
            tok = src[i * 64:(i + 1) * 64]
            compare_outputs(o_h[0, h, tok], O[0, 0, i * 64:(i + 1) * 64], cfg.dtype, what=f"head {h} row {i}")
            assert np.abs(lse_h[0, h, tok] - LSE[0, 0, i * 64:(i + 1) * 64]).max() < 2e-3
    print(f"cfg{ci} (B=1): group density={rp[-1] / cfg.rows / SG:.4f} (rows {cfg.rows // cfg.batch}), "
          f"heads {heads}: mismatches={tot_mis} band={tot_band}")


def test_group_mask_at_the_largest_row():
    """One head with L/4 = 32768 groups (32 x 64 x 64 tokens, S = 2048): the group
    select's LDS row buffer is exactly full."""
    cfg = Config(96, "groups-max", "bf16", 1, 1, 32, 64, 64, 128, 8, 64, 0.2, None, 3.0, seed=19)
    assert cfg.L // G == 32768
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    mask = bsa.build_group_mask(q, k, g, cfg.thr)
    o, lse = bsa.forward_groups(q, k, v, mask, g, return_lse=True)
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    ref = groups.head_group_mask(inputs["q"][0, 0][src], inputs["k"][0, 0][src], 64, G, cfg.thr)
    n_mis, n_band = compare_masks(rp, ci, ref, cfg.thr, cfg.L // G)
    del ref
    rows = [0, 1, 777, 2047]
    qf, kf, vf = (inputs[n][:, :, src] for n in "qkv")
    O, LSE = groups.group_attention(qf, kf, vf, rp, ci, 64, G, rows=rows)
    o_h = to_host_f64(o)
    for i in rows:
        tok = src[i * 64:(i + 1) * 64]
        compare_outputs(o_h[0, 0, tok], O[0, 0, i * 64:(i + 1) * 64], "bf16", what=f"row {i}")
    print(f"groups-max: kept {rp[-1]} of {2048 * 32768}, mismatches={n_mis} band={n_band}")
