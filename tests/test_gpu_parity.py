"""GPU parity of every hot-path step against the oracle, through the C ABI.

Small cases (configs 0 and 1 and hand-made edge cases) are compared element by
element; the full Wan2.1/HunyuanVideo-scale configurations compare the whole
CSR mask and a sample of attention rows (see test_gpu_scale.py)."""
import numpy as np
import pytest
import torch

import oracle
from parity import (compare_masks, compare_outputs, gpu_rows_fractal, oracle_attention_rows, to_device,
                    to_host_f64)
from workloads import get_config, make_inputs
from workloads.configs import Config

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_fractal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa.lib()   # fails loudly when libbsa.so is missing


def grid_of(cfg):
    return bsa.VideoGrid(cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block)


def small_cfg(dtype="bf16", B=1, nh=2, T=3, H=24, W=40, D=128, thr=0.1, window=None, amp=3.0, local=None, seed=7):
    return Config(99, "edge", dtype, B, nh, T, H, W, D, 8, 64, thr, window, amp, local_heads=local, seed=seed)


def run_all(cfg, inputs, thr=None, window="cfg", layout="original"):
    thr = cfg.thr if thr is None else thr
    window = cfg.window if window == "cfg" else window
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    g = grid_of(cfg)
    if layout == "fractal":
        q, k, v = (bsa.permute(x, g) for x in (q, k, v))
    mask = bsa.build_mask(q, k, g, thr, window, layout=layout)
    o, lse = bsa.forward(q, k, v, mask, g, layout=layout, return_lse=True)
    if layout == "fractal":
        o = bsa.permute(o, g, inverse=True)
        idx = torch.from_numpy(oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)).cuda()
        lse_o = torch.empty_like(lse)
        lse_o[:, :, idx] = lse
        lse = lse_o
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy()
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    return {"mask": mask, "row_ptr": rp, "col_idx": ci, "o": to_host_f64(o), "lse": lse.cpu().numpy().astype(np.float64)}


def oracle_mask(cfg, inputs, thr=None, window="cfg"):
    thr = cfg.thr if thr is None else thr
    window = cfg.window if window == "cfg" else window
    return oracle.build_mask(inputs["q"], inputs["k"], cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block, thr, window,
                             details=True)


def oracle_full_attention(cfg, inputs, row_ptr, col_idx):
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    qf, kf, vf = (inputs[n][:, :, src] for n in "qkv")
    O, LSE = oracle.block_sparse_attention(qf, kf, vf, row_ptr, col_idx, cfg.block)
    O_orig = np.empty_like(O)
    O_orig[:, :, src] = O
    L_orig = np.empty_like(LSE)
    L_orig[:, :, src] = LSE
    return O_orig, L_orig


# ------------------------------------------------------------------ a1: permute
@pytest.mark.parametrize("ci", [0, 1])
def test_permute_bit_exact(ci):
    cfg = get_config(ci)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    x = to_device(inputs, "q", cfg.dtype)
    y = bsa.permute(x, g)
    back = bsa.permute(y, g, inverse=True)
    torch.cuda.synchronize()
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    ref = x.cpu()[:, :, torch.from_numpy(src)]
    assert torch.equal(y.cpu().view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                       ref.view(torch.int16 if cfg.dtype == "bf16" else torch.int32))
    assert torch.equal(back.cpu(), x.cpu())


# ------------------------------------------------------------------ a2: pool
@pytest.mark.parametrize("ci", [0, 1])
@pytest.mark.parametrize("layout", ["original", "fractal"])
def test_pool_matches_oracle(ci, layout):
    cfg = get_config(ci)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k = to_device(inputs, "q", cfg.dtype), to_device(inputs, "k", cfg.dtype)
    if layout == "fractal":
        q, k = bsa.permute(q, g), bsa.permute(k, g)
    qp, kp = bsa.pool(q, k, g, layout)
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    for got, name in ((qp, "q"), (kp, "k")):
        ref = oracle.pool_blocks(inputs[name][:, :, src].astype(np.float64), cfg.block)
        got = got.cpu().numpy()
        if cfg.dtype == "bf16":
            assert np.array_equal(got, ref)          # float64 sums of bf16 values are exact
        else:
            assert np.abs(got - ref).max() <= 1e-15 * max(1.0, np.abs(ref).max())


# ------------------------------------------------------------------ a3: reduced map
@pytest.mark.parametrize("ci", [0, 1])
def test_block_map_matches_oracle(ci):
    cfg = get_config(ci)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k = to_device(inputs, "q", cfg.dtype), to_device(inputs, "k", cfg.dtype)
    qp, kp = bsa.pool(q, k, g)
    probs = bsa.block_map(qp, kp, g, dtype=q.dtype).cpu().numpy()
    ref = oracle_mask(cfg, inputs)["A"]
    assert np.abs(probs - ref).max() < 1e-12
    assert np.allclose(probs.sum(-1), 1.0, atol=1e-12)


# ------------------------------------------------------------------ a4: mask
MASK_CASES = [
    ("cfg0", lambda: get_config(0), None, "cfg"),
    ("cfg1", lambda: get_config(1), None, "cfg"),
    ("cfg1-thr0", lambda: get_config(1), 0.0, "cfg"),
    ("cfg1-thr0.6", lambda: get_config(1), 0.6, "cfg"),
    ("cfg1-thr0.999", lambda: get_config(1), 0.999, "cfg"),
    ("hybrid-small", lambda: small_cfg(B=2, nh=3, T=5, H=24, W=40, thr=0.1, window=(1, 1, 1), amp=4.0, local=2), None, "cfg"),
    ("window-asym", lambda: small_cfg(nh=2, T=4, H=32, W=24, thr=0.3, window=(0, 2, 1)), None, "cfg"),
    ("diffuse", lambda: small_cfg(nh=2, T=6, H=32, W=32, thr=0.05, amp=0.0, local=0), None, "cfg"),
]


@pytest.mark.parametrize("name,mk,thr,window", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_mask_matches_oracle(name, mk, thr, window):
    cfg = mk()
    inputs = make_inputs(cfg)
    thr_ = cfg.thr if thr is None else thr
    g = grid_of(cfg)
    q, k = to_device(inputs, "q", cfg.dtype), to_device(inputs, "k", cfg.dtype)
    mask = bsa.build_mask(q, k, g, thr_, cfg.window if window == "cfg" else window)
    rp = mask.row_ptr.cpu().numpy()
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    assert mask.nnz() == rp[-1]
    ref = oracle_mask(cfg, inputs, thr_, window)
    n_mis, n_band = compare_masks(rp, ci, ref, thr_, cfg.S)
    print(f"{name}: nnz={rp[-1]} density={rp[-1] / (len(rp) - 1) / cfg.S:.4f} mismatches={n_mis} band={n_band}")
    if thr_ == 0:
        assert rp[-1] == (len(rp) - 1) * cfg.S


# ------------------------------------------------------------------ a5: attention
@pytest.mark.parametrize("ci", [0, 1])
def test_forward_matches_oracle_on_gpu_mask(ci):
    cfg = get_config(ci)
    inputs = make_inputs(cfg)
    res = run_all(cfg, inputs)
    O, LSE = oracle_full_attention(cfg, inputs, res["row_ptr"], res["col_idx"])
    ma, mr = compare_outputs(res["o"], O, cfg.dtype)
    assert np.abs(res["lse"] - LSE).max() < (1e-5 if cfg.dtype == "f32" else 2e-3)
    print(f"cfg{ci}: max_abs={ma:.3e} mean_rel={mr:.3e}")


@pytest.mark.parametrize("ci", [0, 1])
def test_forward_on_oracle_mask(ci):
    cfg = get_config(ci)
    inputs = make_inputs(cfg)
    ref = oracle_mask(cfg, inputs)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    rp = torch.from_numpy(ref["row_ptr"].astype(np.int32)).cuda()
    cidx = torch.from_numpy(ref["col_idx"].astype(np.int32)).cuda()
    o = bsa.forward(q, k, v, bsa.mask_from_csr(rp, cidx, cfg.S), g)
    O, _ = oracle_full_attention(cfg, inputs, ref["row_ptr"], ref["col_idx"])
    compare_outputs(to_host_f64(o), O, cfg.dtype)


DTYPE_DIMS = [("f32", 64), ("bf16", 128), ("bf16", 64)]


@pytest.mark.parametrize("dtype,D", DTYPE_DIMS)
def test_thr_zero_is_dense_attention(dtype, D):
    cfg = small_cfg(dtype=dtype, nh=2, T=2, H=16, W=24, D=D, thr=0.0)
    inputs = make_inputs(cfg)
    res = run_all(cfg, inputs, thr=0.0)
    assert res["row_ptr"][-1] == (len(res["row_ptr"]) - 1) * cfg.S
    O, LSE = oracle.dense_attention(inputs["q"], inputs["k"], inputs["v"])
    compare_outputs(res["o"], O, dtype)


@pytest.mark.parametrize("dtype,D", DTYPE_DIMS)
def test_single_block_sequence_is_dense(dtype, D):
    cfg = small_cfg(dtype=dtype, nh=3, T=1, H=8, W=8, D=D, thr=0.5)
    inputs = make_inputs(cfg)
    res = run_all(cfg, inputs)
    O, _ = oracle.dense_attention(inputs["q"], inputs["k"], inputs["v"])
    compare_outputs(res["o"], O, dtype)


@pytest.mark.parametrize("dtype,D", DTYPE_DIMS)
def test_fractal_layout_matches_original(dtype, D):
    cfg = small_cfg(dtype=dtype, nh=2, T=3, H=16, W=24, D=D, thr=0.2)
    inputs = make_inputs(cfg)
    a = run_all(cfg, inputs)
    b = run_all(cfg, inputs, layout="fractal")
    assert np.array_equal(a["row_ptr"], b["row_ptr"]) and np.array_equal(a["col_idx"], b["col_idx"])
    assert np.array_equal(a["o"], b["o"])
    assert np.array_equal(a["lse"], b["lse"])


def test_hybrid_window_small_attention():
    cfg = small_cfg(B=2, nh=3, T=5, H=24, W=40, thr=0.1, window=(1, 1, 1), amp=4.0, local=2)
    inputs = make_inputs(cfg)
    res = run_all(cfg, inputs)
    ref = oracle_mask(cfg, inputs)
    compare_masks(res["row_ptr"], res["col_idx"], ref, cfg.thr, cfg.S)
    O, _ = oracle_full_attention(cfg, inputs, res["row_ptr"], res["col_idx"])
    compare_outputs(res["o"], O, "bf16")


def test_deterministic_bitwise():
    cfg = get_config(1)
    inputs = make_inputs(cfg)
    a = run_all(cfg, inputs)
    b = run_all(cfg, inputs)
    assert np.array_equal(a["row_ptr"], b["row_ptr"]) and np.array_equal(a["col_idx"], b["col_idx"])
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["lse"], b["lse"])


def test_max_blocks_per_head():
    """S = 4096, the largest supported row length: mask over the whole row set, attention sampled."""
    cfg = small_cfg(nh=1, T=16, H=128, W=128, thr=0.1, amp=3.0, seed=11)
    assert cfg.S == 4096
    inputs = make_inputs(cfg)
    res = run_all(cfg, inputs)
    ref = oracle_mask(cfg, inputs)
    n_mis, n_band = compare_masks(res["row_ptr"], res["col_idx"], ref, cfg.thr, cfg.S)
    rows = np.random.default_rng(0).choice(cfg.rows, 24, replace=False).tolist() + [0, cfg.rows - 1]
    ro = oracle_attention_rows(inputs, cfg, res["row_ptr"], res["col_idx"], rows)
    go = gpu_rows_fractal(res["o"], None, cfg, rows, 1)
    compare_outputs(np.stack([go[r][0] for r in rows]), np.stack([ro[r][0] for r in rows]), "bf16")


@pytest.mark.parametrize("thr", [0.1, 0.25, 0.5, 0.05])
def test_mask_exact_ties_uniform_rows(thr):
    """Every key block identical -> every reduced-map row is exactly uniform: the kept
    set is the ceil((1-thr)*S) lowest block ids (ties by index), as in the oracle."""
    cfg = small_cfg(nh=2, T=2, H=16, W=32, thr=thr, seed=21)
    inputs = make_inputs(cfg)
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    kb = inputs["k_bits"][:, :, src[:64]]                      # first block, fractal order
    k_bits = np.empty_like(inputs["k_bits"])
    k_bits[:, :, src] = np.tile(kb, (1, 1, cfg.S, 1))         # every block = block 0
    inputs["k_bits"] = k_bits
    from workloads import bf16_bits_to_f32
    inputs["k"] = bf16_bits_to_f32(k_bits)
    g = grid_of(cfg)
    q, k = to_device(inputs, "q", "bf16"), to_device(inputs, "k", "bf16")
    mask = bsa.build_mask(q, k, g, thr)
    rp = mask.row_ptr.cpu().numpy()
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    ref = oracle_mask(cfg, inputs, thr)
    assert np.all(ref["A"] == ref["A"][..., :1])               # the oracle sees exact ties too
    compare_masks(rp, ci, ref, thr, cfg.S)
    K = int(np.ceil((1 - thr) * cfg.S))
    assert np.all(np.diff(rp) == K)
    assert np.array_equal(ci.reshape(-1, K), np.tile(np.arange(K), (len(rp) - 1, 1)))


def test_mask_partial_ties():
    """Half of the key blocks duplicate another block: many exact ties at varying ranks."""
    cfg = small_cfg(nh=2, T=3, H=24, W=40, thr=0.2, amp=0.5, seed=22)
    inputs = make_inputs(cfg)
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    kf = inputs["k_bits"][:, :, src].copy()
    rng = np.random.default_rng(5)
    for b in range(0, cfg.S, 2):
        o = int(rng.integers(0, cfg.S))
        kf[:, :, b * 64:(b + 1) * 64] = kf[:, :, o * 64:(o + 1) * 64]
    k_bits = np.empty_like(kf)
    k_bits[:, :, src] = kf
    from workloads import bf16_bits_to_f32
    inputs["k_bits"], inputs["k"] = k_bits, bf16_bits_to_f32(k_bits)
    g = grid_of(cfg)
    q, k = to_device(inputs, "q", "bf16"), to_device(inputs, "k", "bf16")
    mask = bsa.build_mask(q, k, g, cfg.thr)
    rp = mask.row_ptr.cpu().numpy()
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    compare_masks(rp, ci, oracle_mask(cfg, inputs), cfg.thr, cfg.S)


@pytest.mark.parametrize("T,H,W", [(2, 16, 8), (3, 8, 24), (4, 8, 8)], ids=["one-patch-column", "one-patch-row",
                                                                          "one-patch-frame"])
def test_grids_with_one_patch_per_axis(T, H, W):
    """Frames one patch wide or tall (Wp = 1 or Hp = 1) in the original layout: the
    block-row arithmetic divides by a patch count of 1, which must stay exact."""
    cfg = small_cfg(nh=2, T=T, H=H, W=W, thr=0.1, seed=41)
    inputs = make_inputs(cfg)
    res = run_all(cfg, inputs)
    compare_masks(res["row_ptr"], res["col_idx"], oracle_mask(cfg, inputs), cfg.thr, cfg.S)
    O, LSE = oracle_full_attention(cfg, inputs, res["row_ptr"], res["col_idx"])
    compare_outputs(res["o"], O, "bf16")
    assert np.abs(res["lse"] - LSE).max() < 2e-3


def _scaled_inputs(cfg, q_scale_frames, scale):
    """Inputs whose queries in the first q_scale_frames frames are multiplied by
    `scale`: large channel-wise variation of those query blocks, which the screened
    cut cannot resolve to the band, so their rows go through the float64 path."""
    from workloads import bf16_bits_to_f32, bf16_round
    inputs = make_inputs(cfg)
    x = inputs["q"].copy()
    x[:, :, : q_scale_frames * cfg.H * cfg.W] *= scale
    bits = bf16_round(x)
    inputs["q_bits"], inputs["q"] = bits, bf16_bits_to_f32(bits)
    return inputs


@pytest.mark.parametrize("frames", [4, 2], ids=["every-row-float64", "half-the-rows-float64"])
def test_mask_rows_beyond_the_screen(frames):
    """Rows whose screened logits cannot be trusted to the band are cut from float64
    logits; the CSR must still match the oracle, alone and mixed with screened rows."""
    cfg = small_cfg(nh=2, T=4, H=24, W=40, thr=0.1, window=(1, 1, 1), amp=0.0, local=0, seed=51)
    inputs = _scaled_inputs(cfg, frames, 96.0)
    g = grid_of(cfg)
    q, k = to_device(inputs, "q", "bf16"), to_device(inputs, "k", "bf16")
    mask = bsa.build_mask(q, k, g, cfg.thr, cfg.window)
    rp = mask.row_ptr.cpu().numpy()
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    n_mis, n_band = compare_masks(rp, ci, oracle_mask(cfg, inputs), cfg.thr, cfg.S)
    print(f"frames scaled {frames}: nnz={rp[-1]} mismatches={n_mis} band={n_band}")


BF16_D64 = {
    "local": small_cfg(nh=4, T=8, H=32, W=32, D=64, thr=0.2, seed=71),
    "hybrid": small_cfg(B=2, nh=3, T=5, H=24, W=40, D=64, thr=0.1, window=(1, 1, 1), amp=4.0, local=2, seed=72),
    "diffuse": small_cfg(nh=2, T=6, H=32, W=32, D=64, thr=0.05, amp=0.0, local=0, seed=73),
}


@pytest.mark.parametrize("name", list(BF16_D64))
def test_bf16_head_dim_64_matches_oracle(name):
    """bf16 with head_dim 64 (the second head size the boundary supports): the mask
    against the oracle's, attention on the GPU mask and on the oracle's mask against
    the float64 oracle, LSE included."""
    cfg = BF16_D64[name]
    inputs = make_inputs(cfg)
    res = run_all(cfg, inputs)
    ref = oracle_mask(cfg, inputs)
    n_mis, n_band = compare_masks(res["row_ptr"], res["col_idx"], ref, cfg.thr, cfg.S)
    O, LSE = oracle_full_attention(cfg, inputs, res["row_ptr"], res["col_idx"])
    ma, mr = compare_outputs(res["o"], O, "bf16")
    assert np.abs(res["lse"] - LSE).max() < 2e-3
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    rp = torch.from_numpy(ref["row_ptr"].astype(np.int32)).cuda()
    cidx = torch.from_numpy(ref["col_idx"].astype(np.int32)).cuda()
    o2 = bsa.forward(q, k, v, bsa.mask_from_csr(rp, cidx, cfg.S), g)
    O2, _ = oracle_full_attention(cfg, inputs, ref["row_ptr"], ref["col_idx"])
    compare_outputs(to_host_f64(o2), O2, "bf16")
    print(f"bf16 D=64 {name}: nnz={res['row_ptr'][-1]} mismatches={n_mis} band={n_band} max_abs={ma:.3e} "
          f"mean_rel={mr:.3e}")


def _rising_inputs(D, sign, seed=3, T=2, H=16, W=24, nh=2):
    """bf16 inputs whose logits move by ~16 (log2 units) from one 32-key half of a key
    block to the next, in block order: with sign +1 every half carries a new row max
    (the attention kernel must raise its reference on each of them, including key half
    1 after half 0 of the same tile was already added), with sign -1 the first tile
    holds the max.  Keys are a_f * (1, ..., 1) + noise with a_f = 2 j + h for fractal
    key f in half h of block j; queries are (1, ..., 1) + noise."""
    from workloads.generate import bf16_round
    rng = np.random.default_rng(seed)
    L = T * H * W
    src = oracle.fractal_positions(T, H, W, 8)          # fractal index -> original token
    f = np.arange(L)
    a = np.empty(L)
    a[src] = 2 * (f // 64) + (f % 64) // 32
    amp = 128.0 / D * np.sqrt(D / 128.0)                # logit step per half ~ 16 (log2 units) at any D
    q = 1.0 + 0.1 * rng.standard_normal((1, nh, L, D))
    k = sign * amp * a[None, None, :, None] + 0.1 * rng.standard_normal((1, nh, L, D))
    v = rng.standard_normal((1, nh, L, D))
    out = {}
    for n, x in (("q", q), ("k", k), ("v", v)):
        bits = bf16_round(x.astype(np.float32))
        out[n + "_bits"] = bits
        out[n] = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return out


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("D", [128, 64])
def test_rising_logits_raise_the_reference(D, sign):
    """Dense attention (thr = 0) on logits that rise (or fall) by ~16 log2 units per
    32-key half: the bf16 kernel's lazy reference is raised on every half (or only on
    the first tile), and O and the LSE still match the float64 oracle."""
    cfg = small_cfg(dtype="bf16", nh=2, T=2, H=16, W=24, D=D, thr=0.0)
    inputs = _rising_inputs(D, sign)
    res = run_all(cfg, inputs, thr=0.0)
    assert res["row_ptr"][-1] == (len(res["row_ptr"]) - 1) * cfg.S
    O, LSE = oracle.dense_attention(inputs["q"], inputs["k"], inputs["v"])
    compare_outputs(res["o"], O, "bf16")
    assert np.abs(res["lse"] - LSE).max() < 2e-3
