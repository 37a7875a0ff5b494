"""GPU parity of the SIP mask mode (sampling with inclusion-probability weights,
AB-Attention page, "Los tres recursos de AB-Attention") and of attention with
per-entry logit shifts, against oracle/sip.py through the C ABI.

The budget of every row is the CDF cut's count; the tests take it from the
GPU's own CDF mask (itself checked against the oracle in test_gpu_parity.py), so
both sides sample from identical budgets.  Sampled blocks must agree exactly,
except where the oracle's uniform and inclusion probability are within 1e-9 of
each other (float64 rounding of the two map evaluations); shifts within 1e-5."""
import numpy as np
import pytest
import torch

import oracle
from oracle import sip
from parity import check_csr_wellformed, compare_outputs, csr_to_keep, to_device, to_host_f64
from workloads import get_config, make_inputs
from workloads.configs import Config

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_fractal_amd")

U_BAND = 1e-9


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa.lib()


def grid_of(cfg):
    return bsa.VideoGrid(cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block)


def small_cfg(dtype="bf16", B=1, nh=2, T=3, H=24, W=40, D=128, thr=0.1, window=None, amp=3.0, local=None, seed=7):
    return Config(99, "edge", dtype, B, nh, T, H, W, D, 8, 64, thr, window, amp, local_heads=local, seed=seed)


def oracle_sip(cfg, inputs, budget, seed, thr, window):
    """Oracle SIP mask over all rows: reduced map from the oracle, budgets given."""
    ref = oracle.build_mask(inputs["q"], inputs["k"], cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block, thr, None,
                            details=True)
    A = ref["A"]                                          # [B, nh, S, S]
    B, nh, S, _ = A.shape
    wmask = oracle.sta_window(cfg.T, cfg.H // cfg.patch, cfg.W // cfg.patch, window) if window else None
    keep = np.zeros((B * nh, S, S), bool)
    shift = np.zeros((B * nh, S, S))
    u_all = sip.uniforms(np.arange(B * nh * S), S, seed).reshape(B * nh, S, S)
    pi_all = np.zeros((B * nh, S, S))
    for bh in range(B * nh):
        b, h = divmod(bh, nh)
        kk, sh = sip.build_sip_mask(A[b, h], budget[bh * S:(bh + 1) * S], u_all[bh], thr, wmask)
        keep[bh], shift[bh] = kk, sh
        if thr > 0:
            for i in range(S):
                pi_all[bh, i] = sip.inclusion_probabilities(A[b, h, i], int(budget[bh * S + i]))
    return keep.reshape(-1, S), shift.reshape(-1, S), u_all.reshape(-1, S), pi_all.reshape(-1, S), wmask


def gpu_masks(cfg, inputs, thr, window, seed):
    q, k = to_device(inputs, "q", cfg.dtype), to_device(inputs, "k", cfg.dtype)
    g = grid_of(cfg)
    cdf = bsa.build_mask(q, k, g, thr, None)
    smask = bsa.build_mask(q, k, g, thr, window, sip_seed=seed)
    torch.cuda.synchronize()
    budget = np.diff(cdf.row_ptr.cpu().numpy())
    rp = smask.row_ptr.cpu().numpy().astype(np.int64)
    ci = smask.col_idx[: int(rp[-1])].cpu().numpy()
    sh = smask.shift[: int(rp[-1])].cpu().numpy().astype(np.float64)
    return smask, budget, rp, ci, sh


def compare_sip(cfg, inputs, thr, window, seed):
    smask, budget, rp, ci, sh = gpu_masks(cfg, inputs, thr, window, seed)
    check_csr_wellformed(rp, ci, cfg.S)
    keep_ref, shift_ref, u, pi, wmask = oracle_sip(cfg, inputs, budget, seed, thr, window)
    got = csr_to_keep(rp, ci, cfg.S)
    band = np.abs(u - pi) <= U_BAND
    if wmask is not None:
        band &= ~np.tile(wmask, (got.shape[0] // cfg.S, 1))
    diff = got != keep_ref
    assert not (diff & ~band).any(), f"{int((diff & ~band).sum())} sampled blocks differ outside the band"
    # shifts of the entries both sides kept
    rows = np.repeat(np.arange(got.shape[0]), np.diff(rp))
    both = keep_ref[rows, ci]
    err = np.abs(sh[both] - shift_ref[rows[both], ci[both]])
    assert err.max(initial=0.0) <= 1e-5 * max(1.0, np.abs(shift_ref).max())
    assert np.all(sh >= 0)
    return smask, got, keep_ref, int(diff.sum())


CASES = [
    ("cfg1", lambda: get_config(1), None, "cfg"),
    ("cfg1-thr0.5", lambda: get_config(1), 0.5, "cfg"),
    ("hybrid-small", lambda: small_cfg(B=2, nh=3, T=5, H=24, W=40, thr=0.1, window=(1, 1, 1), amp=4.0, local=2),
     None, "cfg"),
    ("diffuse", lambda: small_cfg(nh=2, T=6, H=32, W=32, thr=0.05, amp=0.0, local=0), None, "cfg"),
    ("cfg0-f32", lambda: get_config(0), None, "cfg"),
]


@pytest.mark.parametrize("name,mk,thr,window", CASES, ids=[c[0] for c in CASES])
def test_sip_mask_matches_oracle(name, mk, thr, window):
    cfg = mk()
    inputs = make_inputs(cfg)
    thr = cfg.thr if thr is None else thr
    window = cfg.window if window == "cfg" else window
    _, got, ref, n_mis = compare_sip(cfg, inputs, thr, window, seed=1234)
    # the sample is a sample: it differs from the deterministic cut
    print(f"{name}: kept {int(got.sum())} of {got.size}, mismatches in band {n_mis}")


def test_sip_seed_determinism_and_variation():
    cfg = get_config(1)
    inputs = make_inputs(cfg)
    q, k = to_device(inputs, "q", "bf16"), to_device(inputs, "k", "bf16")
    g = grid_of(cfg)
    a = bsa.build_mask(q, k, g, 0.3, None, sip_seed=5)
    b = bsa.build_mask(q, k, g, 0.3, None, sip_seed=5)
    c = bsa.build_mask(q, k, g, 0.3, None, sip_seed=6)
    n = a.nnz()
    assert n == b.nnz() and torch.equal(a.row_ptr, b.row_ptr) and torch.equal(a.col_idx[:n], b.col_idx[:n])
    assert torch.equal(a.shift[:n], b.shift[:n])
    m = c.nnz()
    assert n != m or not torch.equal(a.col_idx[:n], c.col_idx[:m])


@pytest.mark.parametrize("ci", [0, 1])
def test_sip_attention_matches_oracle(ci):
    """Attention on the GPU's SIP mask (with its shifts) vs the float64 oracle with
    the same CSR and shifts."""
    cfg = get_config(ci)
    inputs = make_inputs(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    g = grid_of(cfg)
    mask = bsa.build_mask(q, k, g, 0.3, cfg.window, sip_seed=99)
    o, lse = bsa.forward(q, k, v, mask, g, return_lse=True)
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy()
    ci_ = mask.col_idx[: int(rp[-1])].cpu().numpy()
    sh = mask.shift[: int(rp[-1])].cpu().numpy()
    assert (sh > 0).any(), "the sample should include weighted blocks"
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    qf, kf, vf = (inputs[n][:, :, src] for n in "qkv")
    O, LSE = sip.shifted_block_sparse_attention(qf, kf, vf, rp, ci_, sh, cfg.block)
    O_orig = np.empty_like(O)
    O_orig[:, :, src] = O
    L_orig = np.empty_like(LSE)
    L_orig[:, :, src] = LSE
    ma, mr = compare_outputs(to_host_f64(o), O_orig, cfg.dtype)
    assert np.abs(lse.cpu().numpy().astype(np.float64) - L_orig).max() < (1e-5 if cfg.dtype == "f32" else 2e-3)
    print(f"cfg{ci}: max_abs={ma:.3e} mean_rel={mr:.3e}")


def test_sip_thr_zero_is_dense():
    cfg = small_cfg(nh=2, T=2, H=16, W=32, thr=0.0, seed=31)
    inputs = make_inputs(cfg)
    q, k, v = (to_device(inputs, n, "bf16") for n in "qkv")
    g = grid_of(cfg)
    mask = bsa.build_mask(q, k, g, 0.0, None, sip_seed=3)
    assert mask.nnz() == mask.rows * cfg.S
    assert not mask.shift[: mask.nnz()].any()
    o = bsa.forward(q, k, v, mask, g)
    O, _ = oracle.dense_attention(inputs["q"], inputs["k"], inputs["v"])
    compare_outputs(to_host_f64(o), O, "bf16")


def test_sip_fullsize_heads_and_sampled_attention():
    """The HunyuanVideo-scale hybrid workload in the benchmark's launch
    configuration (B = 2, 24 heads, window, one call): the whole SIP mask is built
    on the GPU, three heads (local, diffuse, second batch item) are compared with
    the oracle's sampling on the GPU's CDF budgets, and sampled rows of the
    shifted attention with the oracle."""
    cfg = get_config(4)
    inputs = make_inputs(cfg)
    g = grid_of(cfg)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    for n in ("q_bits", "k_bits", "v_bits"):
        inputs.pop(n)
    seed = 77
    cdf = bsa.build_mask(q, k, g, cfg.thr, None)
    mask = bsa.build_mask(q, k, g, cfg.thr, cfg.window, sip_seed=seed)
    o, lse = bsa.forward(q, k, v, mask, g, return_lse=True)
    torch.cuda.synchronize()
    S = cfg.S
    budget = np.diff(cdf.row_ptr.cpu().numpy())
    rp = mask.row_ptr.cpu().numpy().astype(np.int64)
    src = oracle.fractal_positions(cfg.T, cfg.H, cfg.W, cfg.patch)
    wmask = oracle.sta_window(cfg.T, cfg.H // cfg.patch, cfg.W // cfg.patch, cfg.window)
    o_h = to_host_f64(o)
    lse_h = lse.cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(4)
    for b, h in ((0, 0), (0, 20), (1, 5)):
        bh = b * cfg.heads + h
        r0 = bh * S
        lo, hi = int(rp[r0]), int(rp[r0 + S])
        ci = mask.col_idx[lo:hi].cpu().numpy()
        sh = mask.shift[lo:hi].cpu().numpy().astype(np.float64)
        prp = rp[r0:r0 + S + 1] - lo
        got = csr_to_keep(prp, ci, S)
        A = oracle.head_mask(inputs["q"][b, h][src], inputs["k"][b, h][src], 64, cfg.thr)["A"]
        u = sip.uniforms(np.arange(r0, r0 + S), S, seed)
        keep_ref, shift_ref = sip.build_sip_mask(A, budget[r0:r0 + S], u, cfg.thr, wmask)
        pi = np.stack([sip.inclusion_probabilities(A[i], int(budget[r0 + i])) for i in range(S)])
        band = (np.abs(u - pi) <= U_BAND) & ~wmask
        diff = got != keep_ref
        assert not (diff & ~band).any(), f"head {(b, h)}: {int((diff & ~band).sum())} blocks differ outside the band"
        rows = np.repeat(np.arange(S), np.diff(prp))
        both = keep_ref[rows, ci]
        assert np.abs(sh[both] - shift_ref[rows[both], ci[both]]).max(initial=0.0) <= 1e-5 * max(1.0, shift_ref.max())
        # sampled rows of the shifted attention
        qf, kf, vf = (inputs[n][b:b + 1, h:h + 1][:, :, src] for n in "qkv")
        sample = sorted(set(rng.choice(S, 6, replace=False).tolist()) | {0, S - 1})
        O, LSE = sip.shifted_block_sparse_attention(qf, kf, vf, prp, ci, sh, 64, rows=sample)
        for i in sample:
            tok = src[i * 64:(i + 1) * 64]
            compare_outputs(o_h[b, h, tok], O[0, 0, i * 64:(i + 1) * 64], "bf16", what=f"head {(b, h)} row {i}")
            assert np.abs(lse_h[b, h, tok] - LSE[0, 0, i * 64:(i + 1) * 64]).max() < 2e-3
        print(f"head {(b, h)}: kept {int(got.sum())}, differing in band {int(diff.sum())}")
