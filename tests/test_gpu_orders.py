"""GPU checks of the alternative token orders (tile-major, 3D Hilbert): the
table-driven permutation is a bit-exact row copy, and the whole path run in
those orders (layout "already permuted") matches the oracle run on the same
permuted inputs: masks up to the 1e-4 band, attention within the bf16 / f32
tolerances."""
import numpy as np
import pytest
import torch

import oracle
from oracle import orders
from parity import compare_masks, compare_outputs, to_device, to_host_f64
from workloads import make_inputs
from workloads.configs import Config

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_fractal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa.lib()


def cfg_of(dtype, T, H, W, P, D, thr, seed, nh=2):
    return Config(98, "orders", dtype, 1, nh, T, H, W, D, P, 64, thr, None, 3.0, seed=seed)


def oracle_src(name, T, H, W, P):
    if name == "hilbert":
        return orders.hilbert_positions(T, H, W)
    if name == "tile_major":
        return orders.tile_major_positions(T, H, W, P, 64)
    return oracle.fractal_positions(T, H, W, P)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("name", ["fractal", "tile_major", "hilbert"])
def test_permute_table_bit_exact(name, dtype, D):
    T, H, W, P = 8, 16, 24, (8 if name == "fractal" else 4)
    cfg = cfg_of(dtype, T, H, W, P, D, 0.1, seed=3)
    inputs = make_inputs(cfg)
    x = to_device(inputs, "q", dtype)
    g = bsa.VideoGrid(T, H, W, P, 64)
    table = bsa.order_table(g, name)
    y = bsa.permute_table(x, g, table)
    back = bsa.permute_table(y, g, table, inverse=True)
    torch.cuda.synchronize()
    src = oracle_src(name, T, H, W, P)
    assert np.array_equal(table.numpy(), src)
    xv = x.view(torch.int16) if dtype == "bf16" else x.view(torch.int32)
    yv = y.view(torch.int16) if dtype == "bf16" else y.view(torch.int32)
    assert torch.equal(yv.cpu(), xv.cpu()[:, :, torch.from_numpy(src)])
    assert torch.equal(back.view(xv.dtype), xv)


@pytest.mark.parametrize("name,dtype,D,T,H,W,P", [
    ("hilbert", "bf16", 128, 8, 32, 32, 8),
    ("hilbert", "f32", 64, 4, 16, 24, 8),
    ("tile_major", "bf16", 128, 8, 32, 32, 4),
    ("tile_major", "f32", 64, 4, 16, 16, 4),
])
def test_path_in_other_orders_matches_oracle(name, dtype, D, T, H, W, P):
    thr = 0.1
    cfg = cfg_of(dtype, T, H, W, P, D, thr, seed=5)
    inputs = make_inputs(cfg)
    g = bsa.VideoGrid(T, H, W, P, 64)
    table = bsa.order_table(g, name)
    q, k, v = (bsa.permute_table(to_device(inputs, n, dtype), g, table) for n in "qkv")
    mask = bsa.build_mask(q, k, g, thr, None, layout="fractal")
    o, lse = bsa.forward(q, k, v, mask, g, layout="fractal", return_lse=True)
    o = bsa.permute_table(o, g, table, inverse=True)
    torch.cuda.synchronize()
    rp = mask.row_ptr.cpu().numpy()
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    src = oracle_src(name, T, H, W, P)
    qf, kf, vf = (inputs[n][:, :, src] for n in "qkv")
    ref = oracle.build_mask(qf, kf, T, H, W, P, 64, thr, None, layout="fractal", details=True)
    n_mis, n_band = compare_masks(rp, ci, ref, thr, g.S)
    O, LSE = oracle.block_sparse_attention(qf, kf, vf, rp, ci, 64)
    O_orig = np.empty_like(O)
    O_orig[:, :, src] = O
    compare_outputs(to_host_f64(o), O_orig, dtype)
    # LSE is stored in float32: beyond 1e-5 absolute, allow its own rounding (logits here reach ~10^3)
    lse_err = np.abs(lse.cpu().numpy().astype(np.float64) - LSE)
    assert np.all(lse_err <= (1e-5 if dtype == "f32" else 2e-3) + 2 * 2.0 ** -24 * np.abs(LSE))
    print(f"{name} {dtype}: nnz={rp[-1]} mismatches={n_mis} band={n_band}")
