"""bsa_attend_static (no workspace argument, static scratch) against bsa_attend
(caller's workspace) through the C ABI: the same kernels on the same inputs must
give bit-identical O and LSE, on two calls in a row, the second with a smaller
problem than the first (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

from parity import to_device
from workloads import make_inputs
from workloads.configs import Config

pytestmark = pytest.mark.gpu

bsa = pytest.importorskip("block_sparse_attention_fractal_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bsa.lib()


def _one(cfg, window=None):
    inputs = make_inputs(cfg)
    g = bsa.VideoGrid(cfg.T, cfg.H, cfg.W, cfg.patch, cfg.block)
    q, k, v = (to_device(inputs, n, cfg.dtype) for n in "qkv")
    mask = bsa.build_mask(q, k, g, cfg.thr, window)
    vp = bsa.prepare_v(v, g) if cfg.dtype == "bf16" else v
    o_ref, lse_ref = bsa.attend(q, k, vp, mask, g, return_lse=True)
    o, lse = bsa.attend_static(q, k, vp, mask, g, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                       o_ref.view(torch.int16 if cfg.dtype == "bf16" else torch.int32))
    assert torch.equal(lse, lse_ref)
    return mask.nnz()


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_attend_static_matches_attend_twice_shrinking(dtype, D):
    big = Config(96, "static-big", dtype, 2, 3, 6, 32, 40, D, 8, 64, 0.1, None, 3.0, seed=61)
    small = Config(96, "static-small", dtype, 1, 2, 2, 16, 24, D, 8, 64, 0.2, None, 3.0, seed=62)
    n1 = _one(big, window=(1, 1, 1))
    n2 = _one(small)
    assert n1 > n2 > 0
