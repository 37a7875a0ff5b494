"""CPU oracle for content-adaptive block-sparse video attention (NABLA pipeline).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP kernels or their host
library; the only common dependency is the seeded input generator in
`workloads`, which holds none of the method's arithmetic.

Everything is plain numpy in float64 from the exact input values, following
the steps of the NABLA technical summary (gist.science/es/paper/2507.13546,
"Metodologia: NABLA", items 1-3) in the page's order.  See `nabla.py` for the
per-function citations and the readings taken where the page is silent.

Pinned (checked against closed forms, brute force or library routines in
tests/test_oracle_pins.py): fractal_positions, permute, inverse_permute,
pool_blocks, reduced_map, cdf_keep, sta_window, csr_from_keep,
block_sparse_attention, block_sparse_attention_backward (finite differences
and torch autograd in float64), dense_attention.

`sip.py` adds the sampled selection with inclusion-probability weights of the
AB-Attention page (news.hamidun.com/es/news/14960, "Los tres recursos de
AB-Attention", second resource), pinned in tests/test_oracle_sip_pins.py against
numpy's Philox4x64-10, a bisection solve of the sampling design and Monte-Carlo
unbiasedness.  `orders.py` adds the tile-major (TRA page) and 3D Hilbert
(DFSAttn page) token orders, pinned in tests/test_oracle_orders_pins.py by
bijection, equality with the fractal order for one-frame tiles, cube-shaped
blocks and the unit-step walk of the Hilbert curve over a full 2^b cube.
`groups.py` adds the fine-grained selection of 4-token key groups gathered into
full tiles (AB-Attention page, third resource), pinned in
tests/test_oracle_groups_pins.py by its exact reduction to the block path when
a group is a whole block, by block CSRs expanded to groups, by torch float64
attention with a token-level mask, and by the linearity of group means.
No function is "parity unpinned".
"""
from .nabla import (
    fractal_positions,
    permute,
    inverse_permute,
    pool_blocks,
    reduced_map,
    cdf_keep,
    sta_window,
    csr_from_keep,
    head_mask,
    build_mask,
    block_sparse_attention,
    block_sparse_attention_backward,
    dense_attention,
    attention_pipeline,
    tile_coords,
)

__all__ = [
    "fractal_positions", "permute", "inverse_permute", "pool_blocks", "reduced_map",
    "cdf_keep", "sta_window", "csr_from_keep", "head_mask", "build_mask",
    "block_sparse_attention", "block_sparse_attention_backward", "dense_attention", "attention_pipeline",
    "tile_coords",
]
