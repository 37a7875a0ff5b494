"""Content-adaptive block-sparse video attention (NABLA pipeline) on MI355X.

The computation lives in libbsa.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/bsa.h); this package only marshals torch tensors into it.
"""
from ._lib import BSAError, LIB_PATH, EXPORTED, lib
from .api import (ORDERS, BlockMask, VideoGrid, attend, attention, backward, backward_workspace_bytes, block_map,
                  build_mask, forward, make_problem, mask_from_csr, order_table, permute, permute_table, pool,
                  prepare_v, query_sizes)

__all__ = ["BSAError", "LIB_PATH", "EXPORTED", "lib", "BlockMask", "VideoGrid", "attention", "block_map",
           "build_mask", "forward", "make_problem", "mask_from_csr", "permute", "pool", "query_sizes",
           "prepare_v", "attend", "ORDERS", "order_table", "permute_table", "backward",
           "backward_workspace_bytes"]
