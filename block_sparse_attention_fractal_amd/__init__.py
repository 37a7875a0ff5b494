"""Content-adaptive block-sparse video attention (NABLA pipeline) on MI355X.

The computation lives in libbsa.so (hand-written HIP kernels for gfx950 behind
the C ABI in include/bsa.h); this package only marshals torch tensors into it.
"""
from ._lib import BSAError, LIB_PATH, EXPORTED, lib
from .api import (KEY_GROUP, ORDERS, BlockMask, VideoGrid, attend, attend_groups, attend_groups_workspace_bytes,
                  attend_static, attend_train,
                  attend_workspace_bytes, attention,
                  backward, backward_train, backward_workspace_bytes, block_map, build_group_mask, build_mask, forward, forward_groups,
                  make_problem, mask_from_csr, order_table, permute, permute_table, pool, prepare_v,
                  prepare_v_groups, query_group_sizes, query_sizes)

__all__ = ["BSAError", "LIB_PATH", "EXPORTED", "lib", "BlockMask", "VideoGrid", "attention", "block_map",
           "build_mask", "forward", "make_problem", "mask_from_csr", "permute", "pool", "query_sizes",
           "prepare_v", "attend", "attend_static", "attend_train", "backward_train", "attend_workspace_bytes", "ORDERS", "order_table", "permute_table", "backward",
           "backward_workspace_bytes", "KEY_GROUP", "query_group_sizes", "build_group_mask", "prepare_v_groups",
           "attend_groups", "attend_groups_workspace_bytes", "forward_groups"]
